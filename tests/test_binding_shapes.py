"""The Python binding's host-side shape checks (CPU only).

The library indexes its arrays by the sizes a call states (R target rows,
B sequences, R - B drafts, ...), and cannot see a tensor's length, so the
binding refuses short or mis-shaped tensors before anything reaches the
library.  With CPU tensors a call that passes those checks stops at the
next one, the device check, which tells the two apart."""
import pytest

torch = pytest.importorskip("torch")
import invariant_speculative_decoding_amd as m  # noqa: E402

GPU_MSG = "must be a GPU tensor|Expected a cuda device"  # past the shape checks


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def refused(fn, msg, *a, **kw):
    with pytest.raises(ValueError, match=msg):
        fn(*a, **kw)


def test_spec_verify_lengths():
    B, R, V = 3, 8, 100
    z, rs = f32(R, V), i32(B + 1)
    good = dict(drafts=i32(R - B))
    refused(m.spec_verify, GPU_MSG, z, row_start=rs, **good)
    refused(m.spec_verify, "drafts must hold at least 5", z, i32(R - B - 1), rs)
    refused(m.spec_verify, "accept_len must hold at least 3", z, i32(5), rs, accept_len=i32(2))
    refused(m.spec_verify, "out_tokens must hold at least 27", z, i32(5), rs,
            out_tokens=i32(2, 9))
    refused(m.spec_verify, "row_start must hold B", z, i32(5), i32(1))
    sampled = dict(seq_id=i32(B), pos0=i32(B), temperature=0.8)
    refused(m.spec_verify, GPU_MSG, z, i32(5), rs, draft_logits=f32(R - B, V), **sampled)
    refused(m.spec_verify, r"draft_logits must be \[R - B\]\[V\]", z, i32(5), rs,
            draft_logits=f32(R - B, V + 1), **sampled)
    refused(m.spec_verify, r"draft_logits must be \[R - B\]\[V\]", z, i32(5), rs,
            draft_logits=f32(R - B - 1, V), **sampled)
    refused(m.spec_verify, r"draft_logits must be \[R - B\]\[V\]", z, i32(5), rs, **sampled)
    refused(m.spec_verify, "seq_id must hold at least 3", z, i32(5), rs,
            draft_logits=f32(R - B, V), seq_id=i32(2), pos0=i32(B), temperature=0.8)
    # one row per sequence: no drafts and no drafter rows are needed
    refused(m.spec_verify, GPU_MSG, f32(B, V), i32(0), rs, **sampled)
    refused(m.spec_verify_noalloc, GPU_MSG, f32(B, V), i32(0), rs, **sampled)


def test_greedy_forms_lengths():
    B, R, V = 2, 6, 50
    z, rs = f32(R, V), i32(B + 1)
    refused(m.spec_verify_margin, GPU_MSG, z, i32(R - B), rs, 1e-3)
    refused(m.spec_verify_margin, "margins must hold at least 6", z, i32(R - B), rs, 1e-3,
            margins=f32(5))
    refused(m.spec_verify_margin, "recheck must hold at least 2", z, i32(R - B), rs, 1e-3,
            recheck=i32(1))
    refused(m.spec_verify_commit, GPU_MSG, z, i32(R - B), rs, i32(B), i32(B))
    refused(m.spec_verify_commit, "seq_len must hold at least 2", z, i32(R - B), rs, i32(1),
            i32(B))
    zq = f32(R - B, V)
    refused(m.spec_verify_sampled_commit, GPU_MSG, z, i32(R - B), rs, zq, i32(B), i32(B), i32(B),
            0.8)
    refused(m.spec_verify_sampled_commit, "temperature must be > 0", z, i32(R - B), rs, zq,
            i32(B), i32(B), i32(B), 0.0)
    refused(m.spec_verify_sampled_commit, "seq_len must hold at least 2", z, i32(R - B), rs, zq,
            i32(B), i32(1), i32(B), 0.8)
    refused(m.spec_verify_sampled_commit, "pos_id must hold at least 2", z, i32(R - B), rs, zq,
            i32(B), i32(B), i32(1), 0.8)
    refused(m.spec_verify_sampled_commit, r"draft_logits must be \[R - B\]\[V\]", z,
            i32(R - B), rs, f32(R - B - 1, V), i32(B), i32(B), i32(B), 0.8)
    keys = torch.zeros((R, 7), dtype=torch.int64)
    refused(m.spec_verify_keys, GPU_MSG, keys, i32(R - B), rs)
    refused(m.spec_verify_keys, "drafts must hold at least 4", keys, i32(R - B - 1), rs)
    refused(m.spec_verify_keys, "pos_id must hold at least 2", keys, i32(R - B), rs,
            seq_len=i32(B), pos_id=i32(1))


def test_attention_and_kv_lengths():
    B, R, Hq, Hkv, D, P, MP = 2, 5, 8, 2, 64, 10, 4
    q = torch.zeros((R, Hq, D), dtype=torch.float16)
    kp = torch.zeros((P, Hkv, 16, D), dtype=torch.float16)
    vp = torch.zeros((P, Hkv, D, 16), dtype=torch.float16)
    table = i32(B, MP)
    refused(m.decode_attn, GPU_MSG, q, kp, vp, table, i32(B), i32(B + 1), 0.1)
    refused(m.decode_attn, "row_start must hold B", q, kp, vp, table, i32(B), i32(B), 0.1)
    refused(m.decode_attn, "q_pos must hold at least 2", q, kp, vp, table, i32(1), i32(B + 1),
            0.1)
    refused(m.decode_attn, r"out must be \[R\]\[Hq\]\[D\]", q, kp, vp, table, i32(B),
            i32(B + 1), 0.1, out=f32(R, Hq, D - 1))
    kn = torch.zeros((R, Hkv, D), dtype=torch.float16)
    refused(m.decode_attn_append, "q_pos must hold at least 2", q, kn, kn, kp, vp, table,
            i32(1), i32(B + 1), 0.1)
    refused(m.kv_commit, GPU_MSG, kp, vp, table, i32(B), i32(B), accept_len=i32(B))
    refused(m.kv_commit, "accept_len must hold at least 2", kp, vp, table, i32(B), i32(B),
            accept_len=i32(1))
    refused(m.kv_commit, GPU_MSG, kp, vp, table, i32(B), i32(B), row_start=i32(B + 1),
            k_new=kn, v_new=kn)
    refused(m.kv_commit, r"k_new and v_new must be", kp, vp, table, i32(B), i32(B),
            row_start=i32(B + 1), k_new=kn, v_new=kn[:, :1])
    refused(m.kv_commit, "row_start must hold B", kp, vp, table, i32(B), i32(B),
            row_start=i32(B), k_new=kn, v_new=kn)


def test_row_wise_and_qgemm_shapes():
    refused(m.add_rmsnorm, GPU_MSG, f32(3, 16), f32(16), 1e-6)
    refused(m.add_rmsnorm, "w must hold H entries", f32(3, 16), f32(15), 1e-6)
    refused(m.add_rmsnorm, r"d must be \[rows\]\[H\]", f32(3, 16), f32(16), 1e-6, d=f32(2, 16))
    refused(m.silu_mul, r"gu must be \[rows\]\[2F\]", f32(3, 10), 4)
    refused(m.rope_qkv, r"qkv must be", f32(4, 100), i32(2), i32(1), 2, 1, 16, 1e4)
    refused(m.rope_qkv, "pos_id must hold at least 1", f32(4, 64), i32(2), i32(0), 2, 1, 16, 1e4)
    refused(m.embed_rows, r"h must be \[rows\]\[H\]", i32(4), torch.zeros((10, 8),
            dtype=torch.int16), h=f32(4, 7))
    w = m.PackedW4(torch.zeros(1024, dtype=torch.uint8), torch.zeros(128, dtype=torch.int16),
                   16, 128)
    refused(m.qgemm_w4, GPU_MSG, w, torch.zeros((1, 128), dtype=torch.bfloat16))
    short = m.PackedW4(w.codes[:1000], w.scales, 16, 128)
    refused(m.qgemm_w4, "w does not hold a packed", short, torch.zeros((1, 128),
            dtype=torch.bfloat16))
    refused(m.qgemm_w4_argmax, "w does not hold a packed", short, torch.zeros((1, 128),
            dtype=torch.bfloat16))
    q6 = m.PackedQ6(torch.zeros(10, dtype=torch.uint8), 16, 256)
    refused(m.qgemm_q6, "w does not hold a packed", q6, torch.zeros((1, 256),
            dtype=torch.bfloat16))
