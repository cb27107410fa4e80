// Host-side helpers shared by the isd entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "isd.h"

namespace isd {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

void qgemm_geometry(int N, int K, int x_dtype, int* rt, int* ks, int* wn);

}  // namespace isd
