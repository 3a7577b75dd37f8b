// Host entry points of the resident-W2 persistent kernel (domino_head_res.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace dhres {
int threads();            // threads per block of the kernel
int r_supported();        // the rank it is built for
const void *kernel(int B);  // kernel for B batch rows (B <= 8), launched with one block per compute unit
const void *markov_kernel(int B);  // the same for a Markov head (Params::M set)
size_t smem_bytes(int r, int h, int K, int V, int nblk);  // dynamic LDS of one block
}  // namespace dhres
