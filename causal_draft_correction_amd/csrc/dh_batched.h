// Host entry points of the batched matrix-core W2 kernel (domino_head_bat.hip).
#pragma once

#include <stddef.h>

namespace dhbat {
int r_supported();         // the rank it is built for
int threads();             // threads per block
// k_w2_mfma for B rows (L_base float32 or bf16; L_final stored or not; u_single:
// u as one bf16 operand instead of bf16 hi + lo parts): arguments (Params, int
// position, int groups)
const void *w2_kernel(int B, bool lbase_bf16, bool store_logits, bool u_single);
int w2_groups(int B);           // its third argument
int w2_threads(int B);     // its threads per block
size_t w2_smem();          // its dynamic LDS per block
int w2_grid(int B, int cus);  // blocks for B batch rows on cus compute units
const void *state_kernel(int B, int h);  // state dots on the matrix cores (bf16 weights): arguments (Params, int q)
int state_grid(int B, int r, int h);
const void *ah_kernel(int B, int K, int r);  // k_ah_mfma for B K rows (bf16 H and W1, d and r multiples
                                             // of 32): arguments (Params)
int ah_grid(int B, int K, int r);
}  // namespace dhbat
