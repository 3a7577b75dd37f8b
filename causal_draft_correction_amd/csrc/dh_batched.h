// Host entry points of the batched matrix-core W2 kernel (domino_head_bat.hip).
#pragma once

namespace dhbat {
int r_supported();         // the rank it is built for
int threads();             // threads per block
const void *w2_kernel();   // k_w2_mfma: arguments (Params, int position)
int w2_grid(int B, int cus);  // blocks for B batch rows on cus compute units
}  // namespace dhbat
