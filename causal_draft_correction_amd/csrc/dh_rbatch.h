// Host entry points of the batched resident-W2 persistent kernel (domino_head_rb.hip).
#pragma once

#include <stddef.h>

namespace dhrb {
int threads();                // threads per block
int r_supported();            // the rank it is built for
int max_batch();              // largest batch of one launch
int tiles_per_block();        // 16-row vocabulary tiles a block holds in registers
// Whether a launch of `grid` blocks handles these shapes (h and r+3h multiples of 64, the
// vocabulary split into at most tiles_per_block() tiles per block).
bool supports(int d, int h, int r, int V, int grid);
// Kernel for this L_base element type, L_final store and head (recurrent or Markov);
// arguments (Params).  The vocabulary's row length decides whether L_base rows are copied
// in 16-byte pieces.
const void *kernel(bool lbase_bf16, bool store_logits, int V, bool markov);
}  // namespace dhrb
