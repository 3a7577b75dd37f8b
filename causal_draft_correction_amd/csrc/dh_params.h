// Arguments of one block draft, shared by every kernel of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dhp {

struct Params {
    int d, h, r, V, K, B, maxB;
    const void *W1, *W2, *W_ih, *W_hh, *b_ih, *b_hh, *E;
    const float *P;  // folded input-gate table [V, 3h] or nullptr
    const float *M;  // Markov head: per-token table [V, r] = W1_S GRU(E[t], 0), or nullptr (recurrent head)
    const void *H;
    const void *L_base;  // [B, K, V] float32, or bfloat16 bits when lbase_bf16
    const int *last_tok, *teacher;
    const float *S_init;
    int *tokens;
    float *L_final, *S_out, *u_out;
    // workspace
    float *A_H;      // [maxB, K, r]
    float *S_buf;    // [2, maxB, h]  state carried between stepwise launches
    float *u_buf;    // [maxB, r]
    uint32_t *utag;  // [2, maxB, r] u as matrix-core operand: words (tag << 16) | bf16 bits of the
                     // hi part (plane 0) and lo part (plane 1) of u, or nullptr
    float *q_buf;    // [2, maxB, 3h] W_hh S + b_hh
    uint16_t *s_hl;  // [2, maxB, ldw] bf16 hi and lo parts of S (matrix-core state dots) or nullptr
    const uint16_t *wst;  // [r + 3h, ldw] bf16: the W1_S rows, then the W_hh rows, with a padded
                          // row stride (matrix-core state dots), or nullptr
    int ldw;              // row stride of s_hl and wst in elements
    float *g_buf;    // [maxB, 3h]    W_ih E[x] + b_ih (when not folded)
    uint64_t *gtag;  // [min(maxB, BC), 3h] resident launch, not folded: g as words (tag << 32) |
                     // float bits, which the state phase polls instead of a grid barrier; or nullptr
    uint64_t *keys;  // [K, NG, maxB] partial argmax keys
    uint64_t *bkeys; // batched resident launch: [maxB, grid] argmax key word of every block for every
                     // batch row, generation-tagged
    uint4 *uop;      // batched resident launch: u as the W2 products' operand, one slot per position:
                     // [K][rb_ngr][r/32][64] 16-byte chunks (8 bf16 of one batch row each)
    uint16_t *rb_planes;  // batched resident launch: S as bf16 hi/lo planes, one slot per state:
                          // [K + 1][2][rb_bmax][rb_ldp]
    int rb_bmax, rb_ngr, rb_ldp;
    unsigned *rb_ucnt;    // batched resident launch: [K] blocks whose u operand of the position is written
    unsigned *bar;   // barrier words
    uint64_t *asy;   // argmax barrier words
    unsigned *flags; // device flags
    unsigned spin_limit;
    int persistent;  // 1: blocks keep the state in LDS between phases
    int ah_external; // 1: A_H is computed by its own (matrix-core) launch, not by the prologue
    int bf16w;       // 1: weights are bf16, 0: float32
    int lbase_bf16;  // 1: L_base holds bfloat16 bit patterns
};

}  // namespace dhp
