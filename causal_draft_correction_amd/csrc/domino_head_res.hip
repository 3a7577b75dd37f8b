// The persistent draft kernel that keeps each block's W2 slice on chip, built
// for 256-thread blocks: one wave per SIMD, so each wave may hold up to 512
// registers, enough for its share of the slice (RES_RT tiles of 16 rows x 256).
#define DH_NT 256
#define DH_NS dh256
#include "dh_phases.h"
#include "dh_resident.h"

namespace DH_NS {

// Same draft with the block's W2 slice resident on chip and multiplied on the
// matrix cores (bf16 weights, r = 32 * KS, B <= BC).  The slice is loaded once,
// overlapped with the prologue; every position then reads it from registers
// and LDS instead of streaming 2 r V bytes from HBM.
template <int RT, int KS, int NB>
__global__ __launch_bounds__(NT) void k_persistent_res(Params p)
{
    extern __shared__ float smem[];
    const int blk = blockIdx.x, nblk = gridDim.x;
    float *S_lds = smem + smem_off_S(p.r, lbuf_stride(p.V, nblk));
    float *cache = S_lds + BC * p.h;
    uint4 *tl = reinterpret_cast<uint4 *>(cache + state_cache_floats(p.r, p.h, p.K, nblk, 2));
    int *atok = reinterpret_cast<int *>(smem + smem_off_tok()) + ATOK_OFF;
    int *bad = atok + BC;
    uint64_t *local_keys = reinterpret_cast<uint64_t *>(smem);
    DH_TRACE(511);
    unsigned gen = barrier_gen_init(p.bar);
    block_fail_init();
    if (blk == 0) {
        prologue_bookkeeping(p);
        if (threadIdx.x < p.B)
            bad[threadIdx.x] = row_bad(p, threadIdx.x) ? 1 : 0;
    }
    // u words of a position carry tag gen + 1 (gen: the barrier generation when its
    // state phase runs), never 0, the value cleared words hold
    DH_TRACE(511);
    W2Resident<RT, KS> res;
    if (NB == 1 && !p.S_init && (p.P || p.gtag)) {
        // one batch row, no initial state, folded table or tagged input-gate words:
        // the prologue needs no grid barrier.  Each wave computes the A_H entries of
        // its own u rows, q_0 is b_hh, the anchor step's input part (not folded) goes
        // out in tagged words that its state phase polls, and the W2 slice load is
        // issued after the anchor gate update's loads, so it overlaps the dot
        // products and the first u exchange
        lbase_to_lds(p, blk, nblk, 0, smem);
        DH_TRACE(507);
        state_cache_load<bf16s>(p, blk, nblk, cache, false);
        DH_TRACE(506);
        ah_local_to_cache<bf16s>(p, blk, nblk, cache);
        DH_TRACE(505);
        if (!p.P)
            phase_g<bf16s, 3>(p, blk, nblk, 0, smem, nullptr, gen + 1);
        DH_TRACE(508);
        DH_TRACE(510);
        phase_state<bf16s>(p, blk, nblk, 0, smem, S_lds, nullptr, cache, true, nullptr, gen + 1,
                           [&] { w2_resident_load<RT, KS>(p, blk, nblk, res, tl); });
    } else {
        phase_ah<bf16s>(p, blk, nblk, smem);
        phase_q_init<bf16s>(p, blk, nblk);
        lbase_to_lds(p, blk, nblk, 0, smem);
        // (g words of the anchor step: tagged for the state phase after the barrier below)
        if (!p.P)
            phase_g<bf16s, 3>(p, blk, nblk, 0, smem, nullptr, gen + 2);
        // the slice load overlaps the first barrier
        w2_resident_load<RT, KS>(p, blk, nblk, res, tl);
        DH_TRACE(508);
        if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
            return;
        DH_TRACE(510);
        state_cache_load<bf16s>(p, blk, nblk, cache);
        phase_state<bf16s>(p, blk, nblk, 0, smem, S_lds, nullptr, cache, true, nullptr, gen + 1);
    }
    // from here on one barrier per position: the argmax barrier, which also
    // publishes the q values of the state phase before it; u travels in tagged
    // words that the W2 phase polls
    DH_TRACE(509);
    for (int pos = 0; pos < p.K; ++pos) {
        // the output and exchange pointers pass through an opaque copy each position,
        // so the per-thread addresses derived from them are recomputed here instead of
        // being hoisted out of the loop into (spilled) registers
        Params pl = p;
        asm volatile("" : "+s"(pl.asy), "+s"(pl.tokens), "+s"(pl.utag), "+s"(pl.q_buf), "+s"(pl.P), "+s"(pl.L_final),
                          "+s"(pl.S_out), "+s"(pl.u_out), "+s"(pl.L_base));
        if (!phase_w2_resident<RT, KS, NB>(pl, blk, nblk, pos, smem, res, tl, local_keys, gen + 1))
            return;
        argmax_arrive(pl.asy, gen, local_keys, pl.B);
        DH_TRACE(pos * 32 + 6);
        // L_base of the next position goes to LDS while the barrier is awaited (the
        // compiler makes the thread's next LDS access wait for these loads)
        if (pos + 1 < pl.K)
            lbase_to_lds(pl, blk, nblk, pos + 1, smem);
        DH_TRACE(pos * 32 + 7);
        if (!argmax_wait(pl.asy, gen, pl.B, atok, pl.spin_limit, pl.flags))
            return;
        if (blk == 0 && threadIdx.x < pl.B)
            pl.tokens[static_cast<size_t>(threadIdx.x) * pl.K + pos] = bad[threadIdx.x] ? -1 : atok[threadIdx.x];
        DH_TRACE(pos * 32 + 13);
        DH_TRACE(pos * 32 + 15);  // (back to back: the cost of one mark)
        if (pos + 1 < pl.K) {
            if (!pl.P) {
                // the input product goes out in tagged words, which the state phase
                // polls: no grid barrier
                phase_g<bf16s, 3>(pl, blk, nblk, pos + 1, smem, atok, gen + 1);
                DH_TRACE(pos * 32 + 14);
                if (!pl.gtag && !grid_sync(pl.bar, gen, pl.spin_limit, pl.flags))
                    return;
            }
            // q of this step is visible only after the argmax barrier: its loads go out
            // together with those of the P row
            phase_state<bf16s>(pl, blk, nblk, pos + 1, smem, S_lds, nullptr, cache, true, atok, gen + 1);
        }
    }
    // the last position's tag is gen
    utag_refresh(p, blk, nblk, gen);
    barrier_finish(p.bar, gen);
}


// Markov head (markov_u): the same resident-W2 draft with the state phase
// replaced by a table gather.  Every block forms u of every batch row itself
// from A_H and the table row of the preceding token, so no value crosses
// blocks between the argmax barrier and the W2 phase; the only exchange per
// position is the argmax barrier.  The prologue computes A_H over the grid and
// ends with one grid barrier (the W2 slice load overlaps it).
template <int RT, int KS, int NB>
__global__ __launch_bounds__(NT) void k_markov_res(Params p)
{
    extern __shared__ float smem[];
    const int blk = blockIdx.x, nblk = gridDim.x;
    // LDS as in k_persistent_res (the tiles beyond the register share at the same
    // offset); the state regions are unused
    float *S_lds = smem + smem_off_S(p.r, lbuf_stride(p.V, nblk));
    float *cache = S_lds + BC * p.h;
    uint4 *tl = reinterpret_cast<uint4 *>(cache + state_cache_floats(p.r, p.h, p.K, nblk, 2));
    float *u_lds = smem + smem_off_u();  // [BC][r]
    int *atok = reinterpret_cast<int *>(smem + smem_off_tok()) + ATOK_OFF;
    int *bad = atok + BC;
    uint64_t *local_keys = reinterpret_cast<uint64_t *>(smem);
    const int r = p.r;
    unsigned gen = barrier_gen_init(p.bar);
    block_fail_init();
    if (blk == 0) {
        prologue_bookkeeping(p);
        if (threadIdx.x < p.B)
            bad[threadIdx.x] = row_bad(p, threadIdx.x) ? 1 : 0;
    }
    W2Resident<RT, KS> res;
    phase_ah<bf16s>(p, blk, nblk, smem);
    lbase_to_lds(p, blk, nblk, 0, smem);
    w2_resident_load<RT, KS>(p, blk, nblk, res, tl);
    if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
        return;
    // thread m < r forms u[b][m]; its A_H entries of the coming position are
    // loaded one position ahead (during the argmax barrier wait)
    const int m = threadIdx.x;
    float ah[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
        ah[b] = (b < p.B && m < r) ? xld(&p.A_H[static_cast<size_t>(b) * p.K * r + m]) : 0.f;
    for (int pos = 0; pos < p.K; ++pos) {
        Params pl = p;
        asm volatile("" : "+s"(pl.asy), "+s"(pl.tokens), "+s"(pl.L_final), "+s"(pl.u_out), "+s"(pl.L_base),
                          "+s"(pl.M));
        if (m < r) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b < pl.B) {
                    const float u = markov_u(pl, ah[b], m, gru_input_token(pl, pos, b, atok));
                    u_lds[b * r + m] = u;
                    if (blk == 0 && pl.u_out)
                        pl.u_out[(static_cast<size_t>(b) * pl.K + pos) * r + m] = u;
                }
            }
        }
        __syncthreads();
        if (!phase_w2_resident<RT, KS, NB>(pl, blk, nblk, pos, smem, res, tl, local_keys, 0u, u_lds))
            return;
        argmax_arrive(pl.asy, gen, local_keys, pl.B);
        if (pos + 1 < pl.K) {
            lbase_to_lds(pl, blk, nblk, pos + 1, smem);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < pl.B && m < r)
                    ah[b] = xld(&pl.A_H[(static_cast<size_t>(b) * pl.K + pos + 1) * r + m]);
        }
        if (!argmax_wait(pl.asy, gen, pl.B, atok, pl.spin_limit, pl.flags))
            return;
        if (blk == 0 && threadIdx.x < pl.B)
            pl.tokens[static_cast<size_t>(threadIdx.x) * pl.K + pos] = bad[threadIdx.x] ? -1 : atok[threadIdx.x];
    }
    barrier_finish(p.bar, gen);
}

constexpr int RES_RT = 10;  // W2 tiles per wave kept in registers (4 waves x 10 x 16 rows = 640 rows; the rest in LDS)
constexpr int RES_KS = 8;   // 32-wide steps of r: r = 256

}  // namespace DH_NS

namespace dhres {

using namespace dh256;

int threads() { return NT; }
int r_supported() { return 32 * RES_KS; }
// B = 1 (the common case) gets an instantiation whose per-row registers hold one row
const void *kernel(int B)
{
    return B <= 1 ? reinterpret_cast<const void *>(&k_persistent_res<RES_RT, RES_KS, 1>)
                  : reinterpret_cast<const void *>(&k_persistent_res<RES_RT, RES_KS, BC>);
}
// the Markov head's kernel (same LDS size and grid)
const void *markov_kernel(int B)
{
    return B <= 1 ? reinterpret_cast<const void *>(&k_markov_res<RES_RT, RES_KS, 1>)
                  : reinterpret_cast<const void *>(&k_markov_res<RES_RT, RES_KS, BC>);
}

size_t smem_bytes(int r, int h, int K, int V, int nblk)
{
    const int rows_cap = lbuf_stride(V, nblk);
    const int tiles = rows_cap / 16;
    const int lds_tiles = tiles > NWAVE * RES_RT ? tiles - NWAVE * RES_RT : 0;
    return sizeof(float) * (smem_floats(r, h, rows_cap) + state_cache_floats(r, h, K, nblk, 2)) +
           static_cast<size_t>(lds_tiles) * RES_KS * 64 * 16;
}

}  // namespace dhres
