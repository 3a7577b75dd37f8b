// Batched drafting (9 <= B <= 256 rows, bf16 weights, r = 256, folded gate
// table) in one persistent launch that keeps each block's W2 slice in
// registers for all K positions.  The same method as every other launch
// (paper.oopus.info review, section 二, 第二步 Domino Head; news.sig.ai
// article, section "Domino怎么做"), per position p:
//   u_p = SiLU(A_H[p] + W1_S S_p),  L_p = L_base_p + W2 u_p,  t_p = argmax L_p,
//   S_{p+1} = GRU(E[x_p], S_p)   (x_p = t_p, or the teacher token)
// with the GRU input part a row of the folded table P = E W_ih^T + b_ih.
//
// One block per compute unit, four waves (one per SIMD, up to 512 registers
// each).  Block b owns a contiguous range of 16-row vocabulary tiles; wave w
// holds tiles w, w + 4, ... of it (RT per wave, 320 registers at r = 256).
// Per position the launch runs three phases separated by grid barriers:
//   * W2 phase: for each group of 16 batch rows, D = W2_tile u^T on the matrix
//     cores (v_mfma_f32_16x16x32_bf16, A = the register tile, B = u as bf16 hi
//     and lo operands accumulated into the same result, so the product keeps
//     float32-level accuracy), plus L_base, into a running greedy argmax.  The
//     groups' L_base slices (two groups ahead) and u operands (one ahead) are
//     copied into LDS by direct global-to-LDS loads.  The block's key for each
//     batch row goes to a generation-tagged word bkeys[b][block];
//   * update phase: every block owns a contiguous range of the B x h state
//     entries; it reduces the argmax words of its rows (polling until all carry
//     this position's tag), writes the tokens of the rows whose first entry it
//     owns, and steps the GRU for its entries (P row, q = W_hh S + b_hh and the
//     previous state, which stays with its owner), writing S as float32 and as
//     bf16 hi/lo planes;
//   * state-dot phase: [u | q'] = S [B, h] x [W1_S; W_hh]^T on the matrix cores
//     in jobs of 4 weight tiles x BJ batch tiles (S hi and lo staged in LDS,
//     weight rows from L2), then u = SiLU(A_H + .) as the next W2 phase's bf16
//     hi/lo operand and q' + b_hh for the next update.
// Values that cross blocks (keys, q, the S planes, the u operand) are written
// with agent-scope stores and read with agent-scope loads (or copies with the
// same cache policy), which bypass the per-XCD L2 caches.
#define DH_NT 256
#define DH_NS dh256
#include "dh_phases.h"
#include "dh_rbatch.h"

// Optional instrumentation: a translation unit may define RB_MARK(slot) before
// including this file to record timestamps at phase boundaries (slot = 64 *
// position + point; the prologue uses slots 1018..1023).  The default is a no-op.
#ifndef RB_MARK
#define RB_MARK(slot) ((void)(slot))
#endif

namespace DH_NS {
namespace rbk {

constexpr int RT = 10;               // W2 tiles per wave in registers
constexpr int KS = 8;                // 32-wide steps of r
constexpr int R = 32 * KS;           // r
constexpr int TILES = NWAVE * RT;    // vocabulary tiles per block (40: 640 rows)
constexpr int LROW = TILES * 16;     // L_base values of one batch row in LDS
constexpr int LBUF = 16 * LROW * 4 / 16;  // uint4 per L_base buffer (16 rows of float32)
constexpr int UCH = 2 * KS * 64;     // uint4 of one group's u operand (hi, lo)
constexpr int MAXB = 256;            // batch rows of one launch
constexpr int ROWS = 4;              // batch rows one block updates at most (B <= MAXB)
constexpr int CPT = 2;               // 4-entry state chunks per thread at most
constexpr unsigned AUX_SC1 = 16;     // cache policy of agent-scope coherent accesses (sc1)

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(n), expcnt and lgkmcnt left at their maxima
template <int N>
__device__ inline void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ inline void bare_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ inline void st_agent_u64(void *p, uint64_t v)
{
    __hip_atomic_store(static_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float4 ld_agent_f4(const float *p)
{
    const uint64_t a = ld_agent_u64(reinterpret_cast<const uint64_t *>(p));
    const uint64_t b = ld_agent_u64(reinterpret_cast<const uint64_t *>(p) + 1);
    return make_float4(__uint_as_float(static_cast<uint32_t>(a)), __uint_as_float(static_cast<uint32_t>(a >> 32)),
                       __uint_as_float(static_cast<uint32_t>(b)), __uint_as_float(static_cast<uint32_t>(b >> 32)));
}
__device__ inline void st_agent_f4(float *p, float4 v)
{
    st_agent_u64(p, (static_cast<uint64_t>(__float_as_uint(v.y)) << 32) | __float_as_uint(v.x));
    st_agent_u64(p + 2, (static_cast<uint64_t>(__float_as_uint(v.w)) << 32) | __float_as_uint(v.z));
}
// Direct global-to-LDS copies of 16, 4 or 2 bytes per lane (lane l writes at lds + l * size)
__device__ inline void copy_lds16(const void *g, void *lds, unsigned aux_sc1)
{
    if (aux_sc1)
        __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 16, 0, AUX_SC1);
    else
        __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 16, 0, 0);
}
__device__ inline void copy_lds4(const void *g, void *lds) { __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 4, 0, 0); }
__device__ inline void copy_lds2(const void *g, void *lds) { __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 2, 0, 0); }

__device__ inline uint64_t pack4_bf16(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return static_cast<uint64_t>(a | (b << 16)) | (static_cast<uint64_t>(c | (d << 16)) << 32);
}

// The block's share of the work, the same at every position.
struct Ctx {
    int v0, n;       // vocabulary rows [v0, v0 + n) (v0 a multiple of 16; n may be 0)
    int c0, c1;      // 4-entry state chunks [c0, c1) of the flat [B, h] index
    int rb0, nrows;  // batch rows of those chunks: rb0 .. rb0 + nrows - 1
};

__device__ inline Ctx make_ctx(const Params &p, int blk, int nblk)
{
    Ctx c;
    const long long T = (p.V + 15) / 16;
    const int ta = static_cast<int>(T * blk / nblk), tb = static_cast<int>(T * (blk + 1) / nblk);
    c.v0 = 16 * ta;
    c.n = (16 * tb < p.V ? 16 * tb : p.V) - c.v0;
    if (c.n < 0)
        c.n = 0;
    const int nc = p.B * p.h / 4, per = (nc + nblk - 1) / nblk;
    c.c0 = blk * per < nc ? blk * per : nc;
    c.c1 = c.c0 + per < nc ? c.c0 + per : nc;
    c.rb0 = c.c0 * 4 / p.h;
    c.nrows = c.c1 > c.c0 ? (c.c1 * 4 - 1) / p.h - c.rb0 + 1 : 0;
    return c;
}

// ---- W2 phase ------------------------------------------------------------------
// L_base of batch group g (rows 16 g .. 16 g + 15, clamped to B - 1) at position
// pos into an LDS buffer: row i holds the block's values of batch row 16 g + i in
// 16-byte chunks whose index is XOR-ed with (i & 7), so the 16 rows that one read
// instruction of the epilogue touches fall on different banks.  Every thread issues
// the same number of copies (NLD) whatever B and the block's range: chunks past the
// range re-read the row's first chunk, groups past the last re-read the last group.
// FAST: rows copied in 16-byte pieces (V a multiple of 4 for float32, 8 for bf16,
// so every row starts 16-byte aligned); otherwise one value per lane (bf16 values
// are loaded into registers and stored to LDS: a 2-byte direct copy fills a whole
// 4-byte LDS word per lane).
template <bool LB16, bool FAST>
struct LbCopy {
    static constexpr int EL = LB16 ? 2 : 4;            // bytes per value
    static constexpr int PIECE = FAST ? 16 : EL;       // bytes per lane per copy
    static constexpr int ROWB = LROW * EL;             // bytes of one LDS row
    static constexpr int NLD = 16 * ROWB / (64 * PIECE) / NWAVE;  // copies per thread per group
    static_assert(16 * ROWB % (64 * PIECE * NWAVE) == 0, "whole copies per wave");
};

template <bool LB16, bool FAST>
__device__ __forceinline__ void lb_issue(const Params &p, const Ctx &c, int pos, int g, uint4 *buf)
{
    using C = LbCopy<LB16, FAST>;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const char *base = static_cast<const char *>(p.L_base);
    const int ngr = (p.B + 15) / 16;
    g = g < ngr ? g : ngr - 1;
    constexpr int VPC = 16 / C::EL;  // values per 16-byte chunk
    if constexpr (LB16 && !FAST) {
        constexpr int BATCH = 8;
#pragma unroll
        for (int j0 = 0; j0 < C::NLD; j0 += BATCH) {
            uint16_t v[BATCH];
#pragma unroll
            for (int jj = 0; jj < BATCH; ++jj) {
                const int s = 64 * (wave * C::NLD + j0 + jj) + lane;
                const int row = s / LROW, pr = s % LROW;
                int e = ((pr / 8) ^ (row & 7)) * 8 + pr % 8;
                e = e < c.n ? e : 0;
                const int b = 16 * g + row < p.B ? 16 * g + row : p.B - 1;
                v[jj] = reinterpret_cast<const uint16_t *>(base)[(static_cast<size_t>(b) * p.K + pos) * p.V + c.v0 + e];
            }
#pragma unroll
            for (int jj = 0; jj < BATCH; ++jj)
                reinterpret_cast<uint16_t *>(buf)[64 * (wave * C::NLD + j0 + jj) + lane] = v[jj];
        }
        return;
    }
#pragma unroll
    for (int jj = 0; jj < C::NLD; ++jj) {
        const int i = wave * C::NLD + jj;     // copy index within the group
        const int s = 64 * i + lane;          // this lane's piece
        const int row = s / (C::ROWB / C::PIECE);
        const int pr = s % (C::ROWB / C::PIECE);  // piece within the LDS row
        int e;                                    // value index within the block's range
        if constexpr (FAST) {
            e = ((pr ^ (row & 7)) * VPC);
        } else {
            constexpr int PPC = 16 / C::PIECE;    // pieces per chunk
            e = ((pr / PPC) ^ (row & 7)) * VPC + pr % PPC;
        }
        e = e < c.n ? e : 0;
        const int b = 16 * g + row < p.B ? 16 * g + row : p.B - 1;
        const char *src = base + ((static_cast<size_t>(b) * p.K + pos) * p.V + c.v0 + e) * C::EL;
        char *dst = reinterpret_cast<char *>(buf) + i * 64 * C::PIECE;
        if constexpr (C::PIECE == 16)
            copy_lds16(src, dst, 0);
        else if constexpr (C::PIECE == 4)
            copy_lds4(src, dst);
        else
            copy_lds2(src, dst);
    }
}

// u operand of group g (16 KB, the layout of p.uop) into an LDS buffer: 4 copies per thread.
__device__ __forceinline__ void u_issue(const Params &p, int g, uint4 *buf)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int ngr = (p.B + 15) / 16;
    g = g < ngr ? g : ngr - 1;
#pragma unroll
    for (int jj = 0; jj < UCH / 64 / NWAVE; ++jj) {
        const int i = wave * (UCH / 64 / NWAVE) + jj;
        copy_lds16(p.uop + static_cast<size_t>(g) * UCH + 64 * i + lane, buf + 64 * i, 1);
    }
}

// Four L_base values of this lane for tile t (vocabulary rows 16 t + 4 k .. + 3 of
// batch row `row` of the group, k = lane / 16).
template <bool LB16>
__device__ inline float4 lb_read(const uint4 *buf, int row, int t, int k)
{
    if constexpr (LB16) {
        const int chunk = (2 * t + (k >> 1)) ^ (row & 7);
        const uint2 v = *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(buf) +
                                                         (row * (LROW * 2 / 16) + chunk) * 16 + (k & 1) * 8);
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.y << 16),
                           __uint_as_float(v.y & 0xFFFF0000u));
    } else {
        const uint4 v = buf[row * (LROW / 4) + ((4 * t + k) ^ (row & 7))];
        return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
    }
}

// Products and epilogue of group g for this wave: result lane l holds vocabulary
// rows 16 t + 4 (l / 16) + i (i = 0..3) of tile t = wave + 4 j for batch row
// 16 g + l % 16.  The lane keeps the first of its largest values (a NaN above every
// number, the first NaN kept; -0 == +0 by the float compare); the wave's key for
// each of the group's batch rows goes to kr[wave][0..15].
template <bool LB16, bool ST>
__device__ __forceinline__ void w2_group(const Params &p, const Ctx &c, const W2Resident<RT, KS> &res, int pos, int g,
                                         const uint4 *L, const uint4 *U, uint64_t *kr)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int row = lane & 15, k = lane >> 4;
    f32x4_t acc[RT];
#pragma unroll
    for (int j = 0; j < RT; ++j)
        acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const uint4 uh = U[kk * 64 + lane], ul = U[(KS + kk) * 64 + lane];
#pragma unroll
        for (int j = 0; j < RT; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, res.wt[j][kk]),
                                                             __builtin_bit_cast(bf16x8_t, uh), acc[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < RT; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, res.wt[j][kk]),
                                                             __builtin_bit_cast(bf16x8_t, ul), acc[j], 0, 0, 0);
    }
    const int b = 16 * g + row;
    float best = -__builtin_inff();
    int bpos = -1;
    float *lf = nullptr;
    if constexpr (ST)
        lf = p.L_final + (static_cast<size_t>(b < p.B ? b : 0) * p.K + pos) * p.V + c.v0;
#pragma unroll
    for (int j = 0; j < RT; ++j) {
        const int t = wave + NWAVE * j;
        const float4 lb = lb_read<LB16>(L, row, t, k);
        const float lv[4] = {lb.x, lb.y, lb.z, lb.w};
        const bool full = 16 * (t + 1) <= c.n;  // uniform in the wave
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = acc[j][i] + lv[i];
            const int vr = 16 * t + 4 * k + i;
            const bool ok = full || vr < c.n;
            if constexpr (ST) {
                if (ok && b < p.B)
                    lf[vr] = v;
            }
            const bool take = !(v <= best) & (best == best) & ok;
            best = take ? v : best;
            bpos = take ? 4 * j + i : bpos;
        }
    }
    uint64_t key = 0;
    if (bpos >= 0) {
        const uint32_t idx = static_cast<uint32_t>(c.v0 + 16 * (wave + NWAVE * (bpos >> 2)) + 4 * k + (bpos & 3));
        const uint32_t bits = __float_as_uint(best + 0.f);  // -0 + +0 = +0
        uint32_t ord = bits ^ (static_cast<uint32_t>(static_cast<int32_t>(bits) >> 31) | 0x80000000u);
        ord = (best != best) ? 0xFFFFFFFFu : ord;
        key = (static_cast<uint64_t>(ord) << 32) | (KEY_IDX_MASK - idx);
    }
    key = rows_max_u64(key);
    if (lane < 16)
        kr[wave * 16 + lane] = key;
}

// The W2 phase of position pos: every group's products and argmax, then the
// block's key word of every batch row, tagged `tag14`.
template <bool LB16, bool FAST, bool ST>
__device__ __forceinline__ void w2_phase(const Params &p, const Ctx &c, const W2Resident<RT, KS> &res, int pos,
                                         uint32_t tag14, uint4 *lbA, uint4 *lbB, uint4 *lbC, uint4 *uA, uint4 *uB,
                                         uint64_t *kred, uint64_t *lkey)
{
    using C = LbCopy<LB16, FAST>;
    const int ngr = (p.B + 15) / 16;
    // block key of group gp from the four waves' keys (after a barrier)
    auto fold = [&](int gp) {
        if (threadIdx.x < 16) {
            const uint64_t *kr = kred + (gp & 1) * NWAVE * 16;
            uint64_t m = 0;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w)
                m = max_u64(m, kr[w * 16 + threadIdx.x]);
            lkey[16 * gp + threadIdx.x] = m;
        }
    };
    // group g: wait for its copies (those of the L_base group after it may stay in
    // flight: they were issued last), meet the other waves, fold the previous group's
    // keys, start the copies of u(g + 1) and L_base(g + 2), then the products
    auto iter = [&](int g, const uint4 *Lc, uint4 *Ln2, const uint4 *Uc, uint4 *Un) {
        wait_vm<C::NLD>();
        bare_barrier();
        if (g >= 1)
            fold(g - 1);
        u_issue(p, g + 1, Un);
        lb_issue<LB16, FAST>(p, c, pos, g + 2, Ln2);
        w2_group<LB16, ST>(p, c, res, pos, g, Lc, Uc, kred + (g & 1) * NWAVE * 16);
    };
    lb_issue<LB16, FAST>(p, c, pos, 0, lbA);
    u_issue(p, 0, uA);
    lb_issue<LB16, FAST>(p, c, pos, 1, lbB);
    // group g uses L_base buffer g % 3 and u buffer g % 2
#pragma unroll 1
    for (int g0 = 0; g0 < ngr; g0 += 6) {
        RB_MARK(64 * pos + 8 + g0);
        iter(g0, lbA, lbC, uA, uB);
        if (g0 + 1 >= ngr)
            break;
        iter(g0 + 1, lbB, lbA, uB, uA);
        if (g0 + 2 >= ngr)
            break;
        iter(g0 + 2, lbC, lbB, uA, uB);
        if (g0 + 3 >= ngr)
            break;
        iter(g0 + 3, lbA, lbC, uB, uA);
        if (g0 + 4 >= ngr)
            break;
        iter(g0 + 4, lbB, lbA, uA, uB);
        if (g0 + 5 >= ngr)
            break;
        iter(g0 + 5, lbC, lbB, uB, uA);
    }
    __syncthreads();
    fold(ngr - 1);
    __syncthreads();
    for (int b = threadIdx.x; b < p.B; b += NT) {
        const uint64_t m = lkey[b];
        st_agent_u64(&p.bkeys[static_cast<size_t>(b) * gridDim.x + blockIdx.x],
                     (m & (KEY_ORD_MASK | KEY_IDX_MASK)) | (static_cast<uint64_t>(tag14) << 18));
    }
}

// ---- update phase -----------------------------------------------------------------
// Tokens of position pos for the block's rows (max over every block's word, each
// polled until it carries tag14) into rtok; tokens[b][pos] written for the rows
// whose first state entry this block owns.  False on a timeout.
__device__ __forceinline__ bool resolve(const Params &p, const Ctx &c, int pos, uint32_t tag14, int *rtok,
                                        uint64_t *rred)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nblk = gridDim.x;
    uint64_t best[ROWS];
#pragma unroll
    for (int ri = 0; ri < ROWS; ++ri)
        best[ri] = 0;
    int ok = 1;
    for (int q = threadIdx.x; q < nblk; q += NT) {
#pragma unroll
        for (int ri = 0; ri < ROWS; ++ri) {
            if (ri < c.nrows) {
                const uint64_t *wp = &p.bkeys[static_cast<size_t>(c.rb0 + ri) * nblk + q];
                uint64_t w;
                unsigned spins = 0;
                for (;;) {
                    w = ld_agent_u64(wp);
                    if (static_cast<uint32_t>((w >> 18) & 0x3FFFu) == tag14)
                        break;
                    if (++spins > p.spin_limit) {
                        ok = 0;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                best[ri] = max_u64(best[ri], w & (KEY_ORD_MASK | KEY_IDX_MASK));
            }
        }
    }
#pragma unroll
    for (int ri = 0; ri < ROWS; ++ri) {
        if (ri < c.nrows) {
            const uint64_t m = wave_max_u64(best[ri]);
            if (lane == 0)
                rred[wave * ROWS + ri] = m;
        }
    }
    const bool failed = block_failed(ok);
    if (failed) {
        if (threadIdx.x == 0)
            __hip_atomic_fetch_or(p.flags, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    if (static_cast<int>(threadIdx.x) < c.nrows) {
        uint64_t m = 0;
        for (int w = 0; w < NWAVE; ++w)
            m = max_u64(m, rred[w * ROWS + threadIdx.x]);
        const int tok = m ? static_cast<int>(KEY_IDX_MASK - (m & KEY_IDX_MASK)) : 0;
        rtok[threadIdx.x] = tok;
        const int b = c.rb0 + threadIdx.x;
        if (b * p.h / 4 >= c.c0)  // this block owns the row's first entry
            p.tokens[static_cast<size_t>(b) * p.K + pos] = row_bad(p, b) ? -1 : tok;
    }
    __syncthreads();
    return true;
}

// S_q for the block's entries.  q = -1: only the hi/lo planes of S_init (for the
// dots that give W_hh S_init + b_hh).  Entries stay with their owner thread, so
// S_buf is written and read by the same thread only.
__device__ __forceinline__ void update(const Params &p, const Ctx &c, int q, const int *rtok)
{
    const int h = p.h, h3 = 3 * h;
    uint16_t *plane_hi = p.s_hl, *plane_lo = p.s_hl + static_cast<size_t>(p.maxB) * p.ldw;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int cc = c.c0 + static_cast<int>(threadIdx.x) + u * NT;
        if (cc >= c.c1)
            continue;
        const int e = cc * 4, b = e / h, j = e % h;
        float sn[4];
        if (q < 0) {
            const float4 s = *reinterpret_cast<const float4 *>(p.S_init + static_cast<size_t>(b) * h + j);
            sn[0] = s.x, sn[1] = s.y, sn[2] = s.z, sn[3] = s.w;
        } else {
            int x;
            if (q == 0)
                x = p.last_tok[b];
            else if (p.teacher)
                x = p.teacher[static_cast<size_t>(b) * p.K + (q - 1)];
            else
                x = rtok[b - c.rb0];
            x = tok_ok(x, p.V) ? x : 0;
            const float *prow = p.P + static_cast<size_t>(x) * h3 + j;
            const float4 gr = *reinterpret_cast<const float4 *>(prow);
            const float4 gz = *reinterpret_cast<const float4 *>(prow + h);
            const float4 gn = *reinterpret_cast<const float4 *>(prow + 2 * h);
            float4 qr, qz, qn;
            if (q == 0 && !p.S_init) {
                // W_hh S_init + b_hh with S_init = 0 is b_hh itself
                qr = make_float4(bias_hh(p, j), bias_hh(p, j + 1), bias_hh(p, j + 2), bias_hh(p, j + 3));
                qz = make_float4(bias_hh(p, h + j), bias_hh(p, h + j + 1), bias_hh(p, h + j + 2), bias_hh(p, h + j + 3));
                qn = make_float4(bias_hh(p, 2 * h + j), bias_hh(p, 2 * h + j + 1), bias_hh(p, 2 * h + j + 2),
                                 bias_hh(p, 2 * h + j + 3));
            } else {
                const float *qv = q_slot(p, q) + static_cast<size_t>(b) * h3 + j;
                qr = ld_agent_f4(qv);
                qz = ld_agent_f4(qv + h);
                qn = ld_agent_f4(qv + 2 * h);
            }
            float4 sp;
            if (q == 0)
                sp = p.S_init ? *reinterpret_cast<const float4 *>(p.S_init + static_cast<size_t>(b) * h + j)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
            else
                sp = *reinterpret_cast<const float4 *>(p.S_buf + static_cast<size_t>(b) * h + j);
            const float g3[3][4] = {{gr.x, gr.y, gr.z, gr.w}, {gz.x, gz.y, gz.z, gz.w}, {gn.x, gn.y, gn.z, gn.w}};
            const float q3[3][4] = {{qr.x, qr.y, qr.z, qr.w}, {qz.x, qz.y, qz.z, qz.w}, {qn.x, qn.y, qn.z, qn.w}};
            const float s4[4] = {sp.x, sp.y, sp.z, sp.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the cell of gate_update
                const float rg = sigmoidf_(g3[0][i] + q3[0][i]);
                const float zg = sigmoidf_(g3[1][i] + q3[1][i]);
                const float ng = tanhf(g3[2][i] + rg * q3[2][i]);
                sn[i] = (1.f - zg) * ng + zg * s4[i];
            }
            const float4 s = make_float4(sn[0], sn[1], sn[2], sn[3]);
            *reinterpret_cast<float4 *>(p.S_buf + static_cast<size_t>(b) * h + j) = s;
            if (p.S_out)
                *reinterpret_cast<float4 *>(p.S_out + (static_cast<size_t>(b) * p.K + q) * h + j) = s;
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hi[i] = bf16_rne_bits(sn[i]);
            lo[i] = bf16_rne_bits(sn[i] - __uint_as_float(hi[i] << 16));
        }
        const size_t o = static_cast<size_t>(b) * p.ldw + j;
        st_agent_u64(plane_hi + o, pack4_bf16(hi[0], hi[1], hi[2], hi[3]));
        st_agent_u64(plane_lo + o, pack4_bf16(lo[0], lo[1], lo[2], lo[3]));
    }
}

// ---- state-dot phase ------------------------------------------------------------------
// Products of S_q with the packed state rows wst = [W1_S; W_hh] (R = r + 3h rows of
// ldw bf16): a job is 4 weight tiles (one per wave, A operand from L2) x BJ batch
// tiles (B operand: S hi and lo rows, staged in LDS).  The h reduction runs in stages
// of 64 (two 32-wide steps); a stage's operands (BJ * 4 blocks of 1 KB) are copied by
// direct global-to-LDS loads three stages ahead into a ring of four buffers, each
// wave waiting for its own copies and meeting the others at a bare barrier.  The
// weight operands of a stage are loaded into registers with the copies.  Every copy
// and load is issued on every step (stages past the last repeat it), so the wait
// counts are the same on every path.  q = -1: only the W_hh rows (q of S_init).
template <int BJ>
__device__ __forceinline__ void dots(const Params &p, int blk, int nblk, int q, uint4 *ring0, uint4 *ring1,
                                     uint4 *ring2, uint4 *ring3)
{
    const int lane = threadIdx.x & 63, row = lane & 15, k = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int h = p.h, r = p.r, h3 = 3 * h;
    const int Rall = r + h3, nwg = Rall / 64;
    const int nbt = (p.B + 15) / 16, nbj = (nbt + BJ - 1) / BJ;
    const int NS = h / 64;
    const uint16_t *plane[2] = {p.s_hl, p.s_hl + static_cast<size_t>(p.maxB) * p.ldw};
    constexpr int PER = BJ;  // copies per wave per stage (BJ * 4 blocks over 4 waves)
    for (int job = blk; job < nwg * nbj; job += nblk) {
        const int wg = job / nbj, bj = job % nbj;
        const int wt = wg * 4 + wave;  // this wave's weight tile
        const bool active = !(q < 0 && wt * 16 < r);
        // copy sources of this lane: block i = wave * PER + x = (bt * 2 + hilo) * 2 + ks
        const uint16_t *src[PER];
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int i = wave * PER + x, bt = i >> 2, hl = (i >> 1) & 1, ks = i & 1;
            int b = (bj * BJ + bt) * 16 + row;
            b = b < p.B ? b : p.B - 1;
            src[x] = plane[hl] + static_cast<size_t>(b) * p.ldw + 32 * ks + 8 * k;
        }
        const uint16_t *wrow = p.wst + static_cast<size_t>(wt * 16 + row) * p.ldw + 8 * k;
        uint4 wa[4][2];
        auto issue = [&](int s, uint4 *ring, uint4 (&w)[2]) {
            s = s < NS ? s : NS - 1;
#pragma unroll
            for (int x = 0; x < PER; ++x)
                copy_lds16(src[x] + 64 * s, ring + (wave * PER + x) * 64, 1);
            w[0] = *reinterpret_cast<const uint4 *>(wrow + 64 * s);
            w[1] = *reinterpret_cast<const uint4 *>(wrow + 64 * s + 32);
        };
        f32x4_t acc[BJ];
#pragma unroll
        for (int bt = 0; bt < BJ; ++bt)
            acc[bt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](const uint4 *ring, const uint4 (&w)[2]) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int bt = 0; bt < BJ; ++bt)
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl)
                        acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, w[ks]),
                            __builtin_bit_cast(bf16x8_t, ring[((bt * 2 + hl) * 2 + ks) * 64 + lane]), acc[bt], 0, 0, 0);
        };
        // step s: wait until this wave's copies and loads of stage s are done (those of
        // s + 1 and s + 2 may stay in flight), meet the other waves, issue stage s + 3
        // into the buffer of stage s - 1, multiply stage s
        auto step = [&](int s, const uint4 *cur, uint4 *nxt, const uint4 (&wc)[2], uint4 (&wn)[2]) {
            wait_vm<2 * (PER + 2)>();
            bare_barrier();
            issue(s + 3, nxt, wn);
            if (active && s < NS)
                compute(cur, wc);
        };
        issue(0, ring0, wa[0]);
        issue(1, ring1, wa[1]);
        issue(2, ring2, wa[2]);
#pragma unroll 1
        for (int s = 0; s < NS; s += 4) {
            step(s, ring0, ring3, wa[0], wa[3]);
            step(s + 1, ring1, ring0, wa[1], wa[0]);
            step(s + 2, ring2, ring1, wa[2], wa[1]);
            step(s + 3, ring3, ring2, wa[3], wa[2]);
        }
        // the repeated copies of the last steps land before the ring is reused
        wait_vm<0>();
        bare_barrier();
        if (!active)
            continue;
        // epilogue: lane holds weight rows m = 16 wt + 4 k + i of batch row b
        const int m = 16 * wt + 4 * k;
#pragma unroll
        for (int bt = 0; bt < BJ; ++bt) {
            const int b = (bj * BJ + bt) * 16 + row;
            if (b >= p.B)
                continue;
            if (m < r) {
                const float4 ah = *reinterpret_cast<const float4 *>(p.A_H + (static_cast<size_t>(b) * p.K + q) * r + m);
                const float a4[4] = {ah.x + acc[bt][0], ah.y + acc[bt][1], ah.z + acc[bt][2], ah.w + acc[bt][3]};
                float u4[4];
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    u4[i] = a4[i] * sigmoidf_(a4[i]);
                    hi[i] = bf16_rne_bits(u4[i]);
                    lo[i] = bf16_rne_bits(u4[i] - __uint_as_float(hi[i] << 16));
                }
                if (p.u_out)
                    *reinterpret_cast<float4 *>(p.u_out + (static_cast<size_t>(b) * p.K + q) * r + m) =
                        make_float4(u4[0], u4[1], u4[2], u4[3]);
                // operand chunk of (batch row b, r offsets 8 (m / 8) .. + 8): group b / 16,
                // step m / 32, lane b % 16 + 16 ((m % 32) / 8); these four values are its
                // half (m % 8) / 4
                const size_t ch = (static_cast<size_t>(b >> 4) * 2 * KS + (m >> 5)) * 64 + (b & 15) + 16 * ((m & 31) >> 3);
                char *dst = reinterpret_cast<char *>(p.uop + ch) + (m & 7) * 2;
                st_agent_u64(dst, pack4_bf16(hi[0], hi[1], hi[2], hi[3]));
                st_agent_u64(dst + static_cast<size_t>(KS) * 64 * 16, pack4_bf16(lo[0], lo[1], lo[2], lo[3]));
            } else {
                const int mq = m - r;
                const float4 v = make_float4(acc[bt][0] + bias_hh(p, mq), acc[bt][1] + bias_hh(p, mq + 1),
                                             acc[bt][2] + bias_hh(p, mq + 2), acc[bt][3] + bias_hh(p, mq + 3));
                st_agent_f4(q_slot(p, q + 1) + static_cast<size_t>(b) * h3 + mq, v);
            }
        }
    }
}

__device__ __forceinline__ void dots_any(const Params &p, int blk, int nblk, int q, uint4 *r0, uint4 *r1, uint4 *r2,
                                         uint4 *r3)
{
    const int nbt = (p.B + 15) / 16;
    if (nbt >= 4)
        dots<4>(p, blk, nblk, q, r0, r1, r2, r3);
    else if (nbt >= 2)
        dots<2>(p, blk, nblk, q, r0, r1, r2, r3);
    else
        dots<1>(p, blk, nblk, q, r0, r1, r2, r3);
}

template <bool LB16, bool FAST, bool ST>
__global__ __launch_bounds__(NT) void k_persistent_rb(Params p)
{
    __shared__ uint4 lbA[LBUF], lbB[LBUF], lbC[LBUF];
    __shared__ uint4 uA[UCH], uB[UCH];
    __shared__ uint64_t kred[2 * NWAVE * 16];
    __shared__ uint64_t lkey[MAXB];
    __shared__ uint64_t rred[NWAVE * ROWS];
    __shared__ int rtok[ROWS];
    const int blk = blockIdx.x, nblk = gridDim.x;
    unsigned gen = barrier_gen_init(p.bar);
    block_fail_init();
    if (blk == 0) {
        for (int b = threadIdx.x; b < p.B; b += NT)
            if (row_bad(p, b))
                __hip_atomic_fetch_or(p.flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const Ctx c = make_ctx(p, blk, nblk);
    // the block's W2 slice: tile t = wave + 4 j in registers (zero past the range)
    W2Resident<RT, KS> res;
    {
        const int wave = threadIdx.x >> 6;
        const int T = (c.n + 15) / 16;
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            const int t = wave + NWAVE * j;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                res.wt[j][kk] = t < T ? w2_tile_chunk<KS>(p, c.v0, c.n, t, kk) : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    RB_MARK(1023);
    if (p.S_init) {
        update(p, c, -1, rtok);
        if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
            return;
            dots_any(p, blk, nblk, -1, lbA, lbB, lbC, uA);
        if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
            return;
    }
    update(p, c, 0, rtok);
    RB_MARK(1022);
    if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
        return;
    RB_MARK(1021);
    dots_any(p, blk, nblk, 0, lbA, lbB, lbC, uA);
    RB_MARK(1020);
    if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
        return;
    RB_MARK(1019);
    for (int pos = 0; pos < p.K; ++pos) {
        // argmax words of this position carry tag gen + 1 (every block is at the same
        // generation here; consecutive positions are two generations apart)
        const uint32_t tag14 = (gen + 1) & 0x3FFFu;
        Params pl = p;
        asm volatile("" : "+s"(pl.L_base), "+s"(pl.L_final), "+s"(pl.uop), "+s"(pl.bkeys));
        RB_MARK(64 * pos);
        w2_phase<LB16, FAST, ST>(pl, c, res, pos, tag14, lbA, lbB, lbC, uA, uB, kred, lkey);
        RB_MARK(64 * pos + 1);
        if (!resolve(pl, c, pos, tag14, rtok, rred))
            return;
        RB_MARK(64 * pos + 2);
        if (pos + 1 < pl.K) {
            update(pl, c, pos + 1, rtok);
            RB_MARK(64 * pos + 3);
            if (!grid_sync(pl.bar, gen, pl.spin_limit, pl.flags))
                return;
                    RB_MARK(64 * pos + 4);
            dots_any(pl, blk, nblk, pos + 1, lbA, lbB, lbC, uA);
            RB_MARK(64 * pos + 5);
            if (!grid_sync(pl.bar, gen, pl.spin_limit, pl.flags))
                return;
                    RB_MARK(64 * pos + 6);
        }
    }
    // words of rows this launch did not draft get a tag that no later poll expects
    // (later launches poll for tags at least three generations past gen)
    for (int b = p.B + static_cast<int>(threadIdx.x); b < p.maxB; b += NT)
        st_agent_u64(&p.bkeys[static_cast<size_t>(b) * nblk + blk], static_cast<uint64_t>(gen & 0x3FFFu) << 18);
    barrier_finish(p.bar, gen);
}

}  // namespace rbk
}  // namespace DH_NS

namespace dhrb {

using namespace dh256;

int threads() { return NT; }
int r_supported() { return rbk::R; }
int max_batch() { return rbk::MAXB; }
int tiles_per_block() { return rbk::TILES; }

bool supports(int d, int h, int r, int V, int grid)
{
    // (A_H comes from the matrix-core launch, which takes d in 32-wide steps)
    if (r != rbk::R || d % 32 != 0 || h % 64 != 0 || grid < 1 || grid > MAX_GRID)
        return false;
    const long long T = (V + 15) / 16;
    if ((T + grid - 1) / grid > rbk::TILES || V >= (1 << 18))
        return false;
    // state chunks and rows per block at the largest batch
    const long long nc = static_cast<long long>(rbk::MAXB) * h / 4, per = (nc + grid - 1) / grid;
    return per <= static_cast<long long>(rbk::CPT) * NT && per * 4 / h + 2 <= rbk::ROWS;
}

template <bool LB16, bool FAST>
static const void *pick_st(bool st)
{
    return st ? reinterpret_cast<const void *>(&rbk::k_persistent_rb<LB16, FAST, true>)
              : reinterpret_cast<const void *>(&rbk::k_persistent_rb<LB16, FAST, false>);
}

const void *kernel(bool lbase_bf16, bool store_logits, int V)
{
    const bool fast = V % (lbase_bf16 ? 8 : 4) == 0;
    if (lbase_bf16)
        return fast ? pick_st<true, true>(store_logits) : pick_st<true, false>(store_logits);
    return fast ? pick_st<false, true>(store_logits) : pick_st<false, false>(store_logits);
}

}  // namespace dhrb
