// Batched drafting (9 <= B <= 256 rows, bf16 weights, r = 256, folded gate
// table) in one persistent launch that keeps each block's W2 slice in
// registers for all K positions.  The same method as every other launch
// (paper.oopus.info review, section 二, 第二步 Domino Head; news.sig.ai
// article, section "Domino怎么做"), per position p:
//   u_p = SiLU(A_H[p] + W1_S S_p),  L_p = L_base_p + W2 u_p,  t_p = argmax L_p,
//   S_{p+1} = GRU(E[x_p], S_p)   (x_p = t_p, or the teacher token)
// with the GRU input part a row of the folded table P = E W_ih^T + b_ih.
//
// One block per compute unit, eight waves (two per SIMD, up to 256 registers
// each, so one wave's epilogue and copies overlap the other's matrix-core
// products).  Block b owns a contiguous range of 16-row vocabulary tiles; wave w
// holds tiles w, w + 8, ... of it (RT per wave, 160 registers at r = 256).
// Per position the launch runs three phases.  The W2 phase starts once every
// block of the u rows has counted itself in the position's arrival counter, the
// update once every block's argmax word of its rows carries the position's tag,
// and the state dots after one grid barrier:
//   * W2 phase: for each group of 16 batch rows, D = W2_tile u^T on the matrix
//     cores (v_mfma_f32_16x16x32_bf16, A = the register tile, B = u rounded once
//     to bf16: the products are those of bf16 operands with float32 sums, u's
//     rounding moves the logits by at most a few 1e-3 at the 8B shapes), plus
//     L_base, into a running greedy argmax.  The groups' L_base slices (two
//     groups ahead) and u operands (one ahead) are copied into LDS by direct
//     global-to-LDS loads through buffer resources.  The block's key for each
//     batch row goes to a generation-tagged word bkeys[b][block];
//   * update phase: every block owns a contiguous range of the B x h state
//     entries; it reduces the argmax words of its rows (polling until all carry
//     this position's tag), writes the tokens of the rows whose first entry it
//     owns, and steps the GRU for its entries (P row, q = W_hh S + b_hh and the
//     previous state, which stays with its owner), writing S as float32 and as
//     bf16 hi/lo planes;
//   * state-dot phase: [u | q'] = S [B, h] x [W1_S; W_hh]^T on the matrix cores,
//     S as bf16 hi + lo operands.  Up to four 16-row batch tiles, block b takes
//     weight tile b and its waves split h (dots_small); more tiles run as jobs of
//     4 weight tiles x 4 batch tiles over the grid with S staged in LDS three
//     stages ahead (dots_2d).  Then u = SiLU(A_H + .) as the next W2 phase's bf16
//     operand, and q' + b_hh for the next update.
// Values that cross blocks are written with agent-scope stores, which write
// through the per-XCD L2 caches (not coherent with each other).  The argmax
// words and q, each read by one block, are read with agent-scope loads, which
// bypass them.  The S planes and the u operand, which many blocks read, have one
// slot per state (per position) in the launch and are read with ordinary,
// L2-cached copies, so the blocks of an XCD share each line: no L2 can hold a
// stale copy of such a line, since the launch starts with an agent-scope acquire
// (the L2s hold nothing written before it), nobody reads a slot before the grid
// barrier that follows its writes, and every 128-byte line of a slot is written
// by one block alone (a writer whose L2 keeps the line keeps all of it fresh).
#define DH_NT 512
#define DH_NS dhrbk
#include "dh_phases.h"
#include "dh_rbatch.h"

// Optional instrumentation: a translation unit may define RB_MARK(slot) before
// including this file to record timestamps at phase boundaries (slot = 64 *
// position + point; the prologue uses slots 1019..1023).  The default is a no-op.
#ifndef RB_MARK
#define RB_MARK(slot) ((void)(slot))
#endif
// RB_MARK_LANDED(slot): the same once the thread's memory operations in flight have
// completed (an instrumented build waits for them there; the default is a no-op)
#ifndef RB_MARK_LANDED
#define RB_MARK_LANDED(slot) ((void)(slot))
#endif
// and RB_GMARK(i) to note the time of point i (< 32) of the W2 phase's groups (after
// group g's wait: 2 g, after its products and epilogue: 2 g + 1), which RB_GFLUSH(pos,
// n) records once the phase's copies are complete
#ifndef RB_GMARK
#define RB_GMARK(i) ((void)(i))
#define RB_GFLUSH(pos, n) ((void)(pos), (void)(n))
#endif

namespace DH_NS {
namespace rbk {

constexpr int RT = 5;                // W2 tiles per wave in registers
constexpr int KS = 8;                // 32-wide steps of r
constexpr int R = 32 * KS;           // r
constexpr int TILES = NWAVE * RT;    // vocabulary tiles per block (40: 640 rows)
constexpr int LROW = TILES * 16;     // L_base values of one batch row (float32 rows in LDS)
constexpr int LROW16 = LROW + 128;   // the same for bf16 rows, padded to whole copies per wave
constexpr int LBUF = 16 * LROW * 4 / 16;  // uint4 per L_base buffer (16 rows of float32)
constexpr int UCH = KS * 64;         // uint4 of one group's u operand (bf16)
constexpr int UBUF = 1024;           // uint4 of each of the two small LDS buffers
constexpr int MAXB = 256;            // batch rows of one launch
constexpr int ROWS = 4;              // batch rows one block updates at most (B <= MAXB)
constexpr int CPT = 1;               // 4-entry state chunks per thread at most

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
    __hip_atomic_store(gmem(static_cast<uint64_t *>(p)), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// Direct global-to-LDS copy of 4 bytes per lane (lane l writes at lds + 4 l)
__device__ inline void copy_lds4(const void *g, void *lds) { __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 4, 0, 0); }

// the same through a buffer resource (16 bytes at byte offset voff + soff, voff per lane and
// soff uniform; past the records: zeros).  CP: the load's cache-policy bits
template <int CP = 0>
__device__ inline void copy_lds16_buf(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff, uint32_t soff = 0)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, static_cast<int>(soff), 0, CP);
}
// cache policy of the L_base copies: non-temporal (each value is read once), which
// measured a little faster than the default policy
constexpr int CP_STREAM = 2;

// Buffer resource over `bytes` bytes from `base` (loads past the end read 0).  Copies and
// loads through it keep the base in scalar registers and take a 32-bit per-lane offset,
// so no 64-bit address per lane is held (or spilled and reloaded between copies, which
// would make the compiler wait for every copy in flight).
__device__ inline __amdgpu_buffer_rsrc_t rsrc_of(const void *base, size_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                             static_cast<int>(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull),
                                             0x00020000);
}

// Loads through global-address-space pointers: as flat loads (through a generic
// pointer) they would also count against the LDS counter, and the next LDS read would
// wait for them.
typedef float f4n __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) f4n gf4n;
__device__ inline float4 ld_f4(const float *p)
{
    const f4n v = *reinterpret_cast<const gf4n *>(gmem(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
// entry m of b_hh (bf16 heads only), 0 without biases
__device__ inline float bias_hh_bf16(const Params &p, int m)
{
    return p.b_hh ? __uint_as_float(static_cast<uint32_t>(gmem(static_cast<const uint16_t *>(p.b_hh))[m]) << 16)
                  : 0.f;
}

__device__ inline uint64_t pack4_bf16(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return static_cast<uint64_t>(a | (b << 16)) | (static_cast<uint64_t>(c | (d << 16)) << 32);
}

// The block's share of the work, the same at every position.
struct Ctx {
    int v0, n;       // vocabulary rows [v0, v0 + n) (v0 a multiple of 16; n may be 0)
    int c0, c1;      // 4-entry chunks [c0, c1) of the flat [B, h] state index (of the flat
                     // [B, r] u index for a Markov head)
    int rb0, nrows;  // batch rows of those chunks: rb0 .. rb0 + nrows - 1
    int rc;          // chunks of one batch row (h / 4, or r / 4)
};

// Blocks that hold chunks of the split into whole 16-chunk runs of nc chunks.
__host__ __device__ inline int chunk_blocks(int nc, int nblk)
{
    const int per = ((nc + nblk - 1) / nblk + 15) & ~15;
    return (nc + per - 1) / per;
}

__device__ inline Ctx make_ctx(const Params &p, int blk, int nblk, bool markov)
{
    Ctx c;
    const long long T = (p.V + 15) / 16;
    const int ta = static_cast<int>(T * blk / nblk), tb = static_cast<int>(T * (blk + 1) / nblk);
    c.v0 = 16 * ta;
    c.n = (16 * tb < p.V ? 16 * tb : p.V) - c.v0;
    if (c.n < 0)
        c.n = 0;
    // whole 16-chunk runs (64 entries: one 128-byte line of each plane) per block
    const int e = markov ? p.r : p.h;
    const int nc = p.B * e / 4, per = ((nc + nblk - 1) / nblk + 15) & ~15;
    c.c0 = blk * per < nc ? blk * per : nc;
    c.c1 = c.c0 + per < nc ? c.c0 + per : nc;
    c.rb0 = c.c0 * 4 / e;
    c.nrows = c.c1 > c.c0 ? (c.c1 * 4 - 1) / e - c.rb0 + 1 : 0;
    c.rc = e / 4;
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
    static constexpr int ROWV = LB16 ? LROW16 : LROW;  // values of one LDS row
    static constexpr int ROWB = ROWV * EL;             // bytes of one LDS row
    static constexpr int NLD = 16 * ROWB / (64 * PIECE) / NWAVE;  // copies per thread per group
    static_assert(16 * ROWB % (64 * PIECE * NWAVE) == 0, "whole copies per wave");
    static_assert(16 * ROWB <= LBUF * 16, "group fits one buffer");
};

// Byte offsets, from the first value of the group's first batch row at the
// position, of this lane's 16-byte pieces (FAST copies): piece s = 64 i + lane of
// copy i = wave * NLD + jj lands at LDS row s / (ROWB / 16), chunk s % (ROWB / 16),
// whose value index within the block's range is (chunk ^ (row & 7)) * (16 / EL).
// Rows past B and values past the tensor lie past the buffer resource's records
// and read as 0 (their results are masked).  Pieces past the block's n values
// re-read the row's first piece (a line the copy fetches anyway), so the block
// never pulls in another block's values; those LDS entries are masked too.  The
// same at every group and position.
template <bool LB16>
struct LbOff {
    using C = LbCopy<LB16, true>;
    uint32_t off[C::NLD];
    __device__ LbOff(const Params &p, int v0, int n)
    {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
        const uint32_t rowstride = static_cast<uint32_t>(p.K) * static_cast<uint32_t>(p.V) * C::EL;
#pragma unroll
        for (int jj = 0; jj < C::NLD; ++jj) {
            const int s = 64 * (wave * C::NLD + jj) + lane;
            const int row = s / (C::ROWB / 16), ch = s % (C::ROWB / 16);
            int e = (ch ^ (row & 7)) * (16 / C::EL);
            e = e < n ? e : 0;
            off[jj] = static_cast<uint32_t>(row) * rowstride + static_cast<uint32_t>(v0 + e) * C::EL;
        }
    }
};

template <bool LB16, bool FAST>
__device__ __forceinline__ void lb_issue(const Params &p, const Ctx &c, const LbOff<LB16> &lo, int pos, int g,
                                         uint4 *buf)
{
    using C = LbCopy<LB16, FAST>;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const char *base = static_cast<const char *>(p.L_base);
    const int ngr = (p.B + 15) / 16;
    g = g < ngr ? g : ngr - 1;
    if constexpr (FAST) {
        // buffer resource from the group's first row at this position to the end of L_base
        const long long first = (static_cast<long long>(16 * g) * p.K + pos) * p.V;
        const long long left = (static_cast<long long>(p.B) * p.K * p.V - first) * C::EL;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char *>(base) + first * C::EL, 0,
            static_cast<int>(static_cast<uint32_t>(left > 0xFFFFFFFFll ? 0xFFFFFFFFll : left)), 0x00020000);
#pragma unroll
        for (int jj = 0; jj < C::NLD; ++jj)
            copy_lds16_buf<CP_STREAM>(rs, buf + 64 * (wave * C::NLD + jj), lo.off[jj]);
        return;
    }
    constexpr int VPC = 16 / C::EL;  // values per 16-byte chunk
    if constexpr (LB16 && !FAST) {
        constexpr int BATCH = 8;
#pragma unroll
        for (int j0 = 0; j0 < C::NLD; j0 += BATCH) {
            uint16_t v[BATCH];
#pragma unroll
            for (int jj = 0; jj < BATCH; ++jj) {
                const int s = 64 * (wave * C::NLD + j0 + jj) + lane;
                const int row = s / C::ROWV, pr = s % C::ROWV;
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
        constexpr int PPC = 16 / C::PIECE;        // pieces per chunk
        int e = ((pr / PPC) ^ (row & 7)) * VPC + pr % PPC;  // value index within the block's range
        e = e < c.n ? e : 0;
        const int b = 16 * g + row < p.B ? 16 * g + row : p.B - 1;
        const char *src = base + ((static_cast<size_t>(b) * p.K + pos) * p.V + c.v0 + e) * C::EL;
        copy_lds4(src, reinterpret_cast<char *>(buf) + i * 64 * C::PIECE);
    }
}

// u operand of group g (8 KB, the layout of p.uop) into an LDS buffer: one copy per thread.
__device__ __forceinline__ void u_issue(const Params &p, int pos, int g, uint4 *buf)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int ngr = (p.B + 15) / 16;
    g = g < ngr ? g : ngr - 1;
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(p.uop + (static_cast<size_t>(pos) * p.rb_ngr + g) * UCH, UCH * 16);
#pragma unroll
    for (int jj = 0; jj < UCH / 64 / NWAVE; ++jj) {
        const int i = wave * (UCH / 64 / NWAVE) + jj;
        copy_lds16_buf(rs, buf + 64 * i, static_cast<uint32_t>((64 * i + lane) * 16));
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
                                                         (row * (LROW16 * 2 / 16) + chunk) * 16 + (k & 1) * 8);
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.y << 16),
                           __uint_as_float(v.y & 0xFFFF0000u));
    } else {
        const uint4 v = buf[row * (LROW / 4) + ((4 * t + k) ^ (row & 7))];
        return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
    }
}

// Products and epilogue of group g for this wave: result lane l holds vocabulary
// rows 16 t + 4 (l / 16) + i (i = 0..3) of tile t = wave + NWAVE j for batch row
// 16 g + l % 16.  The accumulators start at the lane's L_base values, so the products
// add onto them.  The lane keeps the first of its largest values (a NaN above every
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
    for (int j = 0; j < RT; ++j) {
        const float4 lb = lb_read<LB16>(L, row, wave + NWAVE * j, k);
        acc[j] = f32x4_t{lb.x, lb.y, lb.z, lb.w};
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const uint4 uh = U[kk * 64 + lane];
#pragma unroll
        for (int j = 0; j < RT; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, res.wt[j][kk]),
                                                             __builtin_bit_cast(bf16x8_t, uh), acc[j], 0, 0, 0);
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
        // tiles wholly inside the block's range skip the per-value bound (uniform)
        if (16 * (t + 1) <= c.n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = acc[j][i];
                if constexpr (ST) {
                    if (b < p.B)
                        lf[16 * t + 4 * k + i] = v;
                }
                const bool take = !(v <= best) & (best == best);
                best = take ? v : best;
                bpos = take ? 4 * j + i : bpos;
            }
        } else if (16 * t < c.n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = acc[j][i];
                const int vr = 16 * t + 4 * k + i;
                const bool ok = vr < c.n;
                if constexpr (ST) {
                    if (ok && b < p.B)
                        lf[vr] = v;
                }
                const bool take = !(v <= best) & (best == best) & ok;
                best = take ? v : best;
                bpos = take ? 4 * j + i : bpos;
            }
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

// Copies of the first two L_base groups of position pos (they depend on nothing
// computed in the launch, so they go out before the wait for the u operand).
template <bool LB16, bool FAST>
__device__ __forceinline__ void w2_prefetch(const Params &p, const Ctx &c, int pos, uint4 *lbA, uint4 *lbB)
{
    const LbOff<LB16> lo(p, c.v0, c.n);
    lb_issue<LB16, FAST>(p, c, lo, pos, 0, lbA);
    lb_issue<LB16, FAST>(p, c, lo, pos, 1, lbB);
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
    const LbOff<LB16> lo(p, c.v0, c.n);
    // block key of group gp from the waves' keys (after a barrier)
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
    // flight: they were issued last; group 0's u copy was issued last, so it waits for
    // all), meet the other waves, fold the previous group's keys, start the copies of
    // u(g + 1) and L_base(g + 2), then the products
    auto iter = [&](int g, const uint4 *Lc, uint4 *Ln2, const uint4 *Uc, uint4 *Un) {
        if (g == 0)
            wait_vm<0>();
        else
            wait_vm<C::NLD>();
        bare_barrier();
        RB_GMARK(2 * g);
        if (g >= 1)
            fold(g - 1);
        u_issue(p, pos, g + 1, Un);
        lb_issue<LB16, FAST>(p, c, lo, pos, g + 2, Ln2);
        w2_group<LB16, ST>(p, c, res, pos, g, Lc, Uc, kred + (g & 1) * NWAVE * 16);
        RB_GMARK(2 * g + 1);
    };
    // L_base groups 0 and 1 were issued by w2_prefetch
    u_issue(p, pos, 0, uA);
    // group g uses L_base buffer g % 3 and u buffer g % 2
#pragma unroll 1
    for (int g0 = 0; g0 < ngr; g0 += 6) {
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
    // the state products (q) this block stored before are complete before its keys,
    // which the update of the next position waits for
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int b = threadIdx.x; b < p.B; b += NT) {
        const uint64_t m = lkey[b];
        st_agent_u64(&p.bkeys[static_cast<size_t>(b) * gridDim.x + blockIdx.x],
                     (m & (KEY_ORD_MASK | KEY_IDX_MASK)) | (static_cast<uint64_t>(tag14) << 18));
    }
    // (an instrumented build writes the groups' times after the keys, so that they do not
    // delay the key words that thread 0's wave stores)
    RB_GFLUSH(pos, 2 * ngr);
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
    RB_MARK(64 * pos + 44);  // every argmax word of the block's rows read
    if (failed) {
        if (threadIdx.x == 0)
            __hip_atomic_fetch_or(gmem(p.flags), 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    if (static_cast<int>(threadIdx.x) < c.nrows) {
        uint64_t m = 0;
        for (int w = 0; w < NWAVE; ++w)
            m = max_u64(m, rred[w * ROWS + threadIdx.x]);
        const int tok = m ? static_cast<int>(KEY_IDX_MASK - (m & KEY_IDX_MASK)) : 0;
        rtok[threadIdx.x] = tok;
        const int b = c.rb0 + threadIdx.x;
        if (b * c.rc >= c.c0)  // this block owns the row's first entry
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
    uint16_t *plane_hi = p.rb_planes + static_cast<size_t>(q + 1) * 2 * p.rb_bmax * p.rb_ldp;
    uint16_t *plane_lo = plane_hi + static_cast<size_t>(p.rb_bmax) * p.rb_ldp;
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
            const float4 gr = ld_f4(prow);
            const float4 gz = ld_f4(prow + h);
            const float4 gn = ld_f4(prow + 2 * h);
            float4 qr, qz, qn;
            if (q == 0 && !p.S_init) {
                // W_hh S_init + b_hh with S_init = 0 is b_hh itself
                qr = make_float4(bias_hh_bf16(p, j), bias_hh_bf16(p, j + 1), bias_hh_bf16(p, j + 2), bias_hh_bf16(p, j + 3));
                qz = make_float4(bias_hh_bf16(p, h + j), bias_hh_bf16(p, h + j + 1), bias_hh_bf16(p, h + j + 2), bias_hh_bf16(p, h + j + 3));
                qn = make_float4(bias_hh_bf16(p, 2 * h + j), bias_hh_bf16(p, 2 * h + j + 1), bias_hh_bf16(p, 2 * h + j + 2),
                                 bias_hh_bf16(p, 2 * h + j + 3));
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
                sp = ld_f4(p.S_buf + static_cast<size_t>(b) * h + j);
            if (u == 0 && q > 0)
                RB_MARK_LANDED(64 * (q - 1) + 46);  // the gate inputs of the first entries landed
            const float g3[3][4] = {{gr.x, gr.y, gr.z, gr.w}, {gz.x, gz.y, gz.z, gz.w}, {gn.x, gn.y, gn.z, gn.w}};
            const float q3[3][4] = {{qr.x, qr.y, qr.z, qr.w}, {qz.x, qz.y, qz.z, qz.w}, {qn.x, qn.y, qn.z, qn.w}};
            const float s4[4] = {sp.x, sp.y, sp.z, sp.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the cell of gate_update
                const float rg = sigmoidf_(g3[0][i] + q3[0][i]);
                const float zg = sigmoidf_(g3[1][i] + q3[1][i]);
                const float ng = tanhf_(g3[2][i] + rg * q3[2][i]);
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
        const size_t o = static_cast<size_t>(b) * p.rb_ldp + j;
        st_agent_u64(plane_hi + o, pack4_bf16(hi[0], hi[1], hi[2], hi[3]));
        st_agent_u64(plane_lo + o, pack4_bf16(lo[0], lo[1], lo[2], lo[3]));
    }
}

// ---- state-dot phase ------------------------------------------------------------------
// Block b < (r + 3h) / 16 owns weight tile b: rows 16 b .. 16 b + 15 of the packed state
// rows wst = [W1_S; W_hh]; wave w takes the 32-wide steps KSW w .. KSW w + KSW - 1 of the
// h reduction (A operands loaded with the first round's copies).  Per state S_q the
// block multiplies its tile with every batch row: in rounds of two 16-row batch tiles,
// each wave copies the S hi and lo rows of its own steps into its own LDS region
// (16 KB), waits for its own copies and multiplies; the eight partial
// sums of each tile are added through LDS in wave order, and waves 0 and 1 finish the
// two tiles: u = SiLU(A_H + .) as the W2 operand of position q (rows m < r) or
// q' = . + b_hh for the next update.  The blocks of the u rows then count themselves
// in rb_ucnt[q], which the W2 phase waits for.  q = -1: only the W_hh rows (q of S_init).
constexpr int KSW = 4;  // 32-wide steps of h per wave (h <= 32 KSW NWAVE = 1024)

struct DotW {
    uint4 w[KSW];
};

__device__ __forceinline__ void dots_small(const Params &p, int blk, int q, uint4 *lbA, uint4 *lbB, uint4 *lbC,
                                           uint4 *uA, uint4 *uB)
{
    const int lane = threadIdx.x & 63, row = lane & 15, k = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int h = p.h, r = p.r, h3 = 3 * h;
    const int nwt = (r + h3) / 16, nks = h / 32, nbt = (p.B + 15) / 16;
    const int m = 16 * blk + 4 * k;  // result rows of this lane: m .. m + 3
    const bool urows = 16 * blk < r;
    if (blk >= nwt || (q < 0 && urows))
        return;
    // the state slot's hi and lo planes through one buffer resource
    const uint32_t plb = static_cast<uint32_t>(p.rb_bmax * p.rb_ldp * 2);  // bytes of one plane
    const __amdgpu_buffer_rsrc_t prs =
        rsrc_of(p.rb_planes + static_cast<size_t>(q + 1) * 2 * p.rb_bmax * p.rb_ldp, 2 * static_cast<size_t>(plb));
    const __amdgpu_buffer_rsrc_t wrs = rsrc_of(p.wst, static_cast<size_t>(r + h3) * p.ldw * 2);
    // this wave's LDS region: 2 tiles x hi/lo x KSW steps of 1 KB
    uint4 *mine = wave < 2 ? lbA + wave * 1024 : wave < 4 ? lbB + (wave - 2) * 1024
                : wave < 6 ? lbC + (wave - 4) * 1024 : wave == 6 ? uA : uB;
    f32x4_t *red = reinterpret_cast<f32x4_t *>(uB);  // [2 tiles][NWAVE][64] partial sums
    DotW dw;
    for (int bt0 = 0; bt0 < nbt; bt0 += 2) {
        const int ntl = nbt - bt0 < 2 ? nbt - bt0 : 2;
        // every copy is issued (rows past B repeat row B - 1, steps past h repeat step
        // 0; those results are not used): a copy in a branch would make the compiler
        // wait for all copies in flight at the branch's end
#pragma unroll
        for (int tl = 0; tl < 2; ++tl) {
            int b = 16 * (bt0 + tl) + row;
            b = b < p.B ? b : p.B - 1;
            // one per-lane offset per tile; the plane and step go in the uniform offset
            const uint32_t lrow = static_cast<uint32_t>((b * p.rb_ldp + 8 * k) * 2);
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                for (int i = 0; i < KSW; ++i) {
                    const int st = wave * KSW + i < nks ? wave * KSW + i : 0;
                    copy_lds16_buf(prs, mine + ((tl * 2 + hl) * KSW + i) * 64, lrow, hl * plb + st * 64);
                }
        }
        // this wave's steps of the block's weight tile (steps past h repeat step 0,
        // unused), and the A_H entries of the round's u rows (clamped when unused)
        if (bt0 == 0) {
            const uint32_t wrow = static_cast<uint32_t>(((16 * blk + row) * p.ldw + 8 * k) * 2);
#pragma unroll
            for (int i = 0; i < KSW; ++i) {
                const int st = wave * KSW + i < nks ? wave * KSW + i : 0;
                dw.w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wrow, st * 64, 0));
            }
        }
        float4 ah = make_float4(0.f, 0.f, 0.f, 0.f);
        {
            int b = 16 * (bt0 + (wave & 1)) + row;
            b = b < p.B ? b : p.B - 1;
            ah = ld_f4(p.A_H + (static_cast<size_t>(b) * p.K + (q > 0 ? q : 0)) * r +
                                                   (urows ? m : 0));
        }
        if (bt0 == 0)
            RB_MARK(64 * (q > 0 ? q : 0) + 40);
        wait_vm<0>();
        if (bt0 == 0)
            RB_MARK(64 * (q > 0 ? q : 0) + 41);
        f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int tl = 0; tl < 2; ++tl) {
            if (tl >= ntl)
                break;
#pragma unroll
            for (int i = 0; i < KSW; ++i) {
                if (wave * KSW + i < nks) {
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl)
                        acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, dw.w[i]),
                            __builtin_bit_cast(bf16x8_t, mine[((tl * 2 + hl) * KSW + i) * 64 + lane]), acc[tl], 0, 0,
                            0);
                }
            }
        }
        __syncthreads();  // every wave's region read (the partial sums go where wave 7's was)
        if (bt0 == 0)
            RB_MARK(64 * (q > 0 ? q : 0) + 42);
#pragma unroll
        for (int tl = 0; tl < 2; ++tl)
            red[(tl * NWAVE + wave) * 64 + lane] = acc[tl];
        __syncthreads();
        if (wave < ntl) {
            const int tl = wave;
            f32x4_t sum = red[(tl * NWAVE) * 64 + lane];
#pragma unroll
            for (int w = 1; w < NWAVE; ++w) {
                const f32x4_t o = red[(tl * NWAVE + w) * 64 + lane];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sum[i] += o[i];
            }
            // lane holds weight rows m .. m + 3 of batch row b
            const int b = 16 * (bt0 + tl) + row;
            if (b < p.B) {
                if (urows) {
                    const float a4[4] = {ah.x + sum[0], ah.y + sum[1], ah.z + sum[2], ah.w + sum[3]};
                    float u4[4];
                    uint32_t hi[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        u4[i] = a4[i] * sigmoidf_(a4[i]);
                        hi[i] = bf16_rne_bits(u4[i]);
                    }
                    if (p.u_out)
                        *reinterpret_cast<float4 *>(p.u_out + (static_cast<size_t>(b) * p.K + q) * r + m) =
                            make_float4(u4[0], u4[1], u4[2], u4[3]);
                    // operand chunk of (batch row b, r offsets 8 (m / 8) .. + 8): group b / 16,
                    // step m / 32, lane b % 16 + 16 ((m % 32) / 8); these four values are its
                    // half (m % 8) / 4
                    const size_t ch = ((static_cast<size_t>(q) * p.rb_ngr + (b >> 4)) * KS + (m >> 5)) * 64 +
                                      (b & 15) + 16 * ((m & 31) >> 3);
                    char *dst = reinterpret_cast<char *>(p.uop + ch) + (m & 7) * 2;
                    st_agent_u64(dst, pack4_bf16(hi[0], hi[1], hi[2], hi[3]));
                } else {
                    const int mq = m - r;
                    const float4 v = make_float4(sum[0] + bias_hh_bf16(p, mq), sum[1] + bias_hh_bf16(p, mq + 1),
                                                 sum[2] + bias_hh_bf16(p, mq + 2), sum[3] + bias_hh_bf16(p, mq + 3));
                    st_agent_f4(q_slot(p, q + 1) + static_cast<size_t>(b) * h3 + mq, v);
                }
            }
        }
        __syncthreads();  // regions and partial sums free for the next round
        if (bt0 == 0)
            RB_MARK(64 * (q > 0 ? q : 0) + 43);
    }
    if (urows && q >= 0) {
        // this block's share of u_q is written: count it
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(gmem(&p.rb_ucnt[q]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Larger batches: a job is 4 weight tiles x BJ batch tiles (2-D tiles: each block reads
// a slice of S and a slice of the weights instead of all of S).  Waves w and w + 4 take
// weight tile w % 4 (A operand from L2) and the first or second 32-wide step of each
// 64-wide stage of the h reduction; the B operand (S hi and lo rows of the BJ batch
// tiles) is staged in LDS: a stage's BJ * 4 blocks of 1 KB are copied three stages
// ahead into a ring of four buffers, each wave waiting for its own copies and meeting
// the others at a bare barrier.  Every copy and load is issued on every step (stages
// past the last repeat it), so the wait counts are the same on every path.  At the end
// waves 4..7 hand their partial sums to waves 0..3 through LDS.  Jobs of the u rows
// count themselves in rb_ucnt[q].
constexpr int DOTS_BJ = 4;
__host__ __device__ inline bool dots_tiled(int B) { return (B + 15) / 16 > 4; }
__host__ __device__ inline int u_producers(int B, int r)
{
    return dots_tiled(B) ? (r / 64) * (((B + 15) / 16 + DOTS_BJ - 1) / DOTS_BJ) : r / 16;
}

__device__ __forceinline__ void dots_2d(const Params &p, int blk, int nblk, int q, uint4 *ring0, uint4 *ring1,
                                        uint4 *ring2, uint4 *ring3)
{
    constexpr int BJ = DOTS_BJ;
    const int lane = threadIdx.x & 63, row = lane & 15, k = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int tw = wave & 3, ks = wave >> 2;
    const int h = p.h, r = p.r, h3 = 3 * h;
    const int nwg = (r + h3) / 64;
    const int nbt = (p.B + 15) / 16, nbj = (nbt + BJ - 1) / BJ;
    const int NS = h / 64;
    const uint32_t plb = static_cast<uint32_t>(p.rb_bmax * p.rb_ldp * 2);  // bytes of one plane
    const __amdgpu_buffer_rsrc_t prs =
        rsrc_of(p.rb_planes + static_cast<size_t>(q + 1) * 2 * p.rb_bmax * p.rb_ldp, 2 * static_cast<size_t>(plb));
    const __amdgpu_buffer_rsrc_t wrs = rsrc_of(p.wst, static_cast<size_t>(r + h3) * p.ldw * 2);
    constexpr int NB1 = BJ * 4;                      // 1 KB operand blocks per stage: (bt, hi/lo, step)
    constexpr int PER = (NB1 + NWAVE - 1) / NWAVE;   // copies per wave per stage
    static_assert(NWAVE * PER <= 16, "copies fit one 16 KB ring buffer");
    f32x4_t *xch = reinterpret_cast<f32x4_t *>(ring0);
    for (int job = blk; job < nwg * nbj; job += nblk) {
        const int wg = job / nbj, bj = job % nbj;
        const int wt = wg * 4 + tw;  // this wave's weight tile
        const bool urows = wg * 64 < r;
        const bool active = !(q < 0 && urows);
        uint32_t src[PER], srcs[PER];  // per-lane and uniform byte offsets in the planes' resource
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int ib = (wave * PER + x) % NB1, bt = ib >> 2, hl = (ib >> 1) & 1, st = ib & 1;
            int b = (bj * BJ + bt) * 16 + row;
            b = b < p.B ? b : p.B - 1;
            src[x] = static_cast<uint32_t>((b * p.rb_ldp + 8 * k) * 2);
            srcs[x] = hl * plb + 64 * st;
        }
        const uint32_t wrow = static_cast<uint32_t>(((wt * 16 + row) * p.ldw + 32 * ks + 8 * k) * 2);
        uint4 wa[4];
        // the jobs of one batch job read the same S slices: each weight group starts
        // the h reduction at its own stage, so concurrent jobs request different lines
        const int srot = wg % NS;
        auto issue = [&](int s, uint4 *ring, uint4 &w) {
            s = s < NS ? s : NS - 1;
            s = s + srot < NS ? s + srot : s + srot - NS;
#pragma unroll
            for (int x = 0; x < PER; ++x)
                copy_lds16_buf(prs, ring + (wave * PER + x) * 64, src[x], srcs[x] + 128 * s);
            w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wrow, 128 * s, 0));
        };
        f32x4_t acc[BJ];
#pragma unroll
        for (int bt = 0; bt < BJ; ++bt)
            acc[bt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](const uint4 *ring, const uint4 &w) {
#pragma unroll
            for (int bt = 0; bt < BJ; ++bt)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
                    acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, w),
                        __builtin_bit_cast(bf16x8_t, ring[((bt * 2 + hl) * 2 + ks) * 64 + lane]), acc[bt], 0, 0, 0);
        };
        auto step = [&](int s, const uint4 *cur, uint4 *nxt, const uint4 &wc, uint4 &wn) {
            wait_vm<2 * (PER + 1)>();
            bare_barrier();
            issue(s + 3, nxt, wn);
            if (active && s < NS)
                compute(cur, wc);
        };
        const bool first = job == blk;
        issue(0, ring0, wa[0]);
        issue(1, ring1, wa[1]);
        issue(2, ring2, wa[2]);
        if (first)
            RB_MARK(64 * (q > 0 ? q : 0) + 40);
#pragma unroll 1
        for (int s = 0; s < NS; s += 4) {
            step(s, ring0, ring3, wa[0], wa[3]);
            if (first && s == 0)
                RB_MARK(64 * (q > 0 ? q : 0) + 41);
            step(s + 1, ring1, ring0, wa[1], wa[0]);
            step(s + 2, ring2, ring1, wa[2], wa[1]);
            step(s + 3, ring3, ring2, wa[3], wa[2]);
        }
        wait_vm<0>();
        bare_barrier();
        if (first)
            RB_MARK(64 * (q > 0 ? q : 0) + 42);
        if (ks == 1) {
#pragma unroll
            for (int bt = 0; bt < BJ; ++bt)
                xch[(tw * BJ + bt) * 64 + lane] = acc[bt];
        }
        __syncthreads();
        if (ks == 0 && active) {
#pragma unroll
            for (int bt = 0; bt < BJ; ++bt) {
                const f32x4_t o = xch[(tw * BJ + bt) * 64 + lane];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[bt][i] += o[i];
            }
            const int m = 16 * wt + 4 * k;
#pragma unroll
            for (int bt = 0; bt < BJ; ++bt) {
                const int b = (bj * BJ + bt) * 16 + row;
                if (b >= p.B)
                    continue;
                if (m < r) {
                    const float4 ah =
                        ld_f4(p.A_H + (static_cast<size_t>(b) * p.K + q) * r + m);
                    const float a4[4] = {ah.x + acc[bt][0], ah.y + acc[bt][1], ah.z + acc[bt][2], ah.w + acc[bt][3]};
                    float u4[4];
                    uint32_t hi[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        u4[i] = a4[i] * sigmoidf_(a4[i]);
                        hi[i] = bf16_rne_bits(u4[i]);
                    }
                    if (p.u_out)
                        *reinterpret_cast<float4 *>(p.u_out + (static_cast<size_t>(b) * p.K + q) * r + m) =
                            make_float4(u4[0], u4[1], u4[2], u4[3]);
                    const size_t ch = ((static_cast<size_t>(q) * p.rb_ngr + (b >> 4)) * KS + (m >> 5)) * 64 +
                                      (b & 15) + 16 * ((m & 31) >> 3);
                    char *dst = reinterpret_cast<char *>(p.uop + ch) + (m & 7) * 2;
                    st_agent_u64(dst, pack4_bf16(hi[0], hi[1], hi[2], hi[3]));
                } else {
                    const int mq = m - r;
                    const float4 v = make_float4(acc[bt][0] + bias_hh_bf16(p, mq), acc[bt][1] + bias_hh_bf16(p, mq + 1),
                                                 acc[bt][2] + bias_hh_bf16(p, mq + 2), acc[bt][3] + bias_hh_bf16(p, mq + 3));
                    st_agent_f4(q_slot(p, q + 1) + static_cast<size_t>(b) * h3 + mq, v);
                }
            }
        }
        if (urows && q >= 0) {
            // this job's share of u_q is written: count it
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(gmem(&p.rb_ucnt[q]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // the exchange buffer is the first ring buffer of the next job
        __syncthreads();
        if (first)
            RB_MARK(64 * (q > 0 ? q : 0) + 43);
    }
}

__device__ __forceinline__ void dots(const Params &p, int blk, int nblk, int q, uint4 *lbA, uint4 *lbB, uint4 *lbC,
                                     uint4 *uA, uint4 *uB)
{
    if (dots_tiled(p.B))
        dots_2d(p, blk, nblk, q, lbA, lbB, lbC, uA);
    else
        dots_small(p, blk, q, lbA, lbB, lbC, uA, uB);
}

// Markov head: u_q = SiLU(A_H[q] + M[x_q]) (the table row of the token before position
// q) for the block's chunks of the flat [B, r] index, as the W2 phase's bf16 operand
// (and u_out), then the block counts itself in the position's arrival counter.  rtok:
// the tokens of position q - 1 of the block's rows.
__device__ __forceinline__ void markov_phase(const Params &p, const Ctx &c, int q, const int *rtok)
{
    const int r = p.r;
    for (int cc = c.c0 + static_cast<int>(threadIdx.x); cc < c.c1; cc += NT) {
        const int b = cc / c.rc, m = (cc % c.rc) * 4;
        int x;
        if (q == 0)
            x = p.last_tok[b];
        else if (p.teacher)
            x = p.teacher[static_cast<size_t>(b) * p.K + (q - 1)];
        else
            x = rtok[b - c.rb0];
        x = tok_ok(x, p.V) ? x : 0;
        const float4 ah = ld_f4(p.A_H + (static_cast<size_t>(b) * p.K + q) * r + m);
        const float4 mr = ld_f4(p.M + static_cast<size_t>(x) * r + m);
        const float a4[4] = {ah.x + mr.x, ah.y + mr.y, ah.z + mr.z, ah.w + mr.w};
        float u4[4];
        uint32_t hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u4[i] = a4[i] * sigmoidf_(a4[i]);
            hi[i] = bf16_rne_bits(u4[i]);
        }
        if (p.u_out)
            *reinterpret_cast<float4 *>(p.u_out + (static_cast<size_t>(b) * p.K + q) * r + m) =
                make_float4(u4[0], u4[1], u4[2], u4[3]);
        const size_t ch = ((static_cast<size_t>(q) * p.rb_ngr + (b >> 4)) * KS + (m >> 5)) * 64 + (b & 15) +
                          16 * ((m & 31) >> 3);
        st_agent_u64(reinterpret_cast<char *>(p.uop + ch) + (m & 7) * 2, pack4_bf16(hi[0], hi[1], hi[2], hi[3]));
    }
    if (c.c1 > c.c0) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(gmem(&p.rb_ucnt[q]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The W2 phase of position q waits until every block of the u rows has written its
// share of u_q.  False on a timeout.
template <bool MK>
__device__ __forceinline__ bool wait_u(const Params &p, int q)
{
    int ok = 1;
    if (threadIdx.x == 0) {
        const unsigned want =
            static_cast<unsigned>(MK ? chunk_blocks(p.B * p.r / 4, gridDim.x) : u_producers(p.B, p.r));
        unsigned spins = 0;
        while (__hip_atomic_load(gmem(&p.rb_ucnt[q]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
            if (++spins > p.spin_limit) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    if (block_failed(ok)) {
        if (threadIdx.x == 0)
            __hip_atomic_fetch_or(gmem(p.flags), 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    return true;
}

template <bool LB16, bool FAST, bool ST, bool MK>
__global__ __launch_bounds__(NT) void k_persistent_rb(Params p)
{
    __shared__ uint4 lbA[LBUF], lbB[LBUF], lbC[LBUF];
    __shared__ uint4 uA[UBUF], uB[UBUF];
    __shared__ uint64_t kred[2 * NWAVE * 16];
    __shared__ uint64_t lkey[MAXB];
    __shared__ uint64_t rred[NWAVE * ROWS];
    __shared__ int rtok[ROWS];
    const int blk = blockIdx.x, nblk = gridDim.x;
    RB_MARK(1019);
    // nothing in this XCD's L2 predates the launch (see the header comment)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    unsigned gen = barrier_gen_init(p.bar);
    block_fail_init();
    if (blk == 0) {
        for (int b = threadIdx.x; b < p.B; b += NT)
            if (row_bad(p, b))
                __hip_atomic_fetch_or(gmem(p.flags), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the u counters of this launch start at 0 (the first increment follows a barrier)
        if (threadIdx.x < static_cast<unsigned>(p.K))
            __hip_atomic_store(gmem(&p.rb_ucnt[threadIdx.x]), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const Ctx c = make_ctx(p, blk, nblk, MK);
    // the block's W2 slice: tile t = wave + NWAVE j in registers (zero past the range),
    // and its tile of the state rows
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
    if constexpr (MK) {
        // Markov head: no state.  One grid barrier (the u counters are zero before any
        // block counts itself), then u_0 from the last tokens
        if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
            return;
        markov_phase(p, c, 0, rtok);
    } else {
        if (p.S_init) {
            // q = W_hh S_init + b_hh for the anchor step
            update(p, c, -1, rtok);
            if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
                return;
            dots(p, blk, nblk, -1, lbA, lbB, lbC, uA, uB);
            if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
                return;
        }
        update(p, c, 0, rtok);
        RB_MARK(1022);
        if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
            return;
        RB_MARK(1021);
        dots(p, blk, nblk, 0, lbA, lbB, lbC, uA, uB);
    }
    RB_MARK(1020);
    // per position: W2 phase (after the blocks of the u rows have written u), argmax
    // words, update of the block's state entries, one grid barrier, state products
    for (int pos = 0; pos < p.K; ++pos) {
        // argmax words of this position carry tag gen + 1 (every block is at the same
        // generation here; consecutive positions are a generation apart)
        const uint32_t tag14 = (gen + 1) & 0x3FFFu;
        // the pointers pass through an opaque copy each position, so the per-thread
        // addresses derived from them are recomputed in each phase instead of being
        // hoisted out of the loop into (spilled) registers
        Params pl = p;
        asm volatile("" : "+s"(pl.L_base), "+s"(pl.L_final), "+s"(pl.uop), "+s"(pl.bkeys), "+s"(pl.rb_planes),
                          "+s"(pl.wst), "+s"(pl.A_H), "+s"(pl.q_buf), "+s"(pl.S_buf), "+s"(pl.P), "+s"(pl.tokens));
        asm volatile("" : "+s"(pl.S_out), "+s"(pl.u_out), "+s"(pl.rb_ucnt), "+s"(pl.teacher), "+s"(pl.last_tok),
                          "+s"(pl.b_hh), "+s"(pl.flags), "+s"(pl.bar));
        w2_prefetch<LB16, FAST>(pl, c, pos, lbA, lbB);
        RB_MARK(64 * pos);
        if (!wait_u<MK>(pl, pos))
            return;
        RB_MARK(64 * pos + 7);
        w2_phase<LB16, FAST, ST>(pl, c, res, pos, tag14, lbA, lbB, lbC, uA, uB, kred, lkey);
        RB_MARK(64 * pos + 1);
        if (!resolve(pl, c, pos, tag14, rtok, rred))
            return;
        RB_MARK(64 * pos + 2);
        if constexpr (MK) {
            // Markov head: u of the next position from the tokens just resolved.  No grid
            // barrier: a block polls argmax words only for rows whose u it forms, and
            // no block writes the next position's words before every such block has
            // counted its u; generations still advance one per position
            if (pos + 1 < pl.K) {
                markov_phase(pl, c, pos + 1, rtok);
                ++gen;
            }
        } else if (pos + 1 < pl.K) {
            update(pl, c, pos + 1, rtok);
            RB_MARK(64 * pos + 3);
            if (!grid_sync(pl.bar, gen, pl.spin_limit, pl.flags))
                return;
            RB_MARK(64 * pos + 4);
            dots(pl, blk, nblk, pos + 1, lbA, lbB, lbC, uA, uB);
            RB_MARK(64 * pos + 5);
        }
    }
    // words of rows this launch did not draft get a tag that no later poll expects
    // (later launches poll for tags at least two generations past gen)
    for (int b = p.B + static_cast<int>(threadIdx.x); b < p.maxB; b += NT)
        st_agent_u64(&p.bkeys[static_cast<size_t>(b) * nblk + blk], static_cast<uint64_t>(gen & 0x3FFFu) << 18);
    barrier_finish(p.bar, gen);
}

}  // namespace rbk
}  // namespace DH_NS

namespace dhrb {

using namespace dhrbk;

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
    // state chunks and rows per block at the largest batch, in whole 16-chunk runs as the
    // kernel splits them
    const long long nc = static_cast<long long>(rbk::MAXB) * h / 4, per = ((nc + grid - 1) / grid + 15) & ~15ll;
    // (a Markov head splits the u entries the same way: r = 256 needs no more rows)
    const long long ncu = static_cast<long long>(rbk::MAXB) * r / 4, peru = ((ncu + grid - 1) / grid + 15) & ~15ll;
    return per <= static_cast<long long>(rbk::CPT) * NT && per * 4 / h + 2 <= rbk::ROWS &&
           peru <= static_cast<long long>(rbk::CPT) * NT && peru * 4 / r + 2 <= rbk::ROWS;
}

template <bool LB16, bool FAST, bool ST>
static const void *pick_mk(bool mk)
{
    return mk ? reinterpret_cast<const void *>(&rbk::k_persistent_rb<LB16, FAST, ST, true>)
              : reinterpret_cast<const void *>(&rbk::k_persistent_rb<LB16, FAST, ST, false>);
}

template <bool LB16, bool FAST>
static const void *pick_st(bool st, bool mk)
{
    return st ? pick_mk<LB16, FAST, true>(mk) : pick_mk<LB16, FAST, false>(mk);
}

const void *kernel(bool lbase_bf16, bool store_logits, int V, bool markov)
{
    const bool fast = V % (lbase_bf16 ? 8 : 4) == 0;
    if (lbase_bf16)
        return fast ? pick_st<true, true>(store_logits, markov) : pick_st<true, false>(store_logits, markov);
    return fast ? pick_st<false, true>(store_logits, markov) : pick_st<false, false>(store_logits, markov);
}

}  // namespace dhrb
