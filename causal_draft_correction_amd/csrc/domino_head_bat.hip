// Batched W2 phase on the matrix cores (bf16 W2, r = 32 * KS), for the
// stepwise launches at B > 8: per position p,
//   L_p[b][v] = L_base[b][p][v] + sum_k W2[v][k] u_p[b][k],  t_p[b] = argmax_v L_p[b][v]
// (paper.oopus.info review, section 二, 第二步 Domino Head: low-rank logit
// correction added to the base logits; news.sig.ai article, section
// "Domino怎么做": greedy decoding).  Built for 256-thread blocks.
#define DH_NT 256
#define DH_NS dh256
#include "dh_phases.h"
#include "dh_batched.h"

namespace DH_NS {

// Work split.  A block of NTH threads takes a batch tile of up to 128 rows (bt)
// and a contiguous vocabulary range (vb of nvb).  Its waves take 16-row batch
// groups of the tile (ng groups) and, when the tile has fewer groups than
// waves, split each vocabulary chunk's 16-row tiles between nvs = waves / ng
// wave sets (VTG tiles each).  A wave keeps its batch rows of u in registers
// as AT matrix-core A operands.  U1 (drafts of more than 8 rows): u rounded once
// to bf16, one A tile of 16 batch rows, each result lane holding four batch rows.
// Otherwise (the rows of at most 8-row drafts, which must equal the resident
// kernel's logits bit for bit): A tile a holds batch rows a*8 .. a*8+7, row j's
// bf16 hi part in operand row 2j and its lo part (u - hi) in row 2j+1, so each
// result lane holds the hi and lo results of two batch rows side by side.
// Chunks of W2 are staged through LDS in the B-operand layout ([tile][step]
// [lane], 16 bytes each), double buffered, with the registers of the chunk after
// next loaded while the current chunk is multiplied (v_mfma_f32_16x16x32_bf16,
// D = A W2_tile^T).  The epilogue of a chunk runs one step late, beside the next
// chunk's products: it adds each batch row's hi and lo results (hi + lo, the
// resident kernel's order), adds L_base (loaded a step ahead, through the
// cache), stores L_final if requested and folds the greedy argmax into a running
// best per lane.  At the end the 16 lanes of a batch row reduce it and one lane
// folds it into the partial key slot of group blockIdx % NG.  512 threads with
// AT = 2: two waves per SIMD, up to 128 rows per tile.
constexpr int XCDS = 8;   // accelerator dies (XCDs) of the MI355X, each with its own L2

template <int KS, int VTG, int NVS, int AT, int NTH, bool LB16, bool ST, bool U1>
__global__ __launch_bounds__(NTH) void k_w2_mfma(Params p, int pos, int ng_arg)
{
    static_assert(U1 ? AT == 1 : (AT == 2 || AT == 4), "A tiles per wave");
    constexpr int RPT = U1 ? 16 : 8;  // batch rows per A tile
    constexpr int VPL = U1 ? 4 : 2;   // batch rows per result lane and A tile
    constexpr int NWV = NTH / 64;
    constexpr int ng = NWV / NVS;  // batch groups of a tile (the host passes the same in ng_arg)
    (void)ng_arg;
    extern __shared__ uint4 wlds[];  // 2 chunk buffers
    const int r = 32 * KS;
    const int B = p.B, V = p.V;
    // XCD-aware split: blocks go round-robin over the XCDs, so block i runs on XCD
    // i % XCDS; the nbt batch tiles of one vocabulary range get consecutive
    // indices within one XCD and read that range's W2 through its L2 together
    const int nbt = (B + 127) / 128, nvb = gridDim.x / nbt;  // nvb is a multiple of XCDS
    const int xcd = blockIdx.x % XCDS, j = blockIdx.x / XCDS;
    const int bt = j % nbt, vb = (j / nbt) * XCDS + xcd;
    const int lane = threadIdx.x & 63, col = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int grp = wave % ng, vs = wave / ng;
    constexpr int CRr = NVS * VTG * 16;  // chunk rows
    const int row0 = bt * 128 + grp * AT * RPT;
    const long long v0 = static_cast<long long>(V) * vb / nvb;
    const int n = static_cast<int>(static_cast<long long>(V) * (vb + 1) / nvb - v0);
    if (n <= 0)
        return;  // an empty range (V below the number of ranges)
    const int nchunk = (n + CRr - 1) / CRr;
    const int g = blockIdx.x % NG;
    constexpr int slots = (CRr / 16) * KS * 64;  // uint4 per chunk
    constexpr int PT = slots / NTH;              // staging registers per thread
    static_assert(slots % NTH == 0, "chunk slots per thread");

    // A operands of this wave
    uint4 ua[AT][KS];
#pragma unroll
    for (int a = 0; a < AT; ++a) {
        // operand row m = col: U1, batch row m; otherwise batch row a*8 + m/2, its hi
        // part in even rows and its lo part in odd ones, so a result lane holds both
        // halves of its rows
        const int b = U1 ? row0 + col : row0 + a * 8 + (col >> 1);
        const bool hi = U1 || (col & 1) == 0;
        const float *src = p.u_buf + static_cast<size_t>(b < B ? b : 0) * r + (lane >> 4) * 8;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float x[8];
            if (b < B) {
                const float4 x0 = *reinterpret_cast<const float4 *>(src + kk * 32);
                const float4 x1 = *reinterpret_cast<const float4 *>(src + kk * 32 + 4);
                x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
                x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            } else {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    x[jj] = 0.f;
            }
            uint32_t hv[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const uint32_t xh = bf16_rne_bits(x[jj]);
                hv[jj] = hi ? xh : bf16_rne_bits(x[jj] - __uint_as_float(xh << 16));
            }
            ua[a][kk] = make_uint4(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                                   hv[6] | (hv[7] << 16));
        }
    }

    // staging: slot s of a chunk = (tile, step, lane) -> 16 bytes of W2.  Every load
    // is issued on every path, so the compiler's wait counts stay exact: a conditional
    // load makes it wait for every load in flight, the chunks loaded ahead included.
    // Both streams are read through buffer resources whose record counts end at the
    // data: a load past the records returns 0 without touching memory, so rows past
    // the range or past B need no clamped index (their results are masked).  W2: from
    // the range's first row, n rows.  The lane's part of every offset is a constant;
    // the rest is uniform.
    const __amdgpu_buffer_rsrc_t w2r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(static_cast<const uint16_t *>(p.W2)) + v0 * r, 0, n * r * 2, 0x00020000);
    const uint32_t w2lane = static_cast<uint32_t>(((lane & 15) * r + (lane >> 4) * 8) * 2);
    auto stage_load = [&](int c, uint4 (&st)[PT]) {
#pragma unroll
        for (int jj = 0; jj < PT; ++jj) {
            // slot s = threadIdx.x + jj * NTH: 64-lane group wo = s / 64 is uniform
            const int wo = wave + jj * NWV, vt = wo / KS, kk = wo % KS;
            const uint32_t off = static_cast<uint32_t>(((c * CRr + vt * 16) * r + kk * 32) * 2) + w2lane;
            st[jj] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(w2r, off, 0, 0));
        }
    };
    auto stage_store = [&](int buf, const uint4 (&st)[PT]) {
#pragma unroll
        for (int jj = 0; jj < PT; ++jj)
            wlds[buf * slots + threadIdx.x + jj * NTH] = st[jj];
    };
    // this lane's batch rows: result rows 4*(lane/16) + i of A tile a are batch rows
    // 4*(lane/16) + i (U1), else hi (i even) and lo (i odd) of batch row
    // a*8 + 2*(lane/16) + i/2
    int brow[AT][VPL];
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int ii = 0; ii < VPL; ++ii)
            brow[a][ii] = row0 + a * RPT + VPL * (lane >> 4) + ii;
    // L_base of this lane's epilogue values for chunk c: a buffer resource from the
    // wave's first batch row at this position to the end of L_base (batch rows past B
    // lie past it; at most 2^32 - 1 bytes, more than the wave's 16 rows span)
    constexpr int LES = LB16 ? 2 : 4;
    const long long lfirst = (static_cast<long long>(row0) * p.K + pos) * V + v0;
    const long long lleft = (static_cast<long long>(B) * p.K * V - lfirst) * LES;
    const __amdgpu_buffer_rsrc_t lbr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(p.L_base)) + (lleft > 0 ? lfirst * LES : 0), 0,
        static_cast<int>(static_cast<uint32_t>(lleft <= 0 ? 0 : lleft > 0xFFFFFFFFll ? 0xFFFFFFFFll : lleft)),
        0x00020000);
    // offsets in 32 bits (the host takes this kernel only for V < 2^22)
    const uint32_t KV = static_cast<uint32_t>(p.K) * static_cast<uint32_t>(V);
    const uint32_t lblane = (static_cast<uint32_t>(VPL * (lane >> 4)) * KV + col) * LES;
    auto lbase_load = [&](int c, float (&lb)[AT][VTG][VPL]) {
#pragma unroll
        for (int a = 0; a < AT; ++a)
#pragma unroll
            for (int ii = 0; ii < VPL; ++ii) {
                const uint32_t off =
                    lblane + (static_cast<uint32_t>(RPT * a + ii) * KV + static_cast<uint32_t>(c * CRr + vs * VTG * 16)) * LES;
#pragma unroll
                for (int vt = 0; vt < VTG; ++vt) {
                    // streamed once, but through the cache: one load covers a 64-byte row
                    // segment of a tile (32 bytes in bf16) and the next tile's load the
                    // rest of the line, which then hits (non-temporal loads measured 8%
                    // slower per call at B = 256)
                    // bf16 values are kept as loaded and widened in the epilogue: a
                    // conversion here would make the step wait for these loads
                    if constexpr (LB16)
                        lb[a][vt][ii] = __uint_as_float(
                            static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(lbr, off + vt * 16 * LES, 0, 0)));
                    else
                        lb[a][vt][ii] =
                            __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lbr, off + vt * 16 * LES, 0, 0));
                }
            }
    };

    LaneBest best[AT][VPL];
    // Software pipeline over chunks, unrolled by two so register sets are fixed
    // by the chunk parity P.  Step c: the W2 registers of chunk c+1 (loaded one
    // step ago) go to LDS buffer P^1, whose chunk c-1 every wave multiplied before
    // the last barrier, and chunk c+2 is loaded into the same registers; chunk c
    // is multiplied into accumulator set P while the epilogue of chunk c-1 runs
    // from set P^1 (independent instructions, so the compiler interleaves the
    // products with the vector work); then L_base of chunk c+1 is loaded into
    // the value set just consumed, a full step before its epilogue.
    uint4 st[PT];
    float lb[2][AT][VTG][VPL];
    f32x4_t acc[2][AT][VTG];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int a = 0; a < AT; ++a)
#pragma unroll
            for (int vt = 0; vt < VTG; ++vt)
#pragma unroll
                for (int ii = 0; ii < VPL; ++ii)
                    lb[s2][a][vt][ii] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int a = 0; a < AT; ++a)
#pragma unroll
            for (int vt = 0; vt < VTG; ++vt)
                acc[s2][a][vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int clast = nchunk - 1;  // loads past the last chunk repeat it
    // the loads in flight when the loop starts are in the order of those at a
    // step's end (W2 registers, then L_base), so the first step's wait for the
    // W2 registers does not also take in the L_base loads
    stage_load(0, st);
    stage_store(0, st);
    stage_load(1 < clast ? 1 : clast, st);
    lbase_load(0, lb[0]);
    __syncthreads();
    // epilogue of chunk c (c < 0: no chunk, every value masked) from accumulator
    // set S and L_base set S
    auto epilogue = [&](int c, int S) {
#pragma unroll
        for (int a = 0; a < AT; ++a)
#pragma unroll
            for (int vt = 0; vt < VTG; ++vt) {
                const int vr = c * CRr + (vs * VTG + vt) * 16 + col;
#pragma unroll
                for (int ii = 0; ii < VPL; ++ii) {
                    // U1: the row's product; else hi + lo of the batch row (the resident
                    // kernel's order)
                    const float w = U1 ? acc[S][a][vt][ii] : acc[S][a][vt][2 * ii] + acc[S][a][vt][2 * ii + 1];
                    const int b = brow[a][ii];
                    // c < 0 gives vr < 0, out of range as unsigned; no short-circuit
                    // branch, so the epilogue stays in the products' basic block.  A
                    // lane's batch row is fixed and a row past B is never folded into
                    // a key, so without L_final stores only the vocabulary bound counts
                    const bool ok = (!ST || b < B) & (static_cast<unsigned>(vr) < static_cast<unsigned>(n));
                    float *lf = ST ? p.L_final + (static_cast<size_t>(b) * p.K + pos) * V + v0 : nullptr;
                    const float lbv = LB16 ? __uint_as_float(__float_as_uint(lb[S][a][vt][ii]) << 16) : lb[S][a][vt][ii];
                    w2_key(w, lbv, lf, static_cast<int>(v0), vr, ok, best[a][ii]);
                }
            }
    };
    auto step = [&](int c, int P) {
        stage_store(P ^ 1, st);
        stage_load(c + 2 < clast ? c + 2 : clast, st);
        // keep these loads at the top of the step: the next step's first
        // instructions wait for them
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < AT; ++a)
#pragma unroll
            for (int vt = 0; vt < VTG; ++vt)
                acc[P][a][vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // the W2 operands of step kk + 1 are read from LDS while step kk is multiplied
        const uint4 *wb = wlds + P * slots + (vs * VTG * KS) * 64 + lane;
        uint4 wf[2][VTG];
#pragma unroll
        for (int vt = 0; vt < VTG; ++vt)
            wf[0][vt] = wb[(vt * KS) * 64];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (kk + 1 < KS) {
#pragma unroll
                for (int vt = 0; vt < VTG; ++vt)
                    wf[(kk + 1) & 1][vt] = wb[(vt * KS + kk + 1) * 64];
            }
#pragma unroll
            for (int vt = 0; vt < VTG; ++vt)
#pragma unroll
                for (int a = 0; a < AT; ++a)
                    acc[P][a][vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, ua[a][kk]), __builtin_bit_cast(bf16x8_t, wf[kk & 1][vt]),
                        acc[P][a][vt], 0, 0, 0);
        }
        epilogue(c - 1, P ^ 1);
        lbase_load(c + 1 < clast ? c + 1 : clast, lb[P ^ 1]);
        __syncthreads();
    };
    // both steps of a loop iteration run unconditionally: with the second one
    // optional, the compiler's wait counts at the loop head would also cover the
    // path that skips it, and the first step would wait for its own L_base loads
    int c = 0;
#pragma unroll 1
    for (; c + 1 < nchunk; c += 2) {
        step(c, 0);
        step(c + 1, 1);
    }
    if (c < nchunk)
        step(c, 0);
    if (clast & 1)
        epilogue(clast, 1);
    else
        epilogue(clast, 0);
    // each batch row's best over its 16 lanes, folded into the partial key slot
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int ii = 0; ii < VPL; ++ii) {
            uint64_t key = best[a][ii].ord ? (static_cast<uint64_t>(best[a][ii].ord) << 32) |
                                                 (0xFFFFFFFFu - best[a][ii].idx)
                                           : 0ull;
            key = max_u64(key, dpp_u64<DPP_QUAD_XOR1>(key));
            key = max_u64(key, dpp_u64<DPP_QUAD_XOR2>(key));
            key = max_u64(key, dpp_u64<DPP_HALF_MIRROR>(key));
            key = max_u64(key, dpp_u64<DPP_ROW_MIRROR>(key));
            const int b = brow[a][ii];
            if (col == 0 && b < B && key)
                __hip_atomic_fetch_max(gmem(key_slot(p, pos, g, b)), key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
}

// Tile order for a launch of n one-tile blocks: blocks are dealt to the XCDs
// round robin (block b runs on XCD b % XCDS), so block b takes tile
// (b % XCDS) * (n / XCDS) + b / XCDS, giving each XCD a contiguous range of
// tiles whose shared operand rows stay in its own L2.
__device__ inline int xcd_tile(int b, int n) { return n % XCDS ? b : (b % XCDS) * (n / XCDS) + b / XCDS; }

// Split-K matrix-core tile shared by the A_H and state launches: the block's
// four waves take consecutive quarters of the K steps (32 wide) of one output
// tile of NA x NB 16x16 blocks, each wave issuing the loads of up to KU steps
// before its first product; wave 0 then adds the partial tiles in wave order.
// ld(s, av, bv) loads step s's operands of this lane.  Returns true in wave 0,
// whose acc holds the tile.
template <int NA, int NB, int KU, typename Ld>
__device__ __forceinline__ bool splitk_tile(int nst, Ld ld, f32x4_t (&acc)[NA][NB], f32x4_t *part)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int t = 0; t < NB; ++t)
            acc[a][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int per = (nst + NWAVE - 1) / NWAVE;
    const int s0 = wave * per, s1 = s0 + per < nst ? s0 + per : nst;
    for (int sb = s0; sb < s1; sb += KU) {
        uint4 av[KU][NA], bv[KU][NB];
        // every load is issued (steps past s1 repeat the last one and are not
        // multiplied), so the compiler waits for each step's operands alone instead
        // of for every load in flight
#pragma unroll
        for (int u = 0; u < KU; ++u)
            ld(sb + u < s1 ? sb + u : s1 - 1, av[u], bv[u]);
#pragma unroll
        for (int u = 0; u < KU; ++u)
            if (sb + u < s1)
#pragma unroll
                for (int t = 0; t < NB; ++t)
#pragma unroll
                    for (int a = 0; a < NA; ++a)
                        acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u][a]),
                                                                           __builtin_bit_cast(bf16x8_t, bv[u][t]),
                                                                           acc[a][t], 0, 0, 0);
    }
    if (wave > 0) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int t = 0; t < NB; ++t)
                part[((wave - 1) * NA * NB + a * NB + t) * 64 + lane] = acc[a][t];
    }
    __syncthreads();
    if (wave > 0)
        return false;
#pragma unroll
    for (int w = 1; w < NWAVE; ++w)
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                const f32x4_t v = part[((w - 1) * NA * NB + a * NB + t) * 64 + lane];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[a][t][i] += v[i];
            }
    return true;
}

// State-phase dot products of the stepwise launches at larger B, on the matrix
// cores (same quantities as phase_state):
//   u_q[b][m]      = SiLU(A_H[b][q][m] + sum_k W1[m][d + k] S_q[b][k])   (m < r)
//   q_{q+1}[b][m'] = sum_k W_hh[m'][k] S_q[b][k] + b_hh[m']             (m' = m - r)
// A operand: S_q as bf16 hi + lo rows of 8 batch rows (planes written by the
// update launch); B operand: 16 weight rows.  A block takes 32 batch rows and
// 32 weight rows (split-K over h).
// Epilogue of the state dot products: u = SiLU(A_H + dot) for rows m < r, the
// next step's q = dot + b_hh for the W_hh rows.  acc holds four 8-row batch tiles
// (hi rows 0..7, lo rows 8..15 of each) by two 16-row weight tiles; weight row m =
// mbase + t*16 + col, batch row b = bbase + (2pp + (lane >> 5))*8 + ((lane >> 4) & 1)*4 + i.
// The A_H and bias values are loaded first, every load on every path (clamped
// indices, unused values dropped), so the compiler waits once for all of them
// instead of once per conditional load.
template <typename WT, int NP = 2>
__device__ __forceinline__ void state_epilogue(const Params &p, int q, const f32x4_t (&acc)[2 * NP][2], int mbase,
                                               int bbase)
{
    const int lane = threadIdx.x & 63, col = lane & 15;
    const int h = p.h, r = p.r, R = r + 3 * p.h, B = p.B, h3 = 3 * h;
    float *qn = q_slot(p, q + 1);
    float ahv[NP][2][4], bias[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int m = mbase + t * 16 + col;
        const int mq = (m >= r && m < R) ? m - r : 0;
        const int mu = m < r ? m : 0;
        bias[t] = p.b_hh ? WT16<WT>::one(p.b_hh, mq) : 0.f;
#pragma unroll
        for (int pp = 0; pp < NP; ++pp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = bbase + (2 * pp + (lane >> 5)) * 8 + ((lane >> 4) & 1) * 4 + i;
                ahv[pp][t][i] = p.A_H[(static_cast<size_t>(b < B ? b : 0) * p.K + q) * r + mu];
            }
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int m = mbase + t * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = w2_hilo(acc[2 * pp][t], i), x1 = w2_hilo(acc[2 * pp + 1][t], i);
                const auto dd = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x1), false,
                                                                 false);
                const float dot = __uint_as_float(dd[0]);
                const int b = bbase + (2 * pp + (lane >> 5)) * 8 + ((lane >> 4) & 1) * 4 + i;
                if (b >= B || m >= R)
                    continue;
                if (m < r) {
                    const float a_ = ahv[pp][t][i] + dot;
                    const float u = a_ * sigmoidf_(a_);
                    p.u_buf[static_cast<size_t>(b) * r + m] = u;
                    if (p.u_out)
                        p.u_out[(static_cast<size_t>(b) * p.K + q) * r + m] = u;
                } else {
                    qn[static_cast<size_t>(b) * h3 + (m - r)] = dot + bias[t];
                }
            }
        }
}

template <typename WT, int KU = 8>
__global__ __launch_bounds__(NT) void k_state_mfma(Params p, int q)
{
    __shared__ f32x4_t part[(NWAVE - 1) * 4 * 2 * 64];
    const int h = p.h, r = p.r, R = r + 3 * p.h, B = p.B;
    const int nbg = (B + 31) / 32, nwb = (R + 31) / 32;
    const int tile = xcd_tile(blockIdx.x, nbg * nwb);
    const int bg = tile % nbg, wb = tile / nbg;
    const int lane = threadIdx.x & 63, col = lane & 15;
    const int mw = wb * 32;  // first weight row of the block
    const int b0 = bg * 32;
    // operand sources of this lane
    const uint16_t *arow[4];
    bool aok[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int b = b0 + a * 8 + (col & 7);
        aok[a] = b < B;
        arow[a] = p.s_hl + (static_cast<size_t>(col >> 3) * p.maxB + (aok[a] ? b : 0)) * p.ldw + (lane >> 4) * 8;
    }
    const bf16s *wrow[2];
    bool wok[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int m = mw + t * 16 + col;
        wok[t] = m < R;
        const int mm = wok[t] ? m : 0;
        wrow[t] = p.wst ? reinterpret_cast<const bf16s *>(p.wst) + static_cast<size_t>(mm) * p.ldw
                  : mm < r ? static_cast<const bf16s *>(p.W1) + static_cast<size_t>(mm) * (p.d + h) + p.d
                           : static_cast<const bf16s *>(p.W_hh) + static_cast<size_t>(mm - r) * h;
        wrow[t] += (lane >> 4) * 8;
    }
    f32x4_t acc[4][2];
    const bool lead = splitk_tile<4, 2, KU>(
        h / 32,
        [&](int s, uint4(&av)[4], uint4(&wv)[2]) {
            const int k = s * 32;
            // rows past B or R read row 0 (clamped pointers); their results are not stored
#pragma unroll
            for (int a = 0; a < 4; ++a)
                av[a] = *reinterpret_cast<const uint4 *>(arow[a] + k);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                wv[t] = *reinterpret_cast<const uint4 *>(wrow[t] + k);
        },
        acc, part);
    if (!lead)
        return;
    state_epilogue<WT>(p, q, acc, mw, b0);
}

// The same state dots with the operands staged in LDS (h a multiple of 256).  A
// block takes 32 batch rows (4 A tiles of S hi/lo rows) x 64 weight rows (4 B
// tiles): more blocks than compute units at B = 256, two resident per unit.  The
// h reduction runs in stages of 64 (two 32-wide steps); a stage's 16 operand
// blocks (per step: 4 A + 4 B tiles, 1 KB each in the matrix-core operand
// layout) are copied by 16-byte direct global-to-LDS loads, three stages ahead,
// into a ring of four LDS buffers, so the loads use no registers and the S rows
// are read once per block instead of once per wave.  Each wave multiplies 2 A
// tiles x 2 B tiles; one barrier per stage.  The products run over k in
// the same order as in k_state_mfma's single pass.
constexpr int SL_BLOCKS = 8;                 // operand blocks per step: 4 A + 4 B tiles
constexpr int SL_STAGE = 2 * SL_BLOCKS * 64; // uint4 per stage (two steps)

template <typename WT>
__global__ __launch_bounds__(NT) void k_state_lds(Params p, int q)
{
    typedef __attribute__((address_space(3))) void lds_void;
    __shared__ uint4 ring0[SL_STAGE], ring1[SL_STAGE], ring2[SL_STAGE], ring3[SL_STAGE];
    static_assert(NWAVE == 4, "four waves: 2 x 2 over the A and B tiles");
    const int h = p.h, r = p.r, R = r + 3 * p.h, B = p.B;
    const int nbg = (B + 31) / 32, nwb = (R + 63) / 64;
    const int tile = xcd_tile(blockIdx.x, nbg * nwb);
    const int bg = tile % nbg, wbk = tile / nbg;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int b0 = bg * 32, mw = wbk * 64;
    const int NS = h / 64;  // stages, a multiple of 4
    // this lane's source of the 4 operand blocks this wave copies per stage:
    // block j = wave * 4 + u = step * 8 + t, t < 4: A tile t, else B tile t - 4.
    // Rows past B or R repeat the last row (their results are not stored).
    const uint16_t *src[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = wave * 4 + u, ks = j / SL_BLOCKS, t = j % SL_BLOCKS, i = lane & 15;
        const uint16_t *base;
        if (t < 4) {
            const int b = b0 + t * 8 + (i & 7) < B ? b0 + t * 8 + (i & 7) : B - 1;
            base = p.s_hl + (static_cast<size_t>(i >> 3) * p.maxB + b) * p.ldw;
        } else {
            const int m = mw + (t - 4) * 16 + i < R ? mw + (t - 4) * 16 + i : R - 1;
            base = p.wst ? p.wst + static_cast<size_t>(m) * p.ldw
                   : m < r ? static_cast<const uint16_t *>(p.W1) + static_cast<size_t>(m) * (p.d + h) + p.d
                           : static_cast<const uint16_t *>(p.W_hh) + static_cast<size_t>(m - r) * h;
        }
        src[u] = base + ks * 32 + (lane >> 4) * 8;
    }
    auto issue = [&](int s, uint4 *ring) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            __builtin_amdgcn_global_load_lds(src[u] + s * 64, (lds_void *)(ring + (wave * 4 + u) * 64), 16, 0, 0);
    };
    const int wa = wave & 1, wb = wave >> 1;
    f32x4_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            acc[a][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const uint4 *ring) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            uint4 av[2], bv[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                av[a] = ring[(ks * SL_BLOCKS + wa * 2 + a) * 64 + lane];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                bv[t] = ring[(ks * SL_BLOCKS + 4 + wb * 2 + t) * 64 + lane];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int a = 0; a < 2; ++a)
                    acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[a]),
                                                                       __builtin_bit_cast(bf16x8_t, bv[t]), acc[a][t],
                                                                       0, 0, 0);
        }
    };
    // wait until at most `later` stages of this wave's copies are outstanding (4 loads
    // each), then a barrier: every wave has waited for its own copies of the stage, so
    // the stage is in LDS for all of them.  The barrier is the bare instruction: a
    // __syncthreads() would also wait for the copies of the later stages.  Each wave's
    // reads of the previous buffer have returned (the products used them) before it
    // arrives, so the buffer the next copy overwrites is free.
    auto arrive = [&](int later) {
        // s_waitcnt vmcnt(N): expcnt and lgkmcnt left at their maxima
        if (later >= 2)
            __builtin_amdgcn_s_waitcnt(8 | (7 << 4) | (15 << 8));
        else if (later == 1)
            __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8));
        else
            __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto step = [&](int s, const uint4 *cur, uint4 *nxt) {
        arrive((NS - 1 - s) < 2 ? NS - 1 - s : 2);
        if (s + 3 < NS)
            issue(s + 3, nxt);  // the buffer of stage s - 1, which every wave has finished
        compute(cur);
    };
    issue(0, ring0);
    issue(1, ring1);
    issue(2, ring2);
#pragma unroll 1
    for (int s = 0; s < NS; s += 4) {
        step(s, ring0, ring3);
        step(s + 1, ring1, ring0);
        step(s + 2, ring2, ring1);
        step(s + 3, ring3, ring2);
    }
    state_epilogue<WT, 1>(p, q, acc, mw + wb * 32, b0 + wa * 16);
}

// A_H = W1[:, :d] H for every position on the matrix cores (same quantity as
// phase_ah): rows R = b * K + i of H (bf16, [B*K, d]) times rows m of W1's
// first d columns; A_H[R][m] in fp32.  A block takes 32 H rows x 32 W1 rows
// (2 x 2 tiles of v_mfma_f32_16x16x32_bf16, split-K over d).
// NA x NB 16-row tiles per block (32 x 32 below 2048 rows; 64 x 64 from there,
// which halves the operand rows each output reads through L2)
template <typename WT, int NA, int NB, int KU>
__global__ __launch_bounds__(NT) void k_ah_mfma(Params p)
{
    __shared__ f32x4_t part[(NWAVE - 1) * NA * NB * 64];
    const int d = p.d, r = p.r, M = p.B * p.K;
    const int lane = threadIdx.x & 63, col = lane & 15;
    const int tiles_n = r / (NB * 16), tiles_m = (M + NA * 16 - 1) / (NA * 16);
    const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile / tiles_n, tn = tile % tiles_n;
    const int R0 = tm * NA * 16, m0 = tn * NB * 16;
    const bf16s *arow[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        const int R = R0 + a * 16 + col;
        arow[a] = static_cast<const bf16s *>(p.H) + static_cast<size_t>(R < M ? R : 0) * d + (lane >> 4) * 8;
    }
    const bf16s *wrow[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t)
        wrow[t] = static_cast<const bf16s *>(p.W1) + static_cast<size_t>(m0 + t * 16 + col) * (d + p.h) + (lane >> 4) * 8;
    f32x4_t acc[NA][NB];
    const bool lead = splitk_tile<NA, NB, KU>(
        d / 32,
        [&](int s, uint4(&av)[NA], uint4(&wv)[NB]) {
            const int k = s * 32;
            // rows past B K read row 0 (clamped pointer); their results are not stored
#pragma unroll
            for (int a = 0; a < NA; ++a)
                av[a] = *reinterpret_cast<const uint4 *>(arow[a] + k);
#pragma unroll
            for (int t = 0; t < NB; ++t)
                wv[t] = *reinterpret_cast<const uint4 *>(wrow[t] + k);
        },
        acc, part);
    if (!lead)
        return;
    // D: lane l holds H rows (l/16)*4 + i of the A tile, W1 row l%16 of the B tile
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int R = R0 + a * 16 + (lane >> 4) * 4 + i;
                if (R < M)
                    p.A_H[static_cast<size_t>(R) * r + m0 + t * 16 + col] = acc[a][t][i];
            }
}

constexpr int BAT_KS = 8;  // r = 256

}  // namespace DH_NS

namespace dhbat {

using namespace dh256;

int r_supported() { return 32 * BAT_KS; }
int threads() { return NT; }
// Launch shape of the batched W2 kernel for B rows: 512 threads (2 A tiles per
// wave, two waves per SIMD) with ng 16-row groups per batch tile.  (Four A tiles
// per wave in 256-thread blocks halve the LDS operand traffic but, with one wave
// per SIMD, measured 123 us against 85 us per 8B position at B = 256.)
struct W2Shape {
    const void *fn;
    int threads, ng;
};
// ng batch groups of 16 rows per 128-row tile; the 8 waves form 8 / ng wave sets that
// split each 64-row chunk (128 rows for ng = 1)
template <bool LB16, bool ST, bool U1>
static const void *w2_fn(int ng)
{
    constexpr int AT = U1 ? 1 : 2;
    return ng == 8   ? reinterpret_cast<const void *>(&k_w2_mfma<BAT_KS, 4, 1, AT, 512, LB16, ST, U1>)
           : ng == 4 ? reinterpret_cast<const void *>(&k_w2_mfma<BAT_KS, 2, 2, AT, 512, LB16, ST, U1>)
           : ng == 2 ? reinterpret_cast<const void *>(&k_w2_mfma<BAT_KS, 1, 4, AT, 512, LB16, ST, U1>)
                     : reinterpret_cast<const void *>(&k_w2_mfma<BAT_KS, 1, 8, AT, 512, LB16, ST, U1>);
}
template <bool U1>
static const void *w2_fn(int ng, bool lb16, bool store)
{
    return lb16 ? (store ? w2_fn<true, true, U1>(ng) : w2_fn<true, false, U1>(ng))
                : (store ? w2_fn<false, true, U1>(ng) : w2_fn<false, false, U1>(ng));
}
static W2Shape w2_shape(int B, bool lb16 = false, bool store = false, bool u1 = false)
{
    const int need = ((B < 128 ? B : 128) + 15) / 16;
    const int ng = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
    return {u1 ? w2_fn<true>(ng, lb16, store) : w2_fn<false>(ng, lb16, store), 512, ng};
}
const void *w2_kernel(int B, bool lbase_bf16, bool store_logits, bool u_single)
{
    return w2_shape(B, lbase_bf16, store_logits, u_single).fn;
}
int w2_groups(int B) { return w2_shape(B).ng; }
int w2_threads(int B) { return w2_shape(B).threads; }
// one block per compute unit: batch tiles times vocabulary ranges
int w2_grid(int B, int cus)
{
    const int nbt = (B + 127) / 128;
    int nvb = (cus + nbt - 1) / nbt;
    nvb = (nvb + XCDS - 1) / XCDS * XCDS;
    return nbt * nvb;
}
// two chunk buffers of up to 128 rows x 256 bf16
size_t w2_smem() { return 2 * sizeof(uint4) * (128 / 16) * BAT_KS * 64; }
// B >= 64 and h a multiple of 256: the LDS-staged kernel (64-row batch tiles); otherwise
// the split-K one (32-row tiles: more blocks at smaller B).  Measured at 8B shapes: the
// staged launch takes 22 us against 31 us at B = 256, while at B = 32 a whole call took
// 877 us with it against 805 us without.
static bool state_staged(int B, int h) { return B >= 64 && h % 256 == 0; }
const void *state_kernel(int B, int h)
{
    return state_staged(B, h) ? reinterpret_cast<const void *>(&k_state_lds<bf16s>)
                              : reinterpret_cast<const void *>(&k_state_mfma<bf16s>);
}
static bool ah_wide(int B, int K, int r) { return B * K >= 2048 && r % 64 == 0; }
const void *ah_kernel(int B, int K, int r)
{
    return ah_wide(B, K, r) ? reinterpret_cast<const void *>(&k_ah_mfma<bf16s, 4, 4, 4>)
                            : reinterpret_cast<const void *>(&k_ah_mfma<bf16s, 2, 2, 8>);
}
int ah_grid(int B, int K, int r)
{
    return ah_wide(B, K, r) ? (B * K + 63) / 64 * (r / 64) : (B * K + 31) / 32 * (r / 32);
}
int state_grid(int B, int r, int h)
{
    return state_staged(B, h) ? ((B + 31) / 32) * ((r + 3 * h + 63) / 64) : ((B + 31) / 32) * ((r + 3 * h + 31) / 32);
}

}  // namespace dhbat
