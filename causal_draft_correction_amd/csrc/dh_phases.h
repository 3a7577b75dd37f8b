// The phases of one Domino head block draft.  Each phase is a device
// function over a slice of independent work (selected by blk of nblk), so
// the same code runs inside the persistent cooperative kernel (phases
// separated by grid barriers) and as separate stepwise launches.
//
// Method (paper.oopus.info review, section 二, 第二步 Domino Head; news.sig.ai
// article, section "Domino怎么做"), positions p = 0..K-1:
//   u_p     = SiLU(W1 [H_p; S_p])
//   L_p     = L_base_p + W2 u_p,  t_p = argmax L_p   (greedy)
//   S_{p+1} = GRU(E[x_p], S_p),   x_p = t_p or the teacher token
// with S_0 = GRU(E[last_tok], S_init).  The work is regrouped as follows; every
// regrouping is an exact identity:
//   * W1 [H_p; S_p] = W1_H H_p + W1_S S_p, and A_H[p] = W1_H H_p for all
//     positions is computed once (phase_ah);
//   * the GRU cell is split into its two affine parts, the input part
//     g = W_ih E[x] + b_ih and the state part q = W_hh S + b_hh, plus the
//     elementwise gate update.  q for the next step and u for the next position
//     depend only on the new state, so both are dot products over S computed
//     right after it (phase_state).  g is either a row of the folded table
//     P = E W_ih^T + b_ih (gathered) or computed after the token is known
//     (phase_g);
//   * the elementwise update is cheap, so every block computes the whole new
//     state for itself: S never has to cross blocks in the persistent launch.
#pragma once

#include <type_traits>

#include "dh_common.h"
#include "dh_params.h"

namespace DH_NS {

using dhp::Params;

// ---- shared-memory layout (floats) ----------------------------------------------
// red [256] | kred [2*NWAVE] | tok [TOK_SLOTS] | u_lds [BC*r] | lbuf [BC*rows_cap] | S_lds [BC*h]
// Every kernel allocates the prefix it uses: the small phases up to tok, the
// W2 phase up to lbuf, phase_state up to S_lds with rows_cap = 0 in stepwise
// launches, the persistent kernel all of it.  TOK_SLOTS covers the batch rows
// one block touches in phase_update (NT/8 + 2 at h >= 8).
constexpr int TOK_SLOTS = 128;
constexpr int ATOK_OFF = 64;  // persistent launch: barrier-delivered tokens at tok + ATOK_OFF
__host__ __device__ inline int smem_off_tok() { return 256 + 2 * NWAVE; }
__host__ __device__ inline int smem_off_u() { return 256 + 2 * NWAVE + TOK_SLOTS; }
__host__ __device__ inline int smem_off_lbuf(int r) { return smem_off_u() + BC * r; }
__host__ __device__ inline int smem_off_S(int r, int rows_cap) { return smem_off_lbuf(r) + BC * rows_cap; }
// First vocabulary row of block blk's slice, V * blk / nblk, in 32-bit arithmetic
// (the resident launches take V <= 2^18 and at most MAX_GRID = 2^10 blocks, so the
// product stays below 2^28; a 64-bit division costs about a hundred instructions).
__host__ __device__ inline int vslice_lo(int V, int blk, int nblk)
{
    return static_cast<int>(static_cast<unsigned>(V) * static_cast<unsigned>(blk) / static_cast<unsigned>(nblk));
}
// Row stride of lbuf: the block's vocabulary rows, padded to whole 16-row tiles.
__host__ __device__ inline int lbuf_stride(int V, int nblk) { return ((V + nblk - 1) / nblk + 15) & ~15; }
__host__ __device__ inline int smem_floats_small() { return smem_off_u(); }
__host__ __device__ inline int smem_floats_w2(int r, int rows_cap) { return smem_off_S(r, rows_cap); }
__host__ __device__ inline int smem_floats(int r, int h, int rows_cap) { return smem_off_S(r, rows_cap) + BC * h; }

// ---- token bookkeeping ------------------------------------------------------

__device__ inline bool tok_ok(int t, int V) { return t >= 0 && t < V; }

// Element i of L_base, float32 or bfloat16 (widened exactly).
__device__ inline float lbase_at(const Params &p, size_t i)
{
    if (p.lbase_bf16)
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p.L_base)[i]) << 16);
    return static_cast<const float *>(p.L_base)[i];
}

// A row is invalid when its anchor or a used teacher token is outside [0, V).
__device__ inline bool row_bad(const Params &p, int b)
{
    if (!tok_ok(p.last_tok[b], p.V))
        return true;
    if (p.teacher) {
        for (int i = 0; i + 1 < p.K; ++i)
            if (!tok_ok(p.teacher[static_cast<size_t>(b) * p.K + i], p.V))
                return true;
    }
    return false;
}

__device__ inline uint64_t *key_slot(const Params &p, int pos, int g, int b)
{
    return p.keys + (static_cast<size_t>(pos) * NG + g) * p.maxB + b;
}

// Greedy token of position `pos` for row b: max over the NG partial keys.  All
// NG loads are issued before the first is used (one memory round trip).
__device__ inline int key_token(const Params &p, int pos, int b)
{
    uint64_t k[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g)
        k[g] = ld_agent_u64(key_slot(p, pos, g, b));
    uint64_t best = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g)
        best = k[g] > best ? k[g] : best;
    return best ? static_cast<int>(key_index(best)) : 0;
}

// GRU input token producing S_q: last_tok for q = 0, else teacher[q-1] or t_{q-1}.
// Invalid ids gather row 0; the row is reported through the flags instead.
// `atok` (persistent launch): greedy tokens of position q-1 delivered by the
// argmax barrier, indexed by batch row; otherwise they are read from the keys.
__device__ inline int gru_input_token(const Params &p, int q, int b, const int *atok = nullptr)
{
    int t;
    if (q == 0)
        t = p.last_tok[b];
    else if (p.teacher)
        t = p.teacher[static_cast<size_t>(b) * p.K + (q - 1)];
    else
        t = atok ? atok[b] : key_token(p, q - 1, b);
    return tok_ok(t, p.V) ? t : 0;
}

// Markov head (news.sig.ai article, section 从Domino看DSpark, names it beside
// the recurrent head without a formula).  Reading: position q is conditioned on
// the token before it alone, S_q = GRU(E[x_q], 0), so W1_S S_q is row x_q of
// the per-token table M = W1_S GRU(E[t], 0) filled at create, and
//   u_q = SiLU(A_H[q] + M[x_q]).
// `ah` is A_H[b][q][m]; x a valid token id (gru_input_token clamps).
__device__ inline float markov_u(const Params &p, float ah, int m, int x)
{
    const float a = ah + p.M[static_cast<size_t>(x) * p.r + m];
    return a * sigmoidf_(a);
}

// Publish tokens[:, pos] once position pos is complete (one block).
__device__ inline void write_tokens(const Params &p, int pos)
{
    for (int b = threadIdx.x; b < p.B; b += NT)
        p.tokens[static_cast<size_t>(b) * p.K + pos] = row_bad(p, b) ? -1 : key_token(p, pos, b);
}

// Zero the partial keys of this call and raise the bad-token flag.  Block 0.
__device__ inline void prologue_bookkeeping(const Params &p)
{
    const int n = p.K * NG;
    for (int i = threadIdx.x; i < n * p.B; i += NT) {
        const int slot = i / p.B, b = i % p.B;
        __hip_atomic_store(gmem(p.keys + static_cast<size_t>(slot) * p.maxB + b), 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int b = threadIdx.x; b < p.B; b += NT)
        if (row_bad(p, b))
            __hip_atomic_fetch_or(gmem(p.flags), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float *q_slot(const Params &p, int s) { return p.q_buf + static_cast<size_t>(s & 1) * p.maxB * 3 * p.h; }
__device__ inline float *S_slot(const Params &p, int s) { return p.S_buf + static_cast<size_t>(s & 1) * p.maxB * p.h; }

// Wave-cooperative dot of one WT row (n elements from `off`) with x given by a
// chunk loader xf(elem, float*).  Lanes take chunks lane, lane+64, ...; the
// per-lane partials are combined with a fixed xor tree, so every lane returns
// the same sum.
template <typename WT, typename XF>
__device__ inline float wave_dot(const void *W, size_t off, int n, XF xf)
{
    constexpr int EPC = WT16<WT>::EPC;
    const int lane = threadIdx.x & 63;
    float acc = 0.f;
#pragma unroll 4
    for (int c = lane; c < n / EPC; c += 64) {
        float x[EPC];
        xf(c * EPC, x);
        acc = dot_chunk<WT>(ld16<WT>(W, off + static_cast<size_t>(c) * EPC), x, acc);
    }
    return wave_sum(acc);
}

// A_H sums have one layout in every kernel: AH_LANES partial sums, lane t taking
// the 8- or 4-element chunks t, t + AH_LANES, ... of the row, reduced by wave
// (64 lanes) and then over the waves in order.  Threads beyond AH_LANES add
// zeros, so each entry is the same bits whatever the block size.
constexpr int AH_LANES = 256;

// ---- phase: A_H = W1[:, :d] H for every position ------------------------------
template <typename WT>
__device__ __forceinline__ void phase_ah(const Params &p, int blk, int nblk, float *red)
{
    constexpr int EPC = WT16<WT>::EPC;
    static_assert(NT >= AH_LANES, "block too small for the A_H sum layout");
    const int nch = p.d / EPC;
    const int ntask = p.B * p.r;
    for (int task = blk; task < ntask; task += nblk) {
        const int b = task / p.r, k = task % p.r;
        float acc[MAXK];
#pragma unroll
        for (int i = 0; i < MAXK; ++i)
            acc[i] = 0.f;
        for (int c = threadIdx.x; threadIdx.x < AH_LANES && c < nch; c += AH_LANES) {
            float w[EPC];
            WT16<WT>::unpack(ld16<WT>(p.W1, static_cast<size_t>(k) * (p.d + p.h) + static_cast<size_t>(c) * EPC), w);
#pragma unroll
            for (int i = 0; i < MAXK; ++i) {
                if (i < p.K) {
                    float x[EPC];
                    WT16<WT>::unpack(
                        ld16<WT>(p.H, (static_cast<size_t>(b) * p.K + i) * p.d + static_cast<size_t>(c) * EPC), x);
#pragma unroll
                    for (int e = 0; e < EPC; ++e)
                        acc[i] = fmaf(w[e], x[e], acc[i]);
                }
            }
        }
        block_sum<MAXK>(acc, red);
        if (threadIdx.x < p.K)
            xst(&p.A_H[(static_cast<size_t>(b) * p.K + threadIdx.x) * p.r + k], red[NWAVE * MAXK + threadIdx.x]);
        __syncthreads();
    }
}

// ---- phase: q for the initial state: W_hh S_init + b_hh ----------------------------
template <typename WT>
__device__ __forceinline__ void phase_q_init(const Params &p, int blk, int nblk)
{
    const int h3 = 3 * p.h;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float *qo = q_slot(p, 0);
    for (int m = blk * NWAVE + wave; m < h3; m += nblk * NWAVE) {
        const float bias = p.b_hh ? WT16<WT>::one(p.b_hh, m) : 0.f;
        for (int b = 0; b < p.B; ++b) {
            float v = bias;
            if (p.S_init) {
                const float *s = p.S_init + static_cast<size_t>(b) * p.h;
                v += wave_dot<WT>(p.W_hh, static_cast<size_t>(m) * p.h, p.h, [&](int e, float *x) {
                    for (int i = 0; i < WT16<WT>::EPC; ++i)
                        x[i] = s[e + i];
                });
            }
            if (lane == 0)
                xst(&qo[static_cast<size_t>(b) * h3 + m], v);
        }
    }
}

// ---- phase: g = W_ih E[x_q] + b_ih for the GRU step producing S_q (not folded) ------
// GRW: rows of a wave whose loads go out together (more rows take more registers: the
// resident persistent kernel, one wave per SIMD, takes 3; the launches that rely on
// several waves per SIMD take 1)
// With p.gtag each value goes out as a word carrying `tag` (see phase_state).
template <typename WT, int GRW = 1>
__device__ __forceinline__ void phase_g(const Params &p, int blk, int nblk, int q, float *smem, const int *atok = nullptr,
                                        unsigned tag = 0)
{
    const int h3 = 3 * p.h;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int *tok = reinterpret_cast<int *>(smem + smem_off_tok());
    for (int b0 = 0; b0 < p.B; b0 += BC) {
        const int nb = (p.B - b0) < BC ? (p.B - b0) : BC;
        __syncthreads();
        if (threadIdx.x < nb)
            tok[threadIdx.x] = gru_input_token(p, q, b0 + threadIdx.x, atok);
        __syncthreads();
        // the wave's rows m = m0 + i mstep go GRW at a time, and for each batch row the
        // loads of GCH chunks per lane of all of them (and of the embedding row) are
        // issued before the first product: one memory round trip per GCH chunks
        // instead of one per row and unrolled step.  Each row's sum is formed as in
        // wave_dot (chunks lane, lane + 64, ... in order, then wave_sum), so the
        // values equal the row-at-a-time ones bit for bit.
        constexpr int EPC = WT16<WT>::EPC;
        constexpr int GCH = 4;
        const int nch = p.d / EPC, mstep = nblk * NWAVE;
        for (int m0 = blk * NWAVE + wave; m0 < h3; m0 += GRW * mstep) {
            float bias[GRW];
#pragma unroll
            for (int i = 0; i < GRW; ++i) {
                const int m = m0 + i * mstep;
                bias[i] = (m < h3 && p.b_ih) ? WT16<WT>::one(p.b_ih, m) : 0.f;
            }
            for (int bb = 0; bb < nb; ++bb) {
                const size_t eo = static_cast<size_t>(tok[bb]) * p.d;
                float acc[GRW];
#pragma unroll
                for (int i = 0; i < GRW; ++i)
                    acc[i] = 0.f;
                for (int c0 = 0; c0 < nch; c0 += 64 * GCH) {
                    uint4 ev[GCH], wv[GRW][GCH];
#pragma unroll
                    for (int k = 0; k < GCH; ++k) {
                        const int c = c0 + k * 64 + lane;
                        const int cc = c < nch ? c : 0;  // past the row: chunk 0, not multiplied
                        ev[k] = ld16<WT>(p.E, eo + static_cast<size_t>(cc) * EPC);
#pragma unroll
                        for (int i = 0; i < GRW; ++i) {
                            const int m = m0 + i * mstep;
                            const int mc = m < h3 ? m : m0;
                            wv[i][k] = ld16<WT>(p.W_ih, static_cast<size_t>(mc) * p.d + static_cast<size_t>(cc) * EPC);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < GCH; ++k) {
                        if (c0 + k * 64 + lane < nch) {
                            float x[EPC];
                            WT16<WT>::unpack(ev[k], x);
#pragma unroll
                            for (int i = 0; i < GRW; ++i)
                                acc[i] = dot_chunk<WT>(wv[i][k], x, acc[i]);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < GRW; ++i) {
                    const int m = m0 + i * mstep;
                    const float v = bias[i] + wave_sum(acc[i]);
                    if (lane == 0 && m < h3) {
                        const size_t o = static_cast<size_t>(b0 + bb) * h3 + m;
                        if (p.gtag)
                            __hip_atomic_store(gmem(&p.gtag[o]),
                                               (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v),
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        else
                            xst(&p.g_buf[o], v);
                    }
                }
            }
        }
    }
}

// Entry m of b_hh (0 without biases), either weight type.
__device__ inline float bias_hh(const Params &p, int m)
{
    if (!p.b_hh)
        return 0.f;
    return p.bf16w ? WT16<bf16s>::one(p.b_hh, m) : WT16<float>::one(p.b_hh, m);
}

// ---- GRU gate update of one state entry ---------------------------------------------
// S_q[b][j] from g (P row or g_buf), q_{q-1} (W_hh S_{q-1} + b_hh) and S_{q-1}[b][j].
__device__ inline float gate_update(const Params &p, int q, int b, int j, int tokb, float sprev)
{
    const int h = p.h, h3 = 3 * h;
    float gr, gz, gn;
    if (p.P) {
        const float *prow = p.P + static_cast<size_t>(tokb) * h3;
        gr = prow[j];
        gz = prow[h + j];
        gn = prow[2 * h + j];
    } else {
        const float *g = p.g_buf + static_cast<size_t>(b) * h3;
        gr = xld(&g[j]);
        gz = xld(&g[h + j]);
        gn = xld(&g[2 * h + j]);
    }
    float qr, qz, qn;
    if (q == 0 && !p.S_init) {
        // W_hh S_init + b_hh with S_init = 0 is b_hh itself
        qr = bias_hh(p, j);
        qz = bias_hh(p, h + j);
        qn = bias_hh(p, 2 * h + j);
    } else {
        const float *qv = q_slot(p, q) + static_cast<size_t>(b) * h3;
        qr = xld(&qv[j]);
        qz = xld(&qv[h + j]);
        qn = xld(&qv[2 * h + j]);
    }
    const float rg = sigmoidf_(gr + qr);
    const float zg = sigmoidf_(gz + qz);
    const float ng = tanhf_(gn + rg * qn);
    return (1.f - zg) * ng + zg * sprev;
}

__device__ inline float state_prev(const Params &p, int q, int b, int j)
{
    if (q == 0)
        return p.S_init ? p.S_init[static_cast<size_t>(b) * p.h + j] : 0.f;
    return xld(&S_slot(p, q - 1)[static_cast<size_t>(b) * p.h + j]);
}

// ---- phase (stepwise launches): distributed gate update producing S_q -------------------
__device__ __forceinline__ void phase_update(const Params &p, int blk, int nblk, int q, float *smem)
{
    if (q >= 1 && blk == 0)
        write_tokens(p, q - 1);
    const int h = p.h;
    int *tok = reinterpret_cast<int *>(smem + smem_off_tok());
    // rows are processed in order, so a block touches few distinct rows
    for (size_t i = static_cast<size_t>(blk) * NT; i < static_cast<size_t>(p.B) * h; i += static_cast<size_t>(nblk) * NT) {
        const size_t e = i + threadIdx.x;
        const int b_first = static_cast<int>(i / h);
        const int b_last = static_cast<int>((i + NT - 1) / h) < p.B - 1 ? static_cast<int>((i + NT - 1) / h) : p.B - 1;
        __syncthreads();
        if (p.P && threadIdx.x <= b_last - b_first)
            tok[threadIdx.x] = gru_input_token(p, q, b_first + threadIdx.x);
        __syncthreads();
        if (e < static_cast<size_t>(p.B) * h) {
            const int b = static_cast<int>(e / h), j = static_cast<int>(e % h);
            const float sn = gate_update(p, q, b, j, p.P ? tok[b - b_first] : 0, state_prev(p, q, b, j));
            xst(&S_slot(p, q)[static_cast<size_t>(b) * h + j], sn);
            if (p.S_out)
                p.S_out[(static_cast<size_t>(b) * p.K + q) * h + j] = sn;
            if (p.s_hl) {  // operand planes for the matrix-core state dots (row stride ldw)
                const uint32_t hi = bf16_rne_bits(sn);
                const size_t o = static_cast<size_t>(b) * p.ldw + j;
                p.s_hl[o] = static_cast<uint16_t>(hi);
                p.s_hl[static_cast<size_t>(p.maxB) * p.ldw + o] =
                    static_cast<uint16_t>(bf16_rne_bits(sn - __uint_as_float(hi << 16)));
            }
        }
    }
}

// ---- phase: dot products over S_q: u_q and q for the next step ------------------------
// Rows m < r are W1_S rows (u_q = SiLU(A_H[q] + W1_S S_q)); rows r.. are W_hh
// rows (W_hh S_q + b_hh, used by the next gate update).  Rows are spread over
// the waves of the grid; each wave dots its row with S_q of every batch row.
// In the persistent launch every block first computes all of S_q itself into
// LDS from its own copy of S_{q-1} (the gate update is cheap), so the state
// never crosses blocks; block 0 also publishes S_q and tokens[:, q-1].  In
// stepwise launches S_q comes from the preceding phase_update.
//
// The weight rows and the A_H entries a wave needs are the same at every
// position, so the persistent kernel copies them into LDS once per launch
// (state_cache_load); the q values of the gate update are loaded before the
// barrier that precedes the phase (state_prefetch).
constexpr int SP_EL = 1024 / NT;  // gate-update elements per thread whose q values are prefetched

struct StatePre {
    float qv[SP_EL][3];
};

__device__ inline int state_rows(const Params &p) { return p.r + 3 * p.h; }

template <typename WT>
__device__ inline size_t state_row_off(const Params &p, int m)
{
    return m < p.r ? static_cast<size_t>(m) * (p.d + p.h) + p.d : static_cast<size_t>(m - p.r) * p.h;
}

// Loads for phase_state(q) that depend on nothing computed after the previous
// barrier: the q values of this thread's first gate-update elements.
template <typename WT>
__device__ __forceinline__ void state_prefetch(const Params &p, int q, StatePre &pre)
{
    const int h = p.h;
    const int nb0 = p.B < BC ? p.B : BC;
#pragma unroll
    for (int e = 0; e < SP_EL; ++e) {
        const int i = threadIdx.x + e * NT;
        if (i < nb0 * h) {
            const float *qv = q_slot(p, q) + static_cast<size_t>(i / h) * 3 * h;
            const int j = i % h;
            pre.qv[e][0] = xld(&qv[j]);
            pre.qv[e][1] = xld(&qv[h + j]);
            pre.qv[e][2] = xld(&qv[2 * h + j]);
        }
    }
}

// Rows of the state phase handled by each wave of a persistent launch (at most), and
// the LDS it takes to keep them: the rows (WT) plus their A_H entries for every
// position and batch row (u rows only).
__host__ __device__ inline int state_rows_per_wave(int r, int h, int nblk)
{
    return (r + 3 * h + nblk * NWAVE - 1) / (nblk * NWAVE);
}

// Dot rows of the state phase (the W1_S rows m < r, giving u, then the W_hh rows,
// giving q).  Block blk owns the rows m = blk + t nblk, t = 0 .. T-1, its U u rows
// first, so the u rows are spread over all blocks.  The u rows go to waves 0, 1, ...
// in turn (slot k of wave w: t = w + k NWAVE).  The q rows go, DOT_RG at a time (one
// dot group), to the waves that hold no u row, so a wave computing a u row -- the
// value the next W2 phase waits for -- gets no q row when the others can take them
// all; when every wave holds a u row, or this would give a wave more than
// state_rows_per_wave rows, or the caller asks for it (`group` false), the q rows go
// round-robin instead (q row t goes to wave t mod NWAVE).
constexpr int DOT_RG = 4;
struct DotRows {
    int blk, nblk;
    int U, Q;     // the block's u and q rows
    int nq, qw0;  // q rows go to waves qw0, qw0 + 1, ... (mod NWAVE), nq of them
    int rg;       // q rows per chunk: DOT_RG, or 1 (round-robin)
};
__host__ __device__ inline int dot_u_rows(const DotRows &d, int w)
{
    return w < d.U ? (d.U - w + NWAVE - 1) / NWAVE : 0;
}
// position of wave w among the q waves, or nq when it takes none
__host__ __device__ inline int dot_q_index(const DotRows &d, int w)
{
    const int iw = (w - d.qw0 + NWAVE) % NWAVE;
    return iw < d.nq ? iw : d.nq;
}
__host__ __device__ inline int dot_rows_of(const DotRows &d, int w)
{
    const int iw = dot_q_index(d, w), nc = (d.Q + d.rg - 1) / d.rg;
    int nqr = 0;
    if (iw < d.nq && iw < nc) {
        nqr = (nc - iw + d.nq - 1) / d.nq * d.rg;
        if ((nc - 1 - iw) % d.nq == 0)
            nqr -= nc * d.rg - d.Q;  // this wave has the last, partial chunk
    }
    return dot_u_rows(d, w) + nqr;
}
__host__ __device__ inline DotRows dot_rows(int r, int R, int blk, int nblk, bool group = true)
{
    DotRows d;
    d.blk = blk;
    d.nblk = nblk;
    const int T = blk < R ? (R - blk + nblk - 1) / nblk : 0;
    d.U = blk < r ? (r - blk + nblk - 1) / nblk : 0;
    d.Q = T - d.U;
    bool grouped = group && d.U < NWAVE;
    if (grouped) {
        d.nq = NWAVE - d.U;
        d.qw0 = d.U;
        d.rg = DOT_RG;
        const int cap = state_rows_per_wave(r, (R - r) / 3, nblk);
        for (int w = 0; w < NWAVE; ++w)
            grouped = grouped && dot_rows_of(d, w) <= cap;
    }
    if (!grouped) {
        d.nq = NWAVE;
        d.qw0 = d.U % NWAVE;
        d.rg = 1;
    }
    return d;
}
// row m of slot k of wave w, or -1
__host__ __device__ inline int dot_row(const DotRows &d, int w, int k)
{
    const int nu = dot_u_rows(d, w);
    int t;
    if (k < nu) {
        t = w + k * NWAVE;
    } else {
        const int iw = dot_q_index(d, w), kq = k - nu;
        const int tq = ((kq / d.rg) * d.nq + iw) * d.rg + kq % d.rg;
        if (iw >= d.nq || tq >= d.Q)
            return -1;
        t = d.U + tq;
    }
    return d.blk + t * d.nblk;
}
// (then each wave's row table: its rows' ids, slots past its last -1, its u row count
// and its row count, NWAVE x (rpw + 2) ints)
__host__ __device__ inline int state_cache_floats(int r, int h, int K, int nblk, int wbytes)
{
    const int rpw = state_rows_per_wave(r, h, nblk);
    return NWAVE * rpw * (h * wbytes / 4 + K * BC) + NWAVE * (rpw + 2);
}

// Once per persistent launch, after the prologue barrier: each wave copies its
// state rows and their A_H entries into LDS.
// with_ah = false leaves the A_H entries to ah_local_to_cache.
template <typename WT>
__device__ __forceinline__ void state_cache_load(const Params &p, int blk, int nblk, float *cache, bool with_ah = true)
{
    constexpr int EPC = WT16<WT>::EPC;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = p.h, R = state_rows(p), rpw = state_rows_per_wave(p.r, h, nblk);
    const int row_words = h * static_cast<int>(sizeof(WT)) / 4;
    uint4 *wc = reinterpret_cast<uint4 *>(cache);
    float *ac = cache + NWAVE * rpw * row_words;
    constexpr int CPL = (2048 / EPC + 63) / 64;  // 16-byte chunks per lane of a row at the largest h
    constexpr int RB = 16 / CPL;                 // rows whose loads go out together (16 registers of 16 bytes)
    const DotRows dr = dot_rows(p.r, R, blk, nblk);
    const int nchk = h / EPC, nrw = dot_rows_of(dr, wave);
    int *tab = reinterpret_cast<int *>(ac + NWAVE * rpw * p.K * BC) + wave * (rpw + 2);
    if (lane < rpw)
        tab[lane] = lane < nrw ? dot_row(dr, wave, lane) : -1;
    if (lane == 0) {
        tab[rpw] = dot_u_rows(dr, wave);
        tab[rpw + 1] = nrw;
    }
    for (int k0 = 0; k0 < nrw; k0 += RB) {
        // the loads of RB rows first, every one issued (rows past the wave's last and
        // chunks past h read the group's first row / chunk 0), then the LDS stores
        uint4 v[RB][CPL];
#pragma unroll
        for (int kk = 0; kk < RB; ++kk) {
            const int k = k0 + kk;
            const int mc = dot_row(dr, wave, k < nrw ? k : k0);
            const void *W = mc < p.r ? p.W1 : p.W_hh;
            const size_t off = state_row_off<WT>(p, mc);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ch = lane + c * 64;
                v[kk][c] = ld16<WT>(W, off + static_cast<size_t>(ch < nchk ? ch : 0) * EPC);
            }
        }
#pragma unroll
        for (int kk = 0; kk < RB; ++kk) {
            const int k = k0 + kk;
            if (k < nrw) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = lane + c * 64;
                    if (ch < nchk)
                        wc[(wave * rpw + k) * nchk + ch] = v[kk][c];
                }
            }
        }
    }
    for (int k = 0; k < nrw; ++k) {
        const int m = dot_row(dr, wave, k);
        if (m < p.r) {
            for (int i = lane; with_ah && i < p.K * p.B; i += 64) {
                const int qq = i / p.B, b = i % p.B;
                ac[((wave * rpw + k) * p.K + qq) * BC + b] = xld(&p.A_H[(static_cast<size_t>(b) * p.K + qq) * p.r + m]);
            }
        } else if (lane == 0) {
            // W_hh rows need no A_H entries: their slot holds the b_hh entry instead
            ac[(wave * rpw + k) * p.K * BC] = p.b_hh ? WT16<WT>::one(p.b_hh, m - p.r) : 0.f;
        }
    }
}

// A_H entries of the block's u rows for batch row 0, computed by the block itself
// into the owner waves' cache slots (persistent launch at B = 1: each u row has
// one owner wave, so nothing crosses blocks): A_H[0][i][m] = W1[m][0:d] . H[0][i].
// Wave w takes the positions i = w, w + NWAVE, ...  Each lane keeps the partial
// sums of the AH_LANES / 64 lanes at its index in the A_H sum layout, over the
// same chunks in the same order, and reduces them in the same order, so the
// entries equal phase_ah's bit for bit.  All loads of a row are issued
// before the first product.
template <typename WT>
__device__ __forceinline__ void ah_local_to_cache(const Params &p, int blk, int nblk, float *cache)
{
    constexpr int EPC = WT16<WT>::EPC;
    constexpr int PW = MAXK / NWAVE;   // positions per wave
    constexpr int KK = 2;              // AH_LANES-chunk strides loaded together
    constexpr int VW = AH_LANES / 64;  // waves of the sum layout
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = p.h, d = p.d, rpw = state_rows_per_wave(p.r, h, nblk);
    const int nch = d / EPC;
    float *ac = cache + NWAVE * rpw * (h * static_cast<int>(sizeof(WT)) / 4);
    const DotRows dr = dot_rows(p.r, state_rows(p), blk, nblk);  // as state_cache_load
    for (int ow = 0; ow < NWAVE; ++ow) {
        for (int k = 0; k < dot_u_rows(dr, ow); ++k) {
            const int m = dot_row(dr, ow, k);
            float acc[PW][VW];
#pragma unroll
            for (int t = 0; t < PW; ++t)
#pragma unroll
                for (int vw = 0; vw < VW; ++vw)
                    acc[t][vw] = 0.f;
            for (int c0 = 0; c0 < nch; c0 += KK * AH_LANES) {
                uint4 wv[KK][VW], xv[KK][VW][PW];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                    for (int vw = 0; vw < VW; ++vw) {
                        // every load is issued (chunks past d and positions past K read
                        // chunk 0 / position 0 and are not multiplied), so they all go out
                        // before the first product instead of one branch at a time
                        const int c = c0 + kk * AH_LANES + vw * 64 + lane;
                        const int cc = c < nch ? c : 0;
                        wv[kk][vw] = ld16<WT>(p.W1, static_cast<size_t>(m) * (d + h) + static_cast<size_t>(cc) * EPC);
#pragma unroll
                        for (int t = 0; t < PW; ++t) {
                            const int ii = wave + t * NWAVE < p.K ? wave + t * NWAVE : 0;
                            xv[kk][vw][t] = ld16<WT>(p.H, static_cast<size_t>(ii) * d + static_cast<size_t>(cc) * EPC);
                        }
                    }
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                    for (int vw = 0; vw < VW; ++vw) {
                        const int c = c0 + kk * AH_LANES + vw * 64 + lane;
                        if (c < nch) {
                            float w[EPC];
                            WT16<WT>::unpack(wv[kk][vw], w);
#pragma unroll
                            for (int t = 0; t < PW; ++t) {
                                if (wave + t * NWAVE < p.K) {
                                    float x[EPC];
                                    WT16<WT>::unpack(xv[kk][vw][t], x);
#pragma unroll
                                    for (int e = 0; e < EPC; ++e)
                                        acc[t][vw] = fmaf(w[e], x[e], acc[t][vw]);
                                }
                            }
                        }
                    }
            }
#pragma unroll
            for (int t = 0; t < PW; ++t) {
                const int i = wave + t * NWAVE;
                if (i < p.K) {
                    float sum = 0.f;
#pragma unroll
                    for (int vw = 0; vw < VW; ++vw)
                        sum += wave_sum(acc[t][vw]);
                    if (lane == 0)
                        ac[((ow * rpw + k) * p.K + i) * BC] = sum;
                }
            }
        }
    }
}

// A launch with B rows writes no tagged u words of rows B..min(BC, maxB)-1.  At
// its end they get the launch's last tag, so every word holds a tag at most one
// launch old: the tags a later launch polls for all lie ahead of it, whatever
// its B.
__device__ inline void utag_refresh(const Params &p, int blk, int nblk, unsigned last_tag)
{
    const int rows = (p.maxB < BC ? p.maxB : BC) - p.B;
    if (rows <= 0)
        return;
    const uint32_t t16 = (last_tag & 0xFFFFu) << 16;
    const size_t base = static_cast<size_t>(p.B) * p.r, n = static_cast<size_t>(rows) * p.r;
    const size_t plane = static_cast<size_t>(p.maxB) * p.r;
    for (size_t i = static_cast<size_t>(blk) * NT + threadIdx.x; i < n; i += static_cast<size_t>(nblk) * NT) {
        __hip_atomic_store(gmem(&p.utag[base + i]), t16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(gmem(&p.utag[plane + base + i]), t16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// With p.utag (resident launch) u_q is published as tagged operand words
// instead of u_buf: (tag << 16) | bf16 bits, hi part in plane 0 and lo part
// (u - hi) in plane 1; readers poll for `tag`.
struct NoHook {
    __device__ void operator()() const {}
};

// after_gate() runs between the gate update and the dot products (a persistent
// kernel issues its long loads there, after the gate update's latency-critical ones).
template <typename WT, typename AfterGate = NoHook>
__device__ __forceinline__ void phase_state(const Params &p, int blk, int nblk, int q, float *smem, float *S_lds,
                                            const StatePre *pre, const float *cache, bool cached,
                                            const int *atok = nullptr, unsigned tag = 0,
                                            AfterGate after_gate = AfterGate())
{
    constexpr int EPC = WT16<WT>::EPC;
    const int h = p.h, h3 = 3 * h, r = p.r;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float *qn_all = q_slot(p, q + 1);
    const int R = state_rows(p), nch = h / EPC;
    const int tslot = (q - 1) * 32 + 16;
    DH_TRACE(tslot);
    for (int b0 = 0; b0 < p.B; b0 += BC) {
        const int nb = (p.B - b0) < BC ? (p.B - b0) : BC;
        if (p.persistent) {
            // B <= BC: one chunk.  Each thread takes the GRU input token itself
            // (atok entries were written before the argmax barrier's last block
            // sync); the state never leaves the block, so S_buf is not written.
            // Elements go in batches of SP_EL per thread: every load of a batch (the
            // gate inputs, q, the previous state) is issued before any is used, at
            // clamped indices for elements past the end, so the batch costs one
            // memory round trip instead of one per element.  The first batch takes
            // the q values prefetched before the barrier when given.
            DH_TRACE(tslot + 1);
            const int ne = nb * h;
            // the GRU input token of each row, once, into LDS: the batch loads below
            // then depend on an LDS read only
            // (the argmax tokens of a persistent launch, atok, are visible to the whole
            // block since the barrier that delivered them: no copy and no block sync)
            const int *tokl = atok;
            if (!(atok && q > 0 && !p.teacher)) {
                int *tl = reinterpret_cast<int *>(smem + smem_off_tok());
                if (p.P && static_cast<int>(threadIdx.x) < nb)
                    tl[threadIdx.x] = gru_input_token(p, q, b0 + threadIdx.x, atok);
                __syncthreads();
                tokl = tl;
            }
            // (one batch row: element i is entry i of row b0, no division by h)
            const bool one = nb == 1;
            // qmode 0: q prefetched before the barrier (first batch), 1: q = b_hh (zero
            // initial state), 2: q loaded; one branch per batch, none per element
            // gmode 0: g from the folded table's row (p.P), 1: g words (p.gtag), 2: g_buf.
            // Both modes are template arguments, so each variant holds only its own
            // loaded values in registers.
            auto batch = [&](auto qmode, auto gmode, int i0) {
                constexpr int QM = decltype(qmode)::value, GM = decltype(gmode)::value;
                float gv[SP_EL][3], qv[SP_EL][3], sp[SP_EL];
                uint64_t gt[GM == 1 ? SP_EL : 1][3];  // tagged g words (p.gtag)
#pragma unroll
                for (int e = 0; e < SP_EL; ++e) {
                    const int i = i0 + e * NT;
                    const int ic = i < ne ? i : 0;
                    const int bb = one ? 0 : ic / h, j = one ? ic : ic % h, b = b0 + bb;
                    // (an element past the end reads no S_lds entry: that entry belongs to
                    // another thread, which may be writing it)
                    sp[e] = (q == 0) ? state_prev(p, 0, b, j) : (i < ne ? S_lds[bb * h + j] : 0.f);
                    if constexpr (GM == 0) {
                        // (global loads: as flat loads they would also hold up the LDS reads)
                        const auto *prow = gmem(p.P + static_cast<size_t>(tokl[bb]) * h3);
                        gv[e][0] = prow[j];
                        gv[e][1] = prow[h + j];
                        gv[e][2] = prow[2 * h + j];
                    } else if constexpr (GM == 1) {
                        const uint64_t *g = p.gtag + static_cast<size_t>(b) * h3;
                        gt[e][0] = ld_agent_u64(&g[j]);
                        gt[e][1] = ld_agent_u64(&g[h + j]);
                        gt[e][2] = ld_agent_u64(&g[2 * h + j]);
                    } else {
                        const float *g = p.g_buf + static_cast<size_t>(b) * h3;
                        gv[e][0] = xld(&g[j]);
                        gv[e][1] = xld(&g[h + j]);
                        gv[e][2] = xld(&g[2 * h + j]);
                    }
                    if constexpr (QM == 0) {
                        qv[e][0] = pre->qv[e][0];
                        qv[e][1] = pre->qv[e][1];
                        qv[e][2] = pre->qv[e][2];
                    } else if constexpr (QM == 1) {
                        // W_hh S_init + b_hh with S_init = 0 is b_hh itself
                        qv[e][0] = bias_hh(p, j);
                        qv[e][1] = bias_hh(p, h + j);
                        qv[e][2] = bias_hh(p, 2 * h + j);
                    } else {
                        const float *qq = q_slot(p, q) + static_cast<size_t>(b) * h3;
                        qv[e][0] = xld(&qq[j]);
                        qv[e][1] = xld(&qq[h + j]);
                        qv[e][2] = xld(&qq[2 * h + j]);
                    }
                }
                if (i0 == static_cast<int>(threadIdx.x))
                    DH_TRACE_LANDED(tslot + 9);
                if constexpr (GM == 1) {
                    // the g words of this step carry `tag` once their producers wrote them:
                    // while any does not, re-read all of them (one round trip per round)
                    unsigned spins = 0;
                    for (;;) {
                        uint32_t stale = 0;  // bit 3 e + c: word c of element e
#pragma unroll
                        for (int x = 0; x < 3 * SP_EL; ++x)
                            stale |= static_cast<uint32_t>(i0 + (x / 3) * NT < ne &&
                                                           static_cast<unsigned>(gt[x / 3][x % 3] >> 32) != tag)
                                     << x;
                        if (!stale)
                            break;
                        if (++spins > p.spin_limit) {
                            __hip_atomic_fetch_or(gmem(p.flags), 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                        // (short loops with constant trips: the compiler unrolls them by itself)
                        for (int e = 0; e < SP_EL; ++e) {
                            const int i = i0 + e * NT;
                            const int ic = i < ne ? i : 0;
                            const uint64_t *g =
                                p.gtag + static_cast<size_t>(b0 + (one ? 0 : ic / h)) * h3 + (one ? ic : ic % h);
                            for (int c = 0; c < 3; ++c)
                                gt[e][c] = ld_agent_u64(&g[c * h]);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < SP_EL; ++e)
#pragma unroll
                        for (int c = 0; c < 3; ++c)
                            gv[e][c] = __uint_as_float(static_cast<uint32_t>(gt[e][c]));
                }
#pragma unroll
                for (int e = 0; e < SP_EL; ++e) {
                    const int i = i0 + e * NT;
                    if (i < ne) {
                        const int bb = one ? 0 : i / h, j = one ? i : i % h, b = b0 + bb;
                        // the cell of gate_update, on the values loaded above
                        const float rg = sigmoidf_(gv[e][0] + qv[e][0]);
                        const float zg = sigmoidf_(gv[e][1] + qv[e][1]);
                        const float ng = tanhf_(gv[e][2] + rg * qv[e][2]);
                        const float sn = (1.f - zg) * ng + zg * sp[e];
                        S_lds[bb * h + j] = sn;  // each thread reads only the entries it writes
                        if (blk == 0 && p.S_out)
                            gmem(p.S_out)[(static_cast<size_t>(b) * p.K + q) * h + j] = sn;
                    }
                }
            };
            const bool use_pre = pre && b0 == 0, qbias = q == 0 && !p.S_init;
            auto by_g = [&](auto qmode, int i0) {
                if (p.P)
                    batch(qmode, std::integral_constant<int, 0>(), i0);
                else if (p.gtag)
                    batch(qmode, std::integral_constant<int, 1>(), i0);
                else
                    batch(qmode, std::integral_constant<int, 2>(), i0);
            };
            for (int i0 = threadIdx.x, it = 0; i0 < ne; i0 += SP_EL * NT, ++it) {
                if (use_pre && it == 0)
                    by_g(std::integral_constant<int, 0>(), i0);
                else if (qbias)
                    by_g(std::integral_constant<int, 1>(), i0);
                else
                    by_g(std::integral_constant<int, 2>(), i0);
            }
        } else {
            __syncthreads();  // S_lds of the previous chunk is no longer read
            for (int i = threadIdx.x; i < nb * h; i += NT)
                S_lds[i] = xld(&S_slot(p, q)[static_cast<size_t>(b0) * h + i]);
        }
        DH_TRACE(tslot + 2);
        after_gate();
        __syncthreads();
        DH_TRACE(tslot + 3);
        // dot rows of this wave: slot k holds row dot_row(dr, wave, k); when `cached`
        // (persistent launch) the row and its A_H entries come from LDS at `cache`.  Rows go in
        // groups of up to RG: the S chunks are read once per group and the sums are
        // reduced together (each row's sum is formed in the same order as alone).
        // The wave's u rows (m < r) form the first groups, so u is published before
        // the q rows are computed.
        constexpr int RG = DOT_RG;
        const int rpw = state_rows_per_wave(r, h, nblk);
        const uint4 *wc = reinterpret_cast<const uint4 *>(cache);
        const float *ac = cache + NWAVE * rpw * (h * static_cast<int>(sizeof(WT)) / 4);
        // this wave's u rows and all its rows: from its row table when cached
        const int *tab = reinterpret_cast<const int *>(ac + NWAVE * rpw * p.K * BC) + wave * (rpw + 2);
        DotRows dr{};
        int ku, nrw;
        if (cached) {
            ku = tab[rpw];
            nrw = tab[rpw + 1];
        } else {
            dr = dot_rows(r, R, blk, nblk);
            ku = dot_u_rows(dr, wave);
            nrw = dot_rows_of(dr, wave);
        }
#pragma unroll 1
        for (int k0 = 0, kend = 0; k0 < nrw; k0 = kend) {
            kend = k0 < ku ? (ku < k0 + RG ? ku : k0 + RG) : (nrw < k0 + RG ? nrw : k0 + RG);
#pragma unroll 1
            for (int bb = 0; bb < nb; ++bb) {
                const int b = b0 + bb;
                const float *s = S_lds + bb * h;
                float acc[RG];
#pragma unroll
                for (int j = 0; j < RG; ++j)
                    acc[j] = 0.f;
                if (k0 == 0 && bb == 0)
                    DH_TRACE(tslot + 7);
#pragma unroll 2
                for (int ch = lane; ch < nch; ch += 64) {
                    float x[EPC];
#pragma unroll
                    for (int i2 = 0; i2 < EPC; ++i2)
                        x[i2] = s[ch * EPC + i2];
#pragma unroll
                    for (int j = 0; j < RG; ++j) {
                        const int k = k0 + j;
                        if (k < kend) {  // (slots below the wave's row count all hold rows)
                            const int m = cached ? 0 : dot_row(dr, wave, k);
                            const uint4 wq = cached ? wc[(wave * rpw + k) * nch + ch]
                                                    : ld16<WT>(m < r ? p.W1 : p.W_hh,
                                                               state_row_off<WT>(p, m) + static_cast<size_t>(ch) * EPC);
                            acc[j] = dot_chunk<WT>(wq, x, acc[j]);
                        }
                    }
                }
                if (k0 == 0 && bb == 0)
                    DH_TRACE(tslot + 8);
                float dot[RG];
#pragma unroll
                for (int j = 0; j < RG; ++j)
                    dot[j] = wave_sum(acc[j]);
                if (k0 == 0 && bb == 0)
                    DH_TRACE(tslot + 5);
#pragma unroll
                for (int j = 0; j < RG; ++j) {
                    const int k = k0 + j;
                    if (lane != 0 || k >= kend)
                        continue;
                    const int m = cached ? tab[k] : dot_row(dr, wave, k);
                    if (m < r) {
                        const float ah = cached ? ac[((wave * rpw + k) * p.K + q) * BC + b]
                                                : xld(&p.A_H[(static_cast<size_t>(b) * p.K + q) * r + m]);
                        const float a = ah + dot[j];
                        const float u = a * sigmoidf_(a);
                        if (p.utag) {
                            const uint32_t hi = bf16_rne_bits(u);
                            const uint32_t lo = bf16_rne_bits(u - __uint_as_float(hi << 16));
                            const uint32_t t16 = (tag & 0xFFFFu) << 16;
                            const size_t o = static_cast<size_t>(b) * r + m;
                            __hip_atomic_store(gmem(&p.utag[o]), t16 | hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            __hip_atomic_store(gmem(&p.utag[static_cast<size_t>(p.maxB) * r + o]), t16 | lo,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        } else {
                            xst(&p.u_buf[static_cast<size_t>(b) * r + m], u);
                        }
                        if (p.u_out)
                            gmem(p.u_out)[(static_cast<size_t>(b) * p.K + q) * r + m] = u;
                    } else {
                        const float bias =
                            cached ? ac[(wave * rpw + k) * p.K * BC] : (p.b_hh ? WT16<WT>::one(p.b_hh, m - r) : 0.f);
                        xst(&qn_all[static_cast<size_t>(b) * h3 + (m - r)], dot[j] + bias);
                    }
                }
                if (k0 == 0 && bb == 0)
                    DH_TRACE(tslot + 6);
            }
        }
    }
    DH_TRACE(tslot + 4);
}

// Epilogue of the W2 phase for batch rows b0..b0+nb-1 of block blk: lbuf holds
// the block's W2 u dot products; add L_base (the first LB values per thread of
// batch row b0 come prefetched in lbv), store L_final, reduce the block's
// greedy argmax key and publish it (LDS local_keys, or the global partial slot).
constexpr int W2_LB = 1024 / NT;
__device__ __forceinline__ void w2_epilogue(const Params &p, int blk, int nblk, int pos, float *smem, int b0, int nb,
                                            const float (&lbv)[W2_LB], uint64_t *local_keys)
{
    const long long v0 = static_cast<long long>(p.V) * blk / nblk;
    const int n = static_cast<int>(static_cast<long long>(p.V) * (blk + 1) / nblk - v0);
    const int rows_cap = lbuf_stride(p.V, nblk);
    uint64_t *kred = reinterpret_cast<uint64_t *>(smem + 256);
    const float *lbuf = smem + smem_off_lbuf(p.r);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = blk % NG;
    for (int bb = 0; bb < nb; ++bb) {
        const int b = b0 + bb;
        const size_t lb = (static_cast<size_t>(b) * p.K + pos) * p.V + v0;
        float *lf = p.L_final ? p.L_final + (static_cast<size_t>(b) * p.K + pos) * p.V + v0 : nullptr;
        uint64_t best = 0;
        for (int i = threadIdx.x, e = 0; i < n; i += NT, ++e) {
            float base_logit = 0.f;
#pragma unroll
            for (int ee = 0; ee < W2_LB; ++ee)
                if (bb == 0 && e == ee)
                    base_logit = lbv[ee];
            if (bb != 0 || e >= W2_LB)
                base_logit = lbase_at(p, lb + i);
            const float v = base_logit + lbuf[bb * rows_cap + i];
            if (lf)
                lf[i] = v;
            const uint64_t key = argmax_key(v, static_cast<uint32_t>(v0 + i));
            best = key > best ? key : best;
        }
        best = wave_max_u64(best);
        if (lane == 0)
            kred[wave] = best;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint64_t m = 0;
            for (int w = 0; w < NWAVE; ++w)
                m = kred[w] > m ? kred[w] : m;
            if (local_keys)
                local_keys[bb] = m ? (m & KEY_ORD_MASK) | (KEY_IDX_MASK - key_index(m)) : 0ull;
            else
                __hip_atomic_fetch_max(gmem(key_slot(p, pos, g, b)), m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    }
}

// L_base values of batch row b0 this thread adds in the epilogue, loaded early.
__device__ __forceinline__ void w2_lbase_prefetch(const Params &p, int blk, int nblk, int pos, int b0,
                                                  float (&lbv)[W2_LB])
{
    const long long v0 = static_cast<long long>(p.V) * blk / nblk;
    const int n = static_cast<int>(static_cast<long long>(p.V) * (blk + 1) / nblk - v0);
#pragma unroll
    for (int e = 0; e < W2_LB; ++e) {
        const int i = threadIdx.x + e * NT;
        lbv[e] = i < n ? lbase_at(p, (static_cast<size_t>(b0) * p.K + pos) * p.V + v0 + i) : 0.f;
    }
}

// ---- phase: L_p = L_base_p + W2 u_p and the greedy argmax ------------------------
// Block blk owns vocabulary rows [v0, v1).  A wave reads 64/LPR rows at a time,
// LPR lanes per row, each lane NL 16-byte chunks (coalesced: the LPR lanes of a
// row read LPR consecutive chunks).  Row partial sums are combined with xor
// shuffles inside the LPR lanes.  Two batches of two row groups are kept in
// flight.  The block's dot products for up to BC batch rows go to LDS; the
// epilogue adds L_base, stores L_final, reduces the block's argmax key and
// folds it into the partial slot of group blk % NG with an atomic max.
template <typename WT, int LPR, int NL>
struct W2Rows {
    static constexpr int RPW = 64 / LPR;  // rows per wave per group
    static constexpr int UG = 1;          // row groups per batch

    __device__ static inline void load(uint4 (&w)[UG][NL], const void *W2, int r, long long v0, int n, int base,
                                       int rw, int sub, int stride)
    {
#pragma unroll
        for (int ug = 0; ug < UG; ++ug) {
            const int row = base + ug * stride + rw;
            if (row < n) {
                const char *rp = static_cast<const char *>(W2) + static_cast<size_t>(v0 + row) * r * sizeof(WT);
#pragma unroll
                for (int q = 0; q < NL; ++q)
                    w[ug][q] = *reinterpret_cast<const uint4 *>(rp + static_cast<size_t>(q * LPR + sub) * 16);
            } else {
#pragma unroll
                for (int q = 0; q < NL; ++q)
                    w[ug][q] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }

    __device__ static inline void compute(const uint4 (&w)[UG][NL], const float *u_lds, float *lbuf, int r,
                                          int rows_cap, int nb, int n, int base, int rw, int sub, int stride)
    {
        constexpr int EPC = WT16<WT>::EPC;
#pragma unroll
        for (int ug = 0; ug < UG; ++ug) {
            const int row = base + ug * stride + rw;
            for (int bb = 0; bb < nb; ++bb) {
                float acc = 0.f;
#pragma unroll
                for (int q = 0; q < NL; ++q)
                    acc = dot_chunk<WT>(w[ug][q], u_lds + bb * r + (q * LPR + sub) * EPC, acc);
                acc = group_sum<LPR>(acc);
                if (sub == 0 && row < n)
                    lbuf[bb * rows_cap + row] = acc;
            }
        }
    }
};

template <typename WT, int LPR, int NL>
struct W2Pre {
    uint4 w[W2Rows<WT, LPR, NL>::UG][NL];
};

// First batch of this wave's W2 rows for position-independent reuse: the
// persistent kernel issues it before the barrier that precedes phase_w2.
template <typename WT, int LPR, int NL>
__device__ __forceinline__ void w2_prefetch(const Params &p, int blk, int nblk, W2Pre<WT, LPR, NL> &pre)
{
    using R = W2Rows<WT, LPR, NL>;
    const long long v0 = static_cast<long long>(p.V) * blk / nblk;
    const int n = static_cast<int>(static_cast<long long>(p.V) * (blk + 1) / nblk - v0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    R::load(pre.w, p.W2, p.r, v0, n, wave * R::RPW, lane / LPR, lane % LPR, NWAVE * R::RPW);
}

// With local_keys (persistent launch), the block's argmax key of each batch row
// goes to local_keys[bb] in LDS (18-bit index form, see grid_argmax_sync)
// instead of the global partial slots.
template <typename WT, int LPR, int NL>
__device__ __forceinline__ void phase_w2(const Params &p, int blk, int nblk, int pos, float *smem, const W2Pre<WT, LPR, NL> *pre,
                         uint64_t *local_keys)
{
    using R = W2Rows<WT, LPR, NL>;
    constexpr int RPW = R::RPW;
    const int r = p.r;
    const long long v0 = static_cast<long long>(p.V) * blk / nblk;
    const long long v1 = static_cast<long long>(p.V) * (blk + 1) / nblk;
    const int n = static_cast<int>(v1 - v0);
    const int rows_cap = lbuf_stride(p.V, nblk);
    float *u_lds = smem + smem_off_u();
    float *lbuf = smem + smem_off_lbuf(r);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPR, rw = lane / LPR;
    const int stride = NWAVE * RPW;   // rows between consecutive groups of one wave
    const int bstride = R::UG * stride;

    for (int b0 = 0; b0 < p.B; b0 += BC) {
        const int nb = (p.B - b0) < BC ? (p.B - b0) : BC;
        uint4 wa[R::UG][NL], wb[R::UG][NL];
        int base = wave * RPW;
        if (pre && b0 == 0) {
#pragma unroll
            for (int ug = 0; ug < R::UG; ++ug)
#pragma unroll
                for (int q = 0; q < NL; ++q)
                    wa[ug][q] = pre->w[ug][q];
        } else {
            R::load(wa, p.W2, r, v0, n, base, rw, sub, stride);
        }
        float lbv[W2_LB];
        w2_lbase_prefetch(p, blk, nblk, pos, b0, lbv);
        __syncthreads();
        for (int i = threadIdx.x; i < nb * r; i += NT)
            u_lds[i] = xld(&p.u_buf[static_cast<size_t>(b0) * r + i]);
        __syncthreads();
        while (base < n) {
            const int nbase = base + bstride;
            if (nbase < n)
                R::load(wb, p.W2, r, v0, n, nbase, rw, sub, stride);
            R::compute(wa, u_lds, lbuf, r, rows_cap, nb, n, base, rw, sub, stride);
            if (nbase >= n)
                break;
            const int nnbase = nbase + bstride;
            if (nnbase < n)
                R::load(wa, p.W2, r, v0, n, nnbase, rw, sub, stride);
            R::compute(wb, u_lds, lbuf, r, rows_cap, nb, n, nbase, rw, sub, stride);
            base = nnbase;
        }
        __syncthreads();
        w2_epilogue(p, blk, nblk, pos, smem, b0, nb, lbv, local_keys);
    }
}

// ---- W2 phase with the block's W2 slice resident on chip (bf16, r = 32 * KS) -------
// The block's rows [v0, v1) form 16-row tiles.  Tile t is held by wave t % NWAVE:
// its first RT tiles in registers (wt), the rest in LDS (`tl`), all loaded once
// per launch.  Per position each wave multiplies its tiles with u on the matrix
// cores (v_mfma_f32_16x16x32_bf16): A = 16 W2 rows x 32 of r, B = 32 of r x 16
// columns, where column b (< 8) carries bf16(u_b) and column 8 + b carries
// bf16(u_b - bf16(u_b)) (the u operand planes written by phase_state); adding
// the two result columns gives W2 u_b with float32-level accuracy.  Lane l
// holds A row l%16 and B column l%16 at r offsets (l/16)*8 .. +8 of each
// 32-wide step, and result rows (l/16)*4 + i of column l%16.  The epilogue
// (L_base add, L_final store, greedy argmax) runs on the result registers.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int RT, int KS>
struct W2Resident {
    uint4 wt[RT][KS];
};

// A operand of tile t, step kk for this lane (zero beyond the block's rows).
template <int KS>
__device__ inline uint4 w2_tile_chunk(const Params &p, long long v0, int n, int t, int kk)
{
    const int lane = threadIdx.x & 63;
    const int row = t * 16 + (lane & 15);
    if (row >= n)
        return make_uint4(0u, 0u, 0u, 0u);
    return ld16<bf16s>(p.W2, static_cast<size_t>(v0 + row) * (32 * KS) + kk * 32 + (lane >> 4) * 8);
}

template <int RT, int KS>
__device__ __forceinline__ void w2_resident_load(const Params &p, int blk, int nblk, W2Resident<RT, KS> &res,
                                                 uint4 *tl)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long v0 = vslice_lo(p.V, blk, nblk);
    const int n = vslice_lo(p.V, blk + 1, nblk) - static_cast<int>(v0);
    const int T = (n + 15) / 16;
#pragma unroll
    for (int j = 0; j < RT; ++j) {
        const int t = wave + j * NWAVE;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            res.wt[j][kk] = t < T ? w2_tile_chunk<KS>(p, v0, n, t, kk) : make_uint4(0u, 0u, 0u, 0u);
    }
    for (int t = NWAVE * RT + wave; t < T; t += NWAVE) {
        const int slot = t - NWAVE * RT;
        for (int kk = 0; kk < KS; ++kk)
            tl[(slot * KS + kk) * 64 + lane] = w2_tile_chunk<KS>(p, v0, n, t, kk);
    }
}

// The block's L_base slice of position pos ([b][i] at lbuf[b * rows_cap + i])
// copied into LDS by direct global-to-LDS loads: nothing waits for them here
// (the compiler waits for them before the next LDS access of the thread).
__device__ __forceinline__ void lbase_to_lds(const Params &p, int blk, int nblk, int pos, float *smem)
{
    typedef __attribute__((address_space(3))) void lds_void;
    const long long v0 = vslice_lo(p.V, blk, nblk);
    const int n = vslice_lo(p.V, blk + 1, nblk) - static_cast<int>(v0);
    const int rows_cap = lbuf_stride(p.V, nblk);
    float *dst = smem + smem_off_lbuf(p.r);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (p.lbase_bf16) {
        // bf16 input: loaded, widened and stored, so the LDS copy is float32 as above
        // (this waits for its loads, which the argmax barrier wait around it covers)
        for (int bb = 0; bb < p.B; ++bb) {
            const uint16_t *src = static_cast<const uint16_t *>(p.L_base) + (static_cast<size_t>(bb) * p.K + pos) * p.V + v0;
#pragma unroll 4
            for (int c = threadIdx.x; c < n; c += NT)
                dst[bb * rows_cap + c] = __uint_as_float(static_cast<uint32_t>(src[c]) << 16);
        }
        return;
    }
    for (int bb = 0; bb < p.B; ++bb) {
        const float *src = static_cast<const float *>(p.L_base) + (static_cast<size_t>(bb) * p.K + pos) * p.V + v0;
        for (int c = wave * 64; c < n; c += NT) {
            if (c + lane < n)
                __builtin_amdgcn_global_load_lds(src + c + lane, (lds_void *)(dst + bb * rows_cap + c), 4, 0, 0);
        }
    }
}

// Running greedy argmax of one lane: order word of the best value (as in
// argmax_key: NaN highest, -0 as +0; 0 = none yet) and its vocabulary index.
// A lane sees its rows in increasing order, so keeping the first of equal
// values keeps the lowest index.
struct LaneBest {
    uint32_t ord = 0, idx = 0;
};

// Result tiles are D = U W2_tile^T (16 x 16): lane l holds D rows (l/16)*4 + i,
// i = 0..3, of column l%16 (the tile's vocabulary row l%16).  U row c < 8 is the
// hi part of batch row c, row 8 + c its lo part, so batch row b's hi values sit
// in acc[b % 4] of lanes 16*(b/4) + 0..15 and its lo values 32 lanes higher.
// w2_hilo returns hi + lo of component i in both halves of the wave.
__device__ inline float w2_hilo(const f32x4_t &acc, int i)
{
    const float x = i == 0 ? acc[0] : i == 1 ? acc[1] : i == 2 ? acc[2] : acc[3];
    uint32_t lo, hi;
    half_values(__float_as_uint(x), lo, hi);
    return __uint_as_float(lo) + __uint_as_float(hi);
}

// Packs one batch row's values of four tiles (from w2_hilo, in lane row 0 of
// each, or lane row 1 when `upper`, i.e. batch rows 4..7) into one register:
// tile j's vocabulary row r at lane 16 j + r.
__device__ inline float w2_pack4(float s0, float s1, float s2, float s3, bool upper)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s2), __float_as_uint(s3), false, false);
    const uint32_t x = upper ? a[1] : a[0], y = upper ? c[1] : c[0];  // {t0, t1, t0, t1}, {t2, t3, t2, t3}
    const auto d = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    return __uint_as_float(d[0]);
}

// Folds one packed value (W2 u of vocabulary row v0 + row) plus its L_base
// value into `best` and stores L_final (lf: the batch row's L_final slice of
// this block, or null).  Lanes with !ok take order 0 (never selected).
__device__ inline void w2_key(float w, float lbv, float *lf, int v0, int row, bool ok, LaneBest &best)
{
    const float v = lbv + w;
    if (lf && ok)
        lf[row] = v;
    const uint32_t bits = __float_as_uint(v + 0.f);  // -0 + +0 = +0
    uint32_t ord = bits ^ (static_cast<uint32_t>(static_cast<int32_t>(bits) >> 31) | 0x80000000u);
    ord = (v != v) ? 0xFFFFFFFFu : ord;
    ord = ok ? ord : 0u;
    const bool take = ord > best.ord;
    best.idx = take ? static_cast<uint32_t>(v0 + row) : best.idx;
    best.ord = take ? ord : best.ord;
}

// Returns false (and sets DOMINO_FLAG_SYNC_TIMEOUT) when the u operand words
// of this position (tag `tag`) did not all arrive within the spin limit.
// NB: largest batch the instantiation handles (B <= NB <= BC); per-row
// registers are sized by it.
// u_src (LDS, [nb][r] floats, or nullptr): the block computed u itself (Markov
// head); the operand is then formed from it with the same hi/lo split.
template <int RT, int KS, int NB>
__device__ __forceinline__ bool phase_w2_resident(const Params &p, int blk, int nblk, int pos, float *smem,
                                                  const W2Resident<RT, KS> &res, const uint4 *tl,
                                                  uint64_t *local_keys, unsigned tag,
                                                  const float *u_src = nullptr)
{
    static_assert(NB >= 1 && NB <= BC, "batch rows of one persistent launch");
    const int r = 32 * KS;
    int v0i = vslice_lo(p.V, blk, nblk);
    int n = vslice_lo(p.V, blk + 1, nblk) - v0i;
    // opaque per call: keeps the compiler from hoisting the per-row index and
    // bound values of every tile out of the position loop into spilled registers
    asm volatile("" : "+s"(v0i), "+s"(n));
    const long long v0 = v0i;
    const int T = (n + 15) / 16;
    const int rows_cap = lbuf_stride(p.V, nblk);
    const float *lbase = smem + smem_off_lbuf(r);
    uint64_t *kred = reinterpret_cast<uint64_t *>(smem + 32);  // after local_keys (BC u64 at smem)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15;
    const int nb = p.B;  // B <= NB
    float *lf = p.L_final ? p.L_final + static_cast<size_t>(pos) * p.V + v0 : nullptr;
    DH_TRACE(pos * 32);
    // A operand (U) from the tagged u words: lane row col = lane % 16 reads plane
    // col / 8 (hi, lo) of batch row col % 8, 8 words per 32-wide step; poll until
    // every word carries this position's tag
    uint4 bop[KS];
    int ok = 1;
    if (u_src) {
        const int b = col & 7;
        const bool hi = col < 8;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            uint32_t hv[8];
            if (b < nb) {
                const float4 x0 = *reinterpret_cast<const float4 *>(u_src + b * r + kk * 32 + (lane >> 4) * 8);
                const float4 x1 = *reinterpret_cast<const float4 *>(u_src + b * r + kk * 32 + (lane >> 4) * 8 + 4);
                const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const uint32_t xh = bf16_rne_bits(x[jj]);
                    hv[jj] = hi ? xh : bf16_rne_bits(x[jj] - __uint_as_float(xh << 16));
                }
            } else {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    hv[jj] = 0u;
            }
            bop[kk] = make_uint4(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                                 hv[6] | (hv[7] << 16));
        }
    } else {
        const int b = col & 7;
        const uint64_t *src = reinterpret_cast<const uint64_t *>(
            p.utag + (static_cast<size_t>(col >> 3) * p.maxB + b) * r + (lane >> 4) * 8);
        const uint32_t want = tag & 0xFFFFu;
        if (b < nb) {
            unsigned spins = 0;
            for (;;) {
                uint32_t bad = 0;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    uint32_t h[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint64_t w = ld_agent_u64(src + kk * 16 + c);
                        const uint32_t w0 = static_cast<uint32_t>(w), w1 = static_cast<uint32_t>(w >> 32);
                        bad |= ((w0 >> 16) ^ want) | ((w1 >> 16) ^ want);
                        h[c] = (w0 & 0xFFFFu) | (w1 << 16);
                    }
                    bop[kk] = make_uint4(h[0], h[1], h[2], h[3]);
                }
                if (!bad)
                    break;
                if (++spins > p.spin_limit) {
                    ok = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                bop[kk] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    DH_TRACE(pos * 32 + 1);
    if (block_failed(ok)) {
        if (threadIdx.x == 0)
            __hip_atomic_fetch_or(gmem(p.flags), 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    DH_TRACE(pos * 32 + 2);
    // per batch row: the lane's running best (batch rows beyond nb stay empty)
    LaneBest best[NB];
    const int jl = lane >> 4, rl = lane & 15;  // packed layout: tile j = jl of a group, row rl
    // register tiles in groups of GR = 4: independent accumulators, steps interleaved
    constexpr int GR = 4;
#pragma unroll
    for (int g0 = 0; g0 < RT; g0 += GR) {
        const int G = RT - g0 < GR ? RT - g0 : GR;  // tiles in this group
        const int row = (wave + (g0 + jl) * NWAVE) * 16 + rl;  // this lane's packed row
        const bool inb = jl < G && row < n;
        float lbv[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            lbv[b] = b < nb ? lbase[b * rows_cap + (inb ? row : 0)] : 0.f;
        f32x4_t acc[GR];
#pragma unroll
        for (int j = 0; j < GR; ++j)
            acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int j = 0; j < GR; ++j)
                if (j < G)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, bop[kk]), __builtin_bit_cast(bf16x8_t, res.wt[g0 + (j < G ? j : 0)][kk]),
                        acc[j], 0, 0, 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < nb) {
                const float w = w2_pack4(w2_hilo(acc[0], b & 3), w2_hilo(acc[1], b & 3), w2_hilo(acc[2], b & 3),
                                         w2_hilo(acc[3], b & 3), b >= 4);
                w2_key(w, lbv[b], lf ? lf + static_cast<size_t>(b) * p.K * p.V : nullptr, v0i, row, inb, best[b]);
            }
        }
    }
    DH_TRACE(pos * 32 + 3);
    // LDS tiles, one at a time: the tile's chunks are read together, then multiplied;
    // only lane row 0 of the packed layout carries rows
#pragma unroll 1
    for (int t = NWAVE * RT + wave; t < T; t += NWAVE) {
        const int sl = t - NWAVE * RT;
        uint4 a[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            a[kk] = tl[(sl * KS + kk) * 64 + lane];
        const int row = t * 16 + rl;
        const bool inb = jl == 0 && row < n;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bop[kk]),
                                                          __builtin_bit_cast(bf16x8_t, a[kk]), acc, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < nb) {
                const float lb = lbase[b * rows_cap + (inb ? row : 0)];
                const float s0 = w2_hilo(acc, b & 3);
                const float w = w2_pack4(s0, s0, s0, s0, b >= 4);
                w2_key(w, lb, lf ? lf + static_cast<size_t>(b) * p.K * p.V : nullptr, v0i, row, inb, best[b]);
            }
        }
    }
    DH_TRACE(pos * 32 + 4);
    // block's key per batch row: over the wave, then over the waves
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (b < nb) {
            uint64_t key = best[b].ord ? (static_cast<uint64_t>(best[b].ord) << 32) | (0xFFFFFFFFu - best[b].idx)
                                       : 0ull;
            key = wave_max_u64(key);
            if (lane == 0)
                kred[wave * BC + b] = key;
        }
    }
    __syncthreads();
    if (threadIdx.x < nb) {
        uint64_t m = 0;
        for (int w = 0; w < NWAVE; ++w)
            m = max_u64(m, kred[w * BC + threadIdx.x]);
        local_keys[threadIdx.x] = m ? (m & KEY_ORD_MASK) | (KEY_IDX_MASK - key_index(m)) : 0ull;
    }
    DH_TRACE(pos * 32 + 5);
    return true;
}

}  // namespace DH_NS
