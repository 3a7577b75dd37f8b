// The phases of one Domino head block draft.  Each phase is a device
// function over a slice of independent work (selected by blk of nblk), so
// the same code runs inside the persistent cooperative kernel (phases
// separated by grid barriers) and as separate stepwise launches.
//
// Method (paper.oopus.info review, section 二, 第二步 Domino Head; news.sig.ai
// article, section "Domino怎么做"), positions p = 0..K-1:
//   A_H[p]  = W1[:, :d] H_p                      (phase_ah, once per call)
//   S_0     = GRU(E[last_tok], S_init)           (phase_gru, q = 0)
//   u_p     = SiLU(A_H[p] + W1[:, d:] S_p)       (phase_u)
//   L_p     = L_base_p + W2 u_p, t_p = argmax    (phase_w2)
//   S_{p+1} = GRU(E[x_p], S_p)                   (phase_gru, q = p+1)
// W1 [H_p; S_p] is split into its H and S column blocks; the H part does not
// depend on the recurrence, so it is computed for all positions up front.
#pragma once

#include "dh_common.h"

namespace dh {

struct Params {
    int d, h, r, V, K, B, maxB;
    const void *W1, *W2, *W_ih, *W_hh, *b_ih, *b_hh, *E;
    const void *H;
    const float *L_base;
    const int *last_tok, *teacher;
    const float *S_init;
    int *tokens;
    float *L_final, *S_out, *u_out;
    // workspace
    float *A_H;      // [maxB, K, r]
    float *S_buf;    // [2, maxB, h]
    float *u_buf;    // [maxB, r]
    uint64_t *keys;  // [K, NG, maxB] partial argmax keys
    unsigned *bar;   // barrier words
    unsigned *flags; // device flags
    unsigned spin_limit;
};

// ---- token bookkeeping ------------------------------------------------------

__device__ inline bool tok_ok(int t, int V) { return t >= 0 && t < V; }

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

// Greedy token of position `pos` for row b: max over the NG partial keys.
__device__ inline int key_token(const Params &p, int pos, int b)
{
    uint64_t best = 0;
    for (int g = 0; g < NG; ++g) {
        uint64_t k = ld_agent_u64(key_slot(p, pos, g, b));
        best = k > best ? k : best;
    }
    return best ? static_cast<int>(key_index(best)) : 0;
}

// GRU input token producing S_q: last_tok for q = 0, else teacher[q-1] or t_{q-1}.
// Invalid ids gather row 0; the row is reported through the flags instead.
__device__ inline int gru_input_token(const Params &p, int q, int b)
{
    int t;
    if (q == 0)
        t = p.last_tok[b];
    else if (p.teacher)
        t = p.teacher[static_cast<size_t>(b) * p.K + (q - 1)];
    else
        t = key_token(p, q - 1, b);
    return tok_ok(t, p.V) ? t : 0;
}

// Block-level side job: publish tokens[:, pos] once position pos is complete.
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
        p.keys[static_cast<size_t>(slot) * p.maxB + b] = 0ull;
    }
    for (int b = threadIdx.x; b < p.B; b += NT)
        if (row_bad(p, b))
            __hip_atomic_fetch_or(p.flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- phase: A_H = W1[:, :d] H for every position ------------------------------
template <typename WT>
__device__ void phase_ah(const Params &p, int blk, int nblk, float *red)
{
    constexpr int EPC = WT16<WT>::EPC;
    const int nch = p.d / EPC;
    const int ntask = p.B * p.r;
    for (int task = blk; task < ntask; task += nblk) {
        const int b = task / p.r, k = task % p.r;
        float acc[MAXK];
#pragma unroll
        for (int i = 0; i < MAXK; ++i)
            acc[i] = 0.f;
        for (int c = threadIdx.x; c < nch; c += NT) {
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
            p.A_H[(static_cast<size_t>(b) * p.K + threadIdx.x) * p.r + k] = red[NWAVE * MAXK + threadIdx.x];
        __syncthreads();
    }
}

// ---- phase: GRU step producing S_q ---------------------------------------------
// Work unit: 4 hidden units of one batch row (12 rows of W_ih, 12 of W_hh).
template <typename WT>
__device__ void phase_gru(const Params &p, int blk, int nblk, int q, float *red)
{
    constexpr int EPC = WT16<WT>::EPC;
    constexpr int UPP = 4;
    __shared__ int s_tok;
    const int h = p.h, d = p.d;
    const int ngrp = (h + UPP - 1) / UPP;
    const int ntask = p.B * ngrp;
    const float *s_prev_all = (q == 0) ? p.S_init : p.S_buf + static_cast<size_t>((q - 1) & 1) * p.maxB * h;
    float *s_next_all = p.S_buf + static_cast<size_t>(q & 1) * p.maxB * h;
    if (q >= 1 && blk == 0)
        write_tokens(p, q - 1);
    for (int task = blk; task < ntask; task += nblk) {
        const int b = task / ngrp, j0 = (task % ngrp) * UPP;
        if (threadIdx.x == 0)
            s_tok = gru_input_token(p, q, b);
        __syncthreads();
        const int tok = s_tok;
        const float *sp = s_prev_all ? s_prev_all + static_cast<size_t>(b) * h : nullptr;
        float acc[UPP * 6];
#pragma unroll
        for (int i = 0; i < UPP * 6; ++i)
            acc[i] = 0.f;
        for (int c = threadIdx.x; c < d / EPC; c += NT) {
            float x[EPC];
            WT16<WT>::unpack(ld16<WT>(p.E, static_cast<size_t>(tok) * d + static_cast<size_t>(c) * EPC), x);
#pragma unroll
            for (int u = 0; u < UPP; ++u) {
                const int j = j0 + u;
                if (j < h) {
#pragma unroll
                    for (int gt = 0; gt < 3; ++gt)
                        acc[u * 6 + gt] = dot_chunk<WT>(
                            ld16<WT>(p.W_ih, static_cast<size_t>(gt * h + j) * d + static_cast<size_t>(c) * EPC), x,
                            acc[u * 6 + gt]);
                }
            }
        }
        if (sp) {
            for (int c = threadIdx.x; c < h / EPC; c += NT) {
                float s[EPC];
                ld_f32<EPC>(sp + static_cast<size_t>(c) * EPC, s);
#pragma unroll
                for (int u = 0; u < UPP; ++u) {
                    const int j = j0 + u;
                    if (j < h) {
#pragma unroll
                        for (int gt = 0; gt < 3; ++gt)
                            acc[u * 6 + 3 + gt] = dot_chunk<WT>(
                                ld16<WT>(p.W_hh, static_cast<size_t>(gt * h + j) * h + static_cast<size_t>(c) * EPC),
                                s, acc[u * 6 + 3 + gt]);
                    }
                }
            }
        }
        block_sum<UPP * 6>(acc, red);
        if (threadIdx.x < UPP) {
            const int j = j0 + threadIdx.x;
            if (j < h) {
                const float *t = red + NWAVE * UPP * 6 + threadIdx.x * 6;
                float gr = t[0], gz = t[1], gn = t[2], qr = t[3], qz = t[4], qn = t[5];
                if (p.b_ih) {
                    gr += WT16<WT>::one(p.b_ih, j);
                    gz += WT16<WT>::one(p.b_ih, h + j);
                    gn += WT16<WT>::one(p.b_ih, 2 * h + j);
                }
                if (p.b_hh) {
                    qr += WT16<WT>::one(p.b_hh, j);
                    qz += WT16<WT>::one(p.b_hh, h + j);
                    qn += WT16<WT>::one(p.b_hh, 2 * h + j);
                }
                const float rg = sigmoidf_(gr + qr);
                const float zg = sigmoidf_(gz + qz);
                const float ng = tanhf(gn + rg * qn);
                const float sprev = sp ? sp[j] : 0.f;
                const float sn = (1.f - zg) * ng + zg * sprev;
                s_next_all[static_cast<size_t>(b) * h + j] = sn;
                if (p.S_out)
                    p.S_out[(static_cast<size_t>(b) * p.K + q) * h + j] = sn;
            }
        }
        __syncthreads();
    }
}

// ---- phase: u_p = SiLU(A_H[p] + W1[:, d:] S_p) ---------------------------------
template <typename WT>
__device__ void phase_u(const Params &p, int blk, int nblk, int pos, float *red)
{
    constexpr int EPC = WT16<WT>::EPC;
    constexpr int KPP = 4;
    const int ngrp = (p.r + KPP - 1) / KPP;
    const int ntask = p.B * ngrp;
    const float *Sb = p.S_buf + static_cast<size_t>(pos & 1) * p.maxB * p.h;
    for (int task = blk; task < ntask; task += nblk) {
        const int b = task / ngrp, k0 = (task % ngrp) * KPP;
        float acc[KPP];
#pragma unroll
        for (int i = 0; i < KPP; ++i)
            acc[i] = 0.f;
        for (int c = threadIdx.x; c < p.h / EPC; c += NT) {
            float s[EPC];
            ld_f32<EPC>(Sb + static_cast<size_t>(b) * p.h + static_cast<size_t>(c) * EPC, s);
#pragma unroll
            for (int kk = 0; kk < KPP; ++kk) {
                const int k = k0 + kk;
                if (k < p.r)
                    acc[kk] = dot_chunk<WT>(
                        ld16<WT>(p.W1, static_cast<size_t>(k) * (p.d + p.h) + p.d + static_cast<size_t>(c) * EPC), s,
                        acc[kk]);
            }
        }
        block_sum<KPP>(acc, red);
        if (threadIdx.x < KPP) {
            const int k = k0 + threadIdx.x;
            if (k < p.r) {
                const float a = p.A_H[(static_cast<size_t>(b) * p.K + pos) * p.r + k] + red[NWAVE * KPP + threadIdx.x];
                const float u = a * sigmoidf_(a);
                p.u_buf[static_cast<size_t>(b) * p.r + k] = u;
                if (p.u_out)
                    p.u_out[(static_cast<size_t>(b) * p.K + pos) * p.r + k] = u;
            }
        }
        __syncthreads();
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
//
// Shared memory: red (256 floats) | kred (NWAVE u64) | u_lds [BC][r] | lbuf [BC][rows_cap]
__host__ __device__ inline int smem_floats(int r, int rows_cap) { return 256 + 2 * NWAVE + BC * (r + rows_cap); }

template <typename WT, int LPR, int NL>
struct W2Rows {
    static constexpr int RPW = 64 / LPR;  // rows per wave per group
    static constexpr int UG = 2;          // row groups per batch

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
#pragma unroll
                for (int o = 1; o < LPR; o <<= 1)
                    acc += __shfl_xor(acc, o);
                if (sub == 0 && row < n)
                    lbuf[bb * rows_cap + row] = acc;
            }
        }
    }
};

template <typename WT, int LPR, int NL>
__device__ void phase_w2(const Params &p, int blk, int nblk, int pos, float *smem)
{
    using R = W2Rows<WT, LPR, NL>;
    constexpr int RPW = R::RPW;
    const int r = p.r;
    const long long v0 = static_cast<long long>(p.V) * blk / nblk;
    const long long v1 = static_cast<long long>(p.V) * (blk + 1) / nblk;
    const int n = static_cast<int>(v1 - v0);
    const int rows_cap = (p.V + nblk - 1) / nblk;
    uint64_t *kred = reinterpret_cast<uint64_t *>(smem + 256);
    float *u_lds = smem + 256 + 2 * NWAVE;
    float *lbuf = u_lds + BC * r;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPR, rw = lane / LPR;
    const int g = blk % NG;
    const int stride = NWAVE * RPW;   // rows between consecutive groups of one wave
    const int bstride = R::UG * stride;

    for (int b0 = 0; b0 < p.B; b0 += BC) {
        const int nb = (p.B - b0) < BC ? (p.B - b0) : BC;
        uint4 wa[R::UG][NL], wb[R::UG][NL];
        int base = wave * RPW;
        R::load(wa, p.W2, r, v0, n, base, rw, sub, stride);
        for (int i = threadIdx.x; i < nb * r; i += NT)
            u_lds[i] = p.u_buf[static_cast<size_t>(b0) * r + i];
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
        for (int bb = 0; bb < nb; ++bb) {
            const int b = b0 + bb;
            const float *lb = p.L_base + (static_cast<size_t>(b) * p.K + pos) * p.V + v0;
            float *lf = p.L_final ? p.L_final + (static_cast<size_t>(b) * p.K + pos) * p.V + v0 : nullptr;
            uint64_t best = 0;
            for (int i = threadIdx.x; i < n; i += NT) {
                const float v = lb[i] + lbuf[bb * rows_cap + i];
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
                __hip_atomic_fetch_max(key_slot(p, pos, g, b), m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        }
    }
}

}  // namespace dh
