// Domino head drafting library for MI355X (gfx950): the host side of the C ABI
// and the kernels built for 512-thread blocks.
//
// Launch kinds over the same phases (dh_phases.h), chosen per call
// (domino_head_exec_info reports which):
//   * persistent, B <= 8: one launch of one block per compute unit runs the
//     whole block draft.  bf16 heads with r = 256 keep each block's W2 slice on
//     chip (domino_head_res.hip); other heads stream W2 every position
//     (k_persistent here).  One argmax barrier per position, plus a grid barrier
//     after each state phase when W2 is streamed;
//   * step launches: one launch per phase and position on the caller's stream;
//     larger bf16 batches run W2, the state dots and A_H on the matrix cores
//     (domino_head_bat.hip), and with a teacher the W2 products of all positions
//     form a single launch.
// Where two launch kinds can run the same call they form every value with the
// same arithmetic, so their outputs are bitwise equal (tested).  The verify
// step is in domino_verify.hip; the prefix match (k_accept_len) is here.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <string>

#include "../../include/domino_head.h"
#include "dh_phases.h"
#include "dh_resident.h"
#include "dh_batched.h"
#include "dh_verify.h"
#include "dh_rbatch.h"

using namespace dh;

// ============================================================================
// kernels
// ============================================================================

// Barrier words, argmax words, u operand words (tag 0: generations restart
// at 0 and the first tag a launch polls for is at least 1) and device flags.
// Argmax words of the batched resident launch: tag 0, which no launch polls for
// (every launch starts from a barrier generation of at least 0 and its first
// poll expects a tag three generations later).
__global__ __launch_bounds__(256) void k_clear_words(uint64_t *w, size_t n)
{
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<size_t>(gridDim.x) * 256)
        w[i] = 0ull;
}

__global__ __launch_bounds__(256) void k_clear_state(unsigned *bar, uint64_t *asy, uint32_t *utag, int n_utag,
                                                     unsigned *flags)
{
    for (int i = threadIdx.x; i < BAR_WORDS_ALL; i += blockDim.x)
        bar[i] = 0u;
    for (int i = threadIdx.x; i < ASYNC_WORDS; i += blockDim.x)
        asy[i] = 0ull;
    for (int i = threadIdx.x; i < n_utag; i += blockDim.x)
        utag[i] = 0u;
    if (threadIdx.x == 0)
        *flags = 0u;
}

// Folded input-gate table P[v][m] = b_ih[m] + sum_k E[v][k] W_ih[m][k]
// (V x 3h, float32), a 64x64 output tile per block, 4x4 per thread.
template <typename WT>
__global__ __launch_bounds__(256) void k_fold(const void *E, const void *W_ih, const void *b_ih, float *P, int V,
                                              int d, int n3)
{
    __shared__ float As[32][68];
    __shared__ float Bs[32][68];
    const int v0 = blockIdx.y * 64, m0 = blockIdx.x * 64;
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < d; k0 += 32) {
        for (int i = threadIdx.x; i < 64 * 32; i += 256) {
            const int rr = i / 32, kk = i % 32, k = k0 + kk;
            const int v = v0 + rr, m = m0 + rr;
            As[kk][rr] = (v < V && k < d) ? WT16<WT>::one(E, static_cast<size_t>(v) * d + k) : 0.f;
            Bs[kk][rr] = (m < n3 && k < d) ? WT16<WT>::one(W_ih, static_cast<size_t>(m) * d + k) : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < 32; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = As[kk][ty * 4 + i];
                b[i] = Bs[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = v0 + ty * 4 + i, m = m0 + tx * 4 + j;
            if (v < V && m < n3)
                P[static_cast<size_t>(v) * n3 + m] = acc[i][j] + (b_ih ? WT16<WT>::one(b_ih, m) : 0.f);
        }
}

// Markov table, create time, for a chunk of n tokens whose folded gate rows
// Pc = E W_ih^T + b_ih are given: the zero-state GRU step of each token,
//   Sc[t][j] = (1 - z) n,  r = sig(g_r + b_hr), z = sig(g_z + b_hz), n = tanh(g_n + r b_hn)
// (W_hh times the zero state vanishes; the z * 0 term is dropped).
template <typename WT>
__global__ __launch_bounds__(256) void k_markov_state(const float *Pc, const void *b_hh, float *Sc, int n, int h)
{
    const size_t total = static_cast<size_t>(n) * h;
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<size_t>(gridDim.x) * 256) {
        const size_t t = i / h;
        const int j = static_cast<int>(i % h);
        const float *g = Pc + t * 3 * h;
        const float br = b_hh ? WT16<WT>::one(b_hh, j) : 0.f;
        const float bz = b_hh ? WT16<WT>::one(b_hh, h + j) : 0.f;
        const float bn = b_hh ? WT16<WT>::one(b_hh, 2 * h + j) : 0.f;
        const float rg = sigmoidf_(g[j] + br);
        const float zg = sigmoidf_(g[h + j] + bz);
        const float ng = tanhf_(g[2 * h + j] + rg * bn);
        Sc[i] = (1.f - zg) * ng;
    }
}

// Create time: the W1_S rows, then the W_hh rows, into wst [r + 3h, ldw] (bf16
// bits), zero padded.
__global__ __launch_bounds__(256) void k_pack_state_rows(const uint16_t *W1, const uint16_t *W_hh, uint16_t *wst,
                                                         int r, int d, int h, int ldw)
{
    const size_t total = static_cast<size_t>(r + 3 * h) * ldw;
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<size_t>(gridDim.x) * 256) {
        const int m = static_cast<int>(i / ldw), j = static_cast<int>(i % ldw);
        uint16_t v = 0;
        if (j < h)
            v = m < r ? W1[static_cast<size_t>(m) * (d + h) + d + j] : W_hh[static_cast<size_t>(m - r) * h + j];
        wst[i] = v;
    }
}

// Create time: the state columns of W1 as a contiguous float32 [r, h] matrix.
template <typename WT>
__global__ __launch_bounds__(256) void k_w1s_widen(const void *W1, float *W1S, int r, int d, int h)
{
    const size_t total = static_cast<size_t>(r) * h;
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<size_t>(gridDim.x) * 256)
        W1S[i] = WT16<WT>::one(W1, (i / h) * (d + h) + d + i % h);
}

// Markov head, step launches: u of position q (q >= 0, into u_buf for the W2
// launch that follows) or of every position (q < 0, teacher forcing), from A_H
// and the table row of the preceding token (markov_u); also into u_out when
// given.  With q >= 1, block 0 first publishes tokens[:, q-1].
__global__ __launch_bounds__(NT) void k_markov_u(Params p, int q)
{
    if (q >= 1 && blockIdx.x == 0)
        write_tokens(p, q - 1);
    const int r = p.r, nq = q < 0 ? p.K : 1;
    const size_t total = static_cast<size_t>(p.B) * nq * r;
    for (size_t i = static_cast<size_t>(blockIdx.x) * NT + threadIdx.x; i < total;
         i += static_cast<size_t>(gridDim.x) * NT) {
        const int m = static_cast<int>(i % r);
        const int bq = static_cast<int>(i / r);
        const int b = bq / nq, qq = q < 0 ? bq % nq : q;
        const size_t o = (static_cast<size_t>(b) * p.K + qq) * r + m;
        const float u = markov_u(p, xld(&p.A_H[o]), m, gru_input_token(p, qq, b));
        if (q >= 0)
            p.u_buf[static_cast<size_t>(b) * r + m] = u;
        if (p.u_out)
            p.u_out[o] = u;
    }
}

// Whole block draft in one cooperative launch.  Barriers per call:
// 2 + K + (K - 1) with the folded table, 2 + K + 2 (K - 1) without.  The
// barrier after each W2 phase also reduces the greedy argmax.
template <typename WT, int LPR, int NL>
__global__ __launch_bounds__(NT) void k_persistent(Params p)
{
    extern __shared__ float smem[];
    const int blk = blockIdx.x, nblk = gridDim.x;
    float *S_lds = smem + smem_off_S(p.r, lbuf_stride(p.V, nblk));
    float *cache = S_lds + BC * p.h;  // state rows and A_H entries (state_cache_load)
    int *atok = reinterpret_cast<int *>(smem + smem_off_tok()) + ATOK_OFF;
    int *bad = atok + BC;  // block 0: rows whose token ids are invalid
    uint64_t *local_keys = reinterpret_cast<uint64_t *>(smem);  // the reduction area is free inside the loop
    unsigned gen = barrier_gen_init(p.bar);
    block_fail_init();
    if (blk == 0) {
        prologue_bookkeeping(p);
        if (threadIdx.x < p.B)
            bad[threadIdx.x] = row_bad(p, threadIdx.x) ? 1 : 0;
    }
    phase_ah<WT>(p, blk, nblk, smem);
    phase_q_init<WT>(p, blk, nblk);
    if (!p.P)
        phase_g<WT>(p, blk, nblk, 0, smem);
    if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
        return;
    StatePre spre;
    W2Pre<WT, LPR, NL> wpre;
    state_cache_load<WT>(p, blk, nblk, cache);
    state_prefetch<WT>(p, 0, spre);
    phase_state<WT>(p, blk, nblk, 0, smem, S_lds, &spre, cache, true);
    grid_arrive(p.bar, gen);
    w2_prefetch<WT, LPR, NL>(p, blk, nblk, wpre);
    if (!grid_wait(p.bar, gen, p.spin_limit, p.flags))
        return;
    for (int pos = 0; pos < p.K; ++pos) {
        phase_w2<WT, LPR, NL>(p, blk, nblk, pos, smem, &wpre, local_keys);
        // loads of data published before the previous barrier go between arrival and wait
        argmax_arrive(p.asy, gen, local_keys, p.B);
        if (pos + 1 < p.K)
            state_prefetch<WT>(p, pos + 1, spre);
        if (!argmax_wait(p.asy, gen, p.B, atok, p.spin_limit, p.flags))
            return;
        if (blk == 0 && threadIdx.x < p.B)
            p.tokens[static_cast<size_t>(threadIdx.x) * p.K + pos] = bad[threadIdx.x] ? -1 : atok[threadIdx.x];
        if (pos + 1 < p.K) {
            if (!p.P) {
                phase_g<WT>(p, blk, nblk, pos + 1, smem, atok);
                if (!grid_sync(p.bar, gen, p.spin_limit, p.flags))
                    return;
            }
            phase_state<WT>(p, blk, nblk, pos + 1, smem, S_lds, &spre, cache, true, atok);
            grid_arrive(p.bar, gen);
            w2_prefetch<WT, LPR, NL>(p, blk, nblk, wpre);
            if (!grid_wait(p.bar, gen, p.spin_limit, p.flags))
                return;
        }
    }
    barrier_finish(p.bar, gen);
}


template <typename WT>
__global__ __launch_bounds__(NT) void k_step_prologue(Params p)
{
    extern __shared__ float smem[];
    // the partial keys of every position, zeroed by all blocks (the launches that
    // fold into them come later on the stream); block 0 flags invalid rows
    const size_t nkeys = static_cast<size_t>(p.K) * NG * p.maxB;
    for (size_t i = static_cast<size_t>(blockIdx.x) * NT + threadIdx.x; i < nkeys;
         i += static_cast<size_t>(gridDim.x) * NT)
        p.keys[i] = 0ull;
    if (blockIdx.x == 0) {
        for (int b = threadIdx.x; b < p.B; b += NT)
            if (row_bad(p, b))
                __hip_atomic_fetch_or(gmem(p.flags), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!p.ah_external)
        phase_ah<WT>(p, blockIdx.x, gridDim.x, smem);
    if (p.M)
        return;  // Markov head: no recurrent state
    // q_0 = W_hh S_init + b_hh; without S_init the gate update reads b_hh itself
    if (p.S_init)
        phase_q_init<WT>(p, blockIdx.x, gridDim.x);
    if (!p.P)
        phase_g<WT>(p, blockIdx.x, gridDim.x, 0, smem);
}

__global__ __launch_bounds__(NT) void k_step_update(Params p, int q)
{
    extern __shared__ float smem[];
    phase_update(p, blockIdx.x, gridDim.x, q, smem);
}

template <typename WT>
__global__ __launch_bounds__(NT) void k_step_state(Params p, int q)
{
    extern __shared__ float smem[];
    phase_state<WT>(p, blockIdx.x, gridDim.x, q, smem, smem + smem_off_S(p.r, 0), nullptr, smem, false);
}

template <typename WT, int LPR, int NL>
__global__ __launch_bounds__(NT) void k_step_w2(Params p, int pos)
{
    extern __shared__ float smem[];
    phase_w2<WT, LPR, NL>(p, blockIdx.x, gridDim.x, pos, smem, static_cast<const W2Pre<WT, LPR, NL> *>(nullptr),
                          nullptr);
}

template <typename WT>
__global__ __launch_bounds__(NT) void k_step_g(Params p, int q)
{
    extern __shared__ float smem[];
    phase_g<WT>(p, blockIdx.x, gridDim.x, q, smem);
}

__global__ __launch_bounds__(NT) void k_step_final(Params p)
{
    write_tokens(p, p.K - 1);
}

// Position-batched launches: zero the partial keys of the one W2 launch over
// n = B K rows, whose slots are keys[g * n + row].
__global__ __launch_bounds__(NT) void k_keys_zero(uint64_t *keys, int n)
{
    for (int i = blockIdx.x * NT + threadIdx.x; i < n; i += gridDim.x * NT)
        keys[i] = 0ull;
}

// Position-batched launches: tokens[b][pos] from the partial keys of row
// b K + pos (p is the call's own Params: B rows, K positions).
__global__ __launch_bounds__(NT) void k_rows_tokens(Params p)
{
    const int n = p.B * p.K;
    for (int i = blockIdx.x * NT + threadIdx.x; i < n; i += gridDim.x * NT) {
        uint64_t best = 0;
        for (int g = 0; g < NG; ++g) {
            const uint64_t k = ld_agent_u64(p.keys + static_cast<size_t>(g) * n + i);
            best = k > best ? k : best;
        }
        p.tokens[i] = row_bad(p, i / p.K) ? -1 : (best ? static_cast<int>(key_index(best)) : 0);
    }
}

// Verify-side accept length: one thread per row.
__global__ __launch_bounds__(256) void k_accept_len(int B, int K, const int *__restrict__ draft,
                                                    const int *__restrict__ target, int *__restrict__ out)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B)
        return;
    const int *d = draft + static_cast<size_t>(b) * K;
    const int *t = target + static_cast<size_t>(b) * K;
    int j = 0;
    while (j < K && d[j] == t[j])
        ++j;
    out[b] = j;
}

// ============================================================================
// host side
// ============================================================================

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(DOMINO_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(call, what)                 \
    do {                                    \
        hipError_t e_ = (call);             \
        if (e_ != hipSuccess)               \
            return hip_fail(e_, what);      \
    } while (0)

constexpr size_t ALIGN = 256;
constexpr int W2_STEP_ROWS = 128;  // vocabulary rows per block in stepwise W2 launches
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
    size_t bar, asy, flags, keys, A_H, S_buf, u_buf, u_all, utag, s_hl, q_buf, g_buf, gtag, P, M, mk_tmp, wst, bkeys,
        uop, rbs, ucnt, total;
};

// Packed state-dot rows for the matrix-core state launches (bf16 heads): the rows of
// W1_S and W_hh copied with a row stride 64 bytes past a multiple of 256 bytes, so the
// rows a tile reads together do not all start on the same memory channel (the
// caller's 2 KiB rows at h = 1024 do)
bool packed_state_rows(const domino_head_config &c)
{
    return c.wdtype == DOMINO_BF16 && c.r % 32 == 0 && c.h % 32 == 0 && c.max_batch > BC;
}
int packed_ldw(const domino_head_config &c) { return (c.h + 127) / 128 * 128 + 32; }
// batched resident launch: batch rows of its buffers, 16-row groups, and the row stride
// of its S planes (elements; h a multiple of 64, so rows are whole 128-byte lines)
int rb_bmax(const domino_head_config &c) { return std::min(c.max_batch, dhrb::max_batch()); }
int rb_ngr(const domino_head_config &c) { return (rb_bmax(c) + 15) / 16; }
int rb_ldp(const domino_head_config &c) { return c.h + 64; }

// Markov table fill: tokens per chunk (create-time region: folded gate rows and
// zero-state GRU rows of one chunk, plus W1_S as float32)
constexpr int MARKOV_CHUNK = 8192;
int markov_chunk(const domino_head_config &c) { return std::min(c.V, MARKOV_CHUNK); }

size_t gtag_words(const domino_head_config &c) { return static_cast<size_t>(std::min(c.max_batch, BC)) * 3 * c.h; }

Layout layout_of(const domino_head_config &c)
{
    Layout L{};
    size_t off = 0;
    L.bar = off;
    off = align_up(off + sizeof(unsigned) * BAR_WORDS_ALL);
    L.asy = off;
    off = align_up(off + sizeof(uint64_t) * ASYNC_WORDS);
    L.flags = off;
    off = align_up(off + 64);
    L.keys = off;
    off = align_up(off + sizeof(uint64_t) * static_cast<size_t>(c.K) * NG * c.max_batch);
    L.A_H = off;
    off = align_up(off + sizeof(float) * static_cast<size_t>(c.max_batch) * c.K * c.r);
    L.S_buf = off;
    off = align_up(off + sizeof(float) * 2 * static_cast<size_t>(c.max_batch) * c.h);
    L.u_buf = off;
    off = align_up(off + sizeof(float) * static_cast<size_t>(c.max_batch) * c.r);
    L.u_all = off;  // u of every position for the position-batched W2 launch
    off = align_up(off + sizeof(float) * static_cast<size_t>(c.max_batch) * c.K * c.r);
    L.utag = off;
    off = align_up(off + sizeof(uint32_t) * 2 * static_cast<size_t>(c.max_batch) * c.r);
    L.s_hl = off;  // rows of packed_ldw elements (used only with packed state rows)
    off = align_up(off + sizeof(uint16_t) * 2 * static_cast<size_t>(c.max_batch) *
                             (packed_state_rows(c) ? packed_ldw(c) : c.h));
    L.q_buf = off;
    off = align_up(off + sizeof(float) * 2 * static_cast<size_t>(c.max_batch) * 3 * c.h);
    L.g_buf = off;
    off = align_up(off + sizeof(float) * static_cast<size_t>(c.max_batch) * 3 * c.h);
    L.gtag = off;  // tagged g words of the resident launch (not folded)
    if (!(c.flags & DOMINO_FOLD_EMBED))
        off = align_up(off + sizeof(uint64_t) * gtag_words(c));
    L.P = off;
    if (c.flags & DOMINO_FOLD_EMBED)
        off = align_up(off + sizeof(float) * static_cast<size_t>(c.V) * 3 * c.h);
    L.wst = off;
    if (packed_state_rows(c))
        off = align_up(off + sizeof(uint16_t) * static_cast<size_t>(c.r + 3 * c.h) * packed_ldw(c));
    // batched resident launch: argmax words [max_batch, MAX_GRID], the u operand of
    // every position [K][groups][r / 32][64] x 16 bytes (bf16), and the S planes of
    // every state [K + 1][hi, lo][rows][rb_ldp] bf16
    L.bkeys = off;
    L.uop = off;
    L.rbs = off;
    if (packed_state_rows(c)) {
        off = align_up(off + sizeof(uint64_t) * static_cast<size_t>(c.max_batch) * MAX_GRID);
        L.uop = off;
        off = align_up(off + sizeof(uint16_t) * static_cast<size_t>(c.K) * rb_ngr(c) * 16 * c.r);
        L.rbs = off;
        off = align_up(off + sizeof(uint16_t) * 2 * static_cast<size_t>(c.K + 1) * rb_bmax(c) * rb_ldp(c));
    }
    L.ucnt = off;
    if (packed_state_rows(c))
        off = align_up(off + sizeof(unsigned) * MAXK);
    L.M = off;
    L.mk_tmp = off;
    if (c.flags & DOMINO_MARKOV) {
        off = align_up(off + sizeof(float) * static_cast<size_t>(c.V) * c.r);
        L.mk_tmp = off;
        const size_t ch = static_cast<size_t>(markov_chunk(c));
        off = align_up(off + sizeof(float) * (ch * 3 * c.h + ch * c.h + static_cast<size_t>(c.r) * c.h));
    }
    L.total = off;
    return L;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int validate_config(const domino_head_config *c)
{
    if (!c)
        return fail(DOMINO_EINVAL, "config is NULL");
    if (c->wdtype != DOMINO_F32 && c->wdtype != DOMINO_BF16)
        return fail(DOMINO_EUNSUPPORTED, "wdtype %d is neither DOMINO_F32 nor DOMINO_BF16", c->wdtype);
    if (c->K < 1 || c->K > MAXK)
        return fail(DOMINO_EINVAL, "K=%d outside [1, %d]", c->K, MAXK);
    if (c->max_batch < 1 || c->max_batch > 1024)
        return fail(DOMINO_EINVAL, "max_batch=%d outside [1, 1024]", c->max_batch);
    if (c->V < 1)
        return fail(DOMINO_EINVAL, "V=%d < 1", c->V);
    if (c->d < 8 || c->d % 8 || c->h < 8 || c->h % 8 || c->h > 2048)
        return fail(DOMINO_EUNSUPPORTED, "d=%d and h=%d must be positive multiples of 8 (h <= 2048)", c->d, c->h);
    const int epc = c->wdtype == DOMINO_BF16 ? 8 : 4;
    if (c->r < epc || c->r % epc || !pow2(c->r / epc) || c->r / epc > 128 || c->r > 1024)
        return fail(DOMINO_EUNSUPPORTED, "r=%d: r/%d must be a power of two <= 128 and r <= 1024", c->r, epc);
    const void *ptrs[] = {c->W1, c->W2, c->W_ih, c->W_hh, c->E};
    const char *names[] = {"W1", "W2", "W_ih", "W_hh", "E"};
    for (int i = 0; i < 5; ++i) {
        if (!ptrs[i])
            return fail(DOMINO_EINVAL, "%s is NULL", names[i]);
        if (!aligned16(ptrs[i]))
            return fail(DOMINO_EINVAL, "%s is not 16-byte aligned", names[i]);
    }
    if (c->flags & ~(DOMINO_EXEC_PERSISTENT | DOMINO_EXEC_STEPWISE | DOMINO_FOLD_EMBED | DOMINO_EXEC_STREAM_W2 |
                     DOMINO_EXEC_PLAIN_LAUNCH | DOMINO_EXEC_POSITION_BATCHED | DOMINO_LBASE_BF16 | DOMINO_MARKOV))
        return fail(DOMINO_EINVAL, "unknown flags 0x%x", c->flags);
    if ((c->flags & DOMINO_MARKOV) && (c->flags & (DOMINO_FOLD_EMBED | DOMINO_EXEC_STREAM_W2)))
        return fail(DOMINO_EINVAL, "DOMINO_MARKOV does not combine with DOMINO_FOLD_EMBED or DOMINO_EXEC_STREAM_W2");
    if ((c->flags & DOMINO_EXEC_PERSISTENT) && (c->flags & DOMINO_EXEC_STEPWISE))
        return fail(DOMINO_EINVAL, "flags ask for both persistent and stepwise execution");
    return DOMINO_OK;
}

// ---- kernel table -------------------------------------------------------------

typedef hipError_t (*FoldLaunch)(const domino_head_config &c, float *P);

template <typename WT>
hipError_t launch_fold(const domino_head_config &c, float *P)
{
    const int n3 = 3 * c.h;
    dim3 grid((n3 + 63) / 64, (c.V + 63) / 64);
    hipLaunchKernelGGL(k_fold<WT>, grid, dim3(256), 0, nullptr, c.E, c.W_ih, c.b_ih, P, c.V, c.d, n3);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : hipStreamSynchronize(nullptr);
}

// Markov table M = W1_S GRU(E[t], 0) for every token, in chunks of tokens:
// folded gate rows (k_fold), zero-state GRU rows (k_markov_state), then the
// product with W1_S (k_fold on float32 operands, no bias).  Null stream, waited for.
template <typename WT>
hipError_t launch_markov(const domino_head_config &c, float *M, float *tmp)
{
    const int ch = markov_chunk(c), h = c.h, n3 = 3 * c.h;
    float *Pc = tmp;
    float *Sc = Pc + static_cast<size_t>(ch) * n3;
    float *W1S = Sc + static_cast<size_t>(ch) * h;
    const size_t esz = c.wdtype == DOMINO_BF16 ? 2 : 4;
    hipLaunchKernelGGL(k_w1s_widen<WT>, dim3(256), dim3(256), 0, nullptr, c.W1, W1S, c.r, c.d, h);
    hipError_t e = hipGetLastError();
    for (int t0 = 0; t0 < c.V && e == hipSuccess; t0 += ch) {
        const int n = std::min(ch, c.V - t0);
        const void *Et = static_cast<const char *>(c.E) + static_cast<size_t>(t0) * c.d * esz;
        hipLaunchKernelGGL(k_fold<WT>, dim3((n3 + 63) / 64, (n + 63) / 64), dim3(256), 0, nullptr, Et, c.W_ih, c.b_ih,
                           Pc, n, c.d, n3);
        hipLaunchKernelGGL(k_markov_state<WT>, dim3(1024), dim3(256), 0, nullptr, Pc, c.b_hh, Sc, n, h);
        hipLaunchKernelGGL(k_fold<float>, dim3((c.r + 63) / 64, (n + 63) / 64), dim3(256), 0, nullptr, Sc, W1S,
                           nullptr, M + static_cast<size_t>(t0) * c.r, n, h, c.r);
        e = hipGetLastError();
    }
    return e != hipSuccess ? e : hipStreamSynchronize(nullptr);
}

typedef hipError_t (*MarkovLaunch)(const domino_head_config &c, float *M, float *tmp);

struct Kernels {
    const void *persistent;
    const void *w2;
    const void *prologue, *state, *g;
    FoldLaunch fold;
    MarkovLaunch markov;
};

template <typename WT, int LPR, int NL>
Kernels kernels_for()
{
    return Kernels{reinterpret_cast<const void *>(&k_persistent<WT, LPR, NL>),
                   reinterpret_cast<const void *>(&k_step_w2<WT, LPR, NL>),
                   reinterpret_cast<const void *>(&k_step_prologue<WT>),
                   reinterpret_cast<const void *>(&k_step_state<WT>), reinterpret_cast<const void *>(&k_step_g<WT>),
                   &launch_fold<WT>, &launch_markov<WT>};
}

template <typename WT>
Kernels pick_lpr(int nchunks)
{
    switch (nchunks) {
    case 1: return kernels_for<WT, 1, 1>();
    case 2: return kernels_for<WT, 2, 1>();
    case 4: return kernels_for<WT, 4, 1>();
    case 8: return kernels_for<WT, 8, 1>();
    case 16: return kernels_for<WT, 8, 2>();
    case 32: return kernels_for<WT, 8, 4>();
    case 64: return kernels_for<WT, 8, 8>();
    default: return kernels_for<WT, 8, 16>();  // 128
    }
}

Kernels pick_kernels(const domino_head_config &c)
{
    if (c.wdtype == DOMINO_BF16)
        return pick_lpr<bf16s>(c.r / 8);
    return pick_lpr<float>(c.r / 4);
}

}  // namespace

struct domino_head {
    domino_head_config cfg;
    char *ws;
    size_t ws_bytes;
    Layout L;
    Kernels kern;
    int device;
    int cus;
    int persist_grid;      // blocks of the persistent launch (0: cannot be co-resident)
    size_t persist_smem;
    int res_grid;          // blocks of the resident-W2 persistent launch (0: not usable)
    int rb_grid;           // blocks of the batched resident-W2 persistent launch (0: not usable)
    size_t res_smem;
    bool state_ready;      // barrier words and flags cleared on the device
    hipStream_t last_stream;
    unsigned spin_limit;
};

// Launch taken by a draft of B rows: the single cooperative launch (persistent) or the
// per-step launches; the persistent one keeps W2 on chip (resident) when that variant
// fits: up to BC rows the kernel that computes the whole state in every block, above
// that (bf16, r = 256, folded table) the batched kernel (*batched) that distributes
// the state update and the state dots.  Returns false when the handle forces a
// persistent launch that cannot run.
static bool choose_launch(const domino_head *hd, int B, bool *persistent, bool *resident, bool *batched)
{
    const unsigned fl = hd->cfg.flags;
    *batched = false;
    // the batched persistent launch (8 < B <= 256) is ahead of the step launches at every batch
    // measured (8B head, K = 16: 454 against 668 us at B = 32, 1009 against 1167 at B = 256),
    // for the recurrent and the Markov head
    if (B > BC && hd->rb_grid > 0 && B <= dhrb::max_batch() && !(fl & (DOMINO_EXEC_STEPWISE | DOMINO_EXEC_STREAM_W2))) {
        *persistent = *resident = *batched = true;
        return true;
    }
    if (fl & DOMINO_MARKOV) {
        // a Markov head takes its resident-W2 kernel (bf16, r = 256, B <= 8) or the step launches
        const bool can = hd->res_grid > 0 && B <= BC;
        const bool pers = (fl & DOMINO_EXEC_PERSISTENT) ? true : (fl & DOMINO_EXEC_STEPWISE) ? false : can;
        if (pers && !can)
            return false;
        *persistent = *resident = pers;
        return true;
    }
    bool pers = (fl & DOMINO_EXEC_PERSISTENT) ? true : (fl & DOMINO_EXEC_STEPWISE) ? false : B <= BC;
    if (pers && (hd->persist_grid == 0 || B > BC)) {
        if (fl & DOMINO_EXEC_PERSISTENT)
            return false;
        pers = false;
    }
    *persistent = pers;
    *resident = pers && hd->res_grid > 0 && !(fl & DOMINO_EXEC_STREAM_W2);
    return true;
}

extern "C" {

const char *domino_last_error(void) { return g_err.c_str(); }

int domino_head_workspace_size(const domino_head_config *cfg, size_t *bytes)
{
    int rc = validate_config(cfg);
    if (rc)
        return rc;
    if (!bytes)
        return fail(DOMINO_EINVAL, "bytes is NULL");
    *bytes = layout_of(*cfg).total;
    return DOMINO_OK;
}

int domino_head_param_count(const domino_head_config *cfg, int64_t *n)
{
    if (!cfg || !n)
        return fail(DOMINO_EINVAL, "NULL argument");
    const int64_t d = cfg->d, h = cfg->h, r = cfg->r, V = cfg->V;
    int64_t c = r * (d + h) + V * r + 3 * h * d + 3 * h * h;
    if (cfg->b_ih)
        c += 3 * h;
    if (cfg->b_hh)
        c += 3 * h;
    *n = c;
    return DOMINO_OK;
}

int domino_head_create(const domino_head_config *cfg, void *workspace, size_t workspace_bytes, domino_head_t *out)
{
    int rc = validate_config(cfg);
    if (rc)
        return rc;
    if (!out)
        return fail(DOMINO_EINVAL, "out is NULL");
    const Layout L = layout_of(*cfg);
    if (!workspace)
        return fail(DOMINO_EWORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % ALIGN)
        return fail(DOMINO_EWORKSPACE, "workspace is not %zu-byte aligned", ALIGN);
    if (workspace_bytes < L.total)
        return fail(DOMINO_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    int cus = 0;
    HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "hipDeviceGetAttribute");
    const Kernels kern = pick_kernels(*cfg);
    int lds_max = 0;
    HIP_TRY(hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev), "hipDeviceGetAttribute");
    // largest stepwise kernel: the W2 phase (rows_cap <= W2_STEP_ROWS) or phase_state (rows_cap = 0)
    const size_t step_smem = sizeof(float) * std::max(smem_floats_w2(cfg->r, W2_STEP_ROWS), smem_floats(cfg->r, cfg->h, 0));
    if (step_smem + 1024 > static_cast<size_t>(lds_max))
        return fail(DOMINO_EUNSUPPORTED, "r=%d, h=%d need %zu bytes of LDS per block, the device has %d", cfg->r,
                    cfg->h, step_smem, lds_max);
    if (cfg->flags & DOMINO_FOLD_EMBED) {
        // one-time table P = E W_ih^T + b_ih on the null stream, waited for here
        HIP_TRY(kern.fold(*cfg, reinterpret_cast<float *>(static_cast<char *>(workspace) + L.P)), "folded gate table");
    }
    if (packed_state_rows(*cfg)) {
        hipLaunchKernelGGL(k_pack_state_rows, dim3(1024), dim3(256), 0, nullptr, static_cast<const uint16_t *>(cfg->W1),
                           static_cast<const uint16_t *>(cfg->W_hh),
                           reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + L.wst), cfg->r, cfg->d, cfg->h,
                           packed_ldw(*cfg));
        HIP_TRY(hipGetLastError(), "launch k_pack_state_rows");
        HIP_TRY(hipStreamSynchronize(nullptr), "packed state rows");
    }
    if (cfg->flags & DOMINO_MARKOV) {
        HIP_TRY(kern.markov(*cfg, reinterpret_cast<float *>(static_cast<char *>(workspace) + L.M),
                            reinterpret_cast<float *>(static_cast<char *>(workspace) + L.mk_tmp)),
                "Markov table");
    }
    domino_head *hd = new domino_head{};
    hd->cfg = *cfg;
    hd->ws = static_cast<char *>(workspace);
    hd->ws_bytes = workspace_bytes;
    hd->L = L;
    hd->kern = kern;
    hd->device = dev;
    hd->cus = cus;
    hd->state_ready = false;
    hd->last_stream = nullptr;
    hd->spin_limit = 1u << 22;
    if (const char *s = std::getenv("DOMINO_BARRIER_SPIN_LIMIT"))
        hd->spin_limit = static_cast<unsigned>(std::strtoul(s, nullptr, 10));
    // persistent launch: one block per compute unit, all co-resident
    const int rows_cap = lbuf_stride(cfg->V, cus);
    hd->persist_smem = sizeof(float) * (smem_floats(cfg->r, cfg->h, rows_cap) +
                                        state_cache_floats(cfg->r, cfg->h, cfg->K, cus,
                                                           cfg->wdtype == DOMINO_BF16 ? 2 : 4));
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern.persistent, NT, hd->persist_smem);
    // the argmax barrier packs token ids into 18 bits
    hd->persist_grid = (e == hipSuccess && per_cu >= 1 && cus <= MAX_GRID && cfg->V <= (1 << 18) &&
                        hd->persist_smem + 1024 <= static_cast<size_t>(lds_max))
                           ? cus
                           : 0;
    // resident-W2 variant: bf16, r = 256, one 256-thread block per compute unit
    hd->res_grid = 0;
    if (cfg->wdtype == DOMINO_BF16 && cfg->r == dhres::r_supported() && hd->persist_grid) {
        hd->res_smem = dhres::smem_bytes(cfg->r, cfg->h, cfg->K, cfg->V, cus);
        // both instantiations (B = 1 and B <= 8) must fit one block per compute unit
        bool fits = hd->res_smem + 1024 <= static_cast<size_t>(lds_max);
        for (int b : {1, BC}) {
            int per_cu_r = 0;
            const void *fn = (cfg->flags & DOMINO_MARKOV) ? dhres::markov_kernel(b) : dhres::kernel(b);
            hipError_t er = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_r, fn, dhres::threads(),
                                                                         hd->res_smem);
            fits = fits && er == hipSuccess && per_cu_r >= 1;
        }
        if (fits)
            hd->res_grid = cus;
    }
    // batched resident-W2 variant (B > BC): bf16, r = 256, folded table (or a Markov
    // head), packed state rows, one 512-thread block per compute unit with static LDS only
    hd->rb_grid = 0;
    if (cfg->wdtype == DOMINO_BF16 && (cfg->flags & (DOMINO_FOLD_EMBED | DOMINO_MARKOV)) &&
        packed_state_rows(*cfg) && dhrb::supports(cfg->d, cfg->h, cfg->r, cfg->V, cus)) {
        bool fits = true;
        for (int lb16 = 0; lb16 < 2; ++lb16)
            for (int stl = 0; stl < 2; ++stl) {
                int per_cu_b = 0;
                hipError_t eb = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &per_cu_b, dhrb::kernel(lb16 != 0, stl != 0, cfg->V, (cfg->flags & DOMINO_MARKOV) != 0),
                    dhrb::threads(), 0);
                fits = fits && eb == hipSuccess && per_cu_b >= 1;
            }
        if (fits)
            hd->rb_grid = cus;
    }
    *out = hd;
    return DOMINO_OK;
}

void domino_head_destroy(domino_head_t hd) { delete hd; }

static Params make_params(domino_head_t hd, int B, const void *H, const void *L_base, const int32_t *last_tok,
                          const int32_t *teacher, const float *S_init, int32_t *tokens, float *L_final, float *S_out,
                          float *u_out, bool persistent)
{
    const domino_head_config &c = hd->cfg;
    Params p{};
    p.bf16w = c.wdtype == DOMINO_BF16 ? 1 : 0;
    p.d = c.d;
    p.h = c.h;
    p.r = c.r;
    p.V = c.V;
    p.K = c.K;
    p.B = B;
    p.maxB = c.max_batch;
    p.W1 = c.W1;
    p.W2 = c.W2;
    p.W_ih = c.W_ih;
    p.W_hh = c.W_hh;
    p.b_ih = c.b_ih;
    p.b_hh = c.b_hh;
    p.E = c.E;
    p.P = (c.flags & DOMINO_FOLD_EMBED) ? reinterpret_cast<const float *>(hd->ws + hd->L.P) : nullptr;
    p.M = (c.flags & DOMINO_MARKOV) ? reinterpret_cast<const float *>(hd->ws + hd->L.M) : nullptr;
    p.H = H;
    p.L_base = L_base;
    p.lbase_bf16 = (hd->cfg.flags & DOMINO_LBASE_BF16) ? 1 : 0;
    p.last_tok = last_tok;
    p.teacher = teacher;
    p.S_init = S_init;
    p.tokens = tokens;
    p.L_final = L_final;
    p.S_out = S_out;
    p.u_out = u_out;
    p.A_H = reinterpret_cast<float *>(hd->ws + hd->L.A_H);
    p.S_buf = reinterpret_cast<float *>(hd->ws + hd->L.S_buf);
    p.u_buf = reinterpret_cast<float *>(hd->ws + hd->L.u_buf);
    p.q_buf = reinterpret_cast<float *>(hd->ws + hd->L.q_buf);
    p.g_buf = reinterpret_cast<float *>(hd->ws + hd->L.g_buf);
    p.keys = reinterpret_cast<uint64_t *>(hd->ws + hd->L.keys);
    p.bar = reinterpret_cast<unsigned *>(hd->ws + hd->L.bar);
    p.asy = reinterpret_cast<uint64_t *>(hd->ws + hd->L.asy);
    p.flags = reinterpret_cast<unsigned *>(hd->ws + hd->L.flags);
    p.spin_limit = hd->spin_limit;
    p.persistent = persistent ? 1 : 0;
    return p;
}

int domino_head_draft(domino_head_t hd, int32_t B, const void *H, const void *L_base, const int32_t *last_tok,
                      const int32_t *teacher, const float *S_init, int32_t *tokens, float *L_final, float *S_out,
                      float *u_out, void *stream)
{
    if (!hd)
        return fail(DOMINO_EINVAL, "handle is NULL");
    const domino_head_config &c = hd->cfg;
    if (B < 1 || B > c.max_batch)
        return fail(DOMINO_EINVAL, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
    const void *req[] = {H, L_base, last_tok, tokens};
    const char *req_names[] = {"H", "L_base", "last_tok", "tokens"};
    for (int i = 0; i < 4; ++i) {
        if (!req[i])
            return fail(DOMINO_EINVAL, "%s is NULL", req_names[i]);
        if (!aligned16(req[i]))
            return fail(DOMINO_EINVAL, "%s is not 16-byte aligned", req_names[i]);
    }
    const void *opt[] = {teacher, S_init, L_final, S_out, u_out};
    const char *opt_names[] = {"teacher", "S_init", "L_final", "S_out", "u_out"};
    for (int i = 0; i < 5; ++i)
        if (opt[i] && !aligned16(opt[i]))
            return fail(DOMINO_EINVAL, "%s is not 16-byte aligned", opt_names[i]);
    const bool markov = (c.flags & DOMINO_MARKOV) != 0;
    if (markov && (S_init || S_out))
        return fail(DOMINO_EINVAL, "a Markov head has no recurrent state: S_init and S_out must be NULL");
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev != hd->device)
        return fail(DOMINO_EINVAL, "current device %d differs from the handle's device %d", dev, hd->device);

    bool persistent, resident, batched;
    if (!choose_launch(hd, B, &persistent, &resident, &batched))
        return fail(DOMINO_EUNSUPPORTED, "persistent launch needs B <= %d, or a bf16 head with r = %d, the folded "
                    "table and B <= %d, and one resident block per compute unit", BC, dhrb::r_supported(),
                    dhrb::max_batch());
    if (teacher && (c.flags & DOMINO_EXEC_POSITION_BATCHED))
        persistent = resident = batched = false;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (persistent && !(c.flags & DOMINO_EXEC_PLAIN_LAUNCH)) {
        // a cooperative launch cannot be recorded into a HIP graph
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        HIP_TRY(hipStreamIsCapturing(st, &cap), "hipStreamIsCapturing");
        if (cap != hipStreamCaptureStatusNone)
            return fail(DOMINO_EUNSUPPORTED, "the persistent launch is cooperative and cannot be captured; create the "
                        "handle with DOMINO_EXEC_PLAIN_LAUNCH or DOMINO_EXEC_STEPWISE to capture draft calls");
    }
    if (!hd->state_ready) {
        hipLaunchKernelGGL(k_clear_state, dim3(1), dim3(256), 0, st, reinterpret_cast<unsigned *>(hd->ws + hd->L.bar),
                           reinterpret_cast<uint64_t *>(hd->ws + hd->L.asy),
                           reinterpret_cast<uint32_t *>(hd->ws + hd->L.utag), 2 * c.max_batch * c.r,
                           reinterpret_cast<unsigned *>(hd->ws + hd->L.flags));
        HIP_TRY(hipGetLastError(), "launch k_clear_state");
        if (hd->L.P > hd->L.gtag) {
            // g words: no tag of the restarted generations may be found in them
            hipLaunchKernelGGL(k_clear_words, dim3(64), dim3(256), 0, st,
                               reinterpret_cast<uint64_t *>(hd->ws + hd->L.gtag), gtag_words(c));
            HIP_TRY(hipGetLastError(), "launch k_clear_words");
        }
        if (hd->L.uop > hd->L.bkeys) {
            // with the barrier generations restarting at 0, no old argmax word may keep its tag
            hipLaunchKernelGGL(k_clear_words, dim3(256), dim3(256), 0, st,
                               reinterpret_cast<uint64_t *>(hd->ws + hd->L.bkeys),
                               static_cast<size_t>(c.max_batch) * MAX_GRID);
            HIP_TRY(hipGetLastError(), "launch k_clear_words");
        }
        hd->state_ready = true;
    }
    Params p = make_params(hd, B, H, L_base, last_tok, teacher, S_init, tokens, L_final, S_out, u_out, persistent);
    if (resident && !markov)
        p.utag = reinterpret_cast<uint32_t *>(hd->ws + hd->L.utag);
    if (resident && !markov && !(c.flags & DOMINO_FOLD_EMBED))
        p.gtag = reinterpret_cast<uint64_t *>(hd->ws + hd->L.gtag);
    hd->last_stream = st;
    if (batched) {
        // A_H of every position on the matrix cores, then the one persistent launch
        p.s_hl = reinterpret_cast<uint16_t *>(hd->ws + hd->L.s_hl);
        p.wst = reinterpret_cast<const uint16_t *>(hd->ws + hd->L.wst);
        p.ldw = packed_ldw(c);
        p.bkeys = reinterpret_cast<uint64_t *>(hd->ws + hd->L.bkeys);
        p.uop = reinterpret_cast<uint4 *>(hd->ws + hd->L.uop);
        p.rb_planes = reinterpret_cast<uint16_t *>(hd->ws + hd->L.rbs);
        p.rb_bmax = rb_bmax(c);
        p.rb_ngr = rb_ngr(c);
        p.rb_ldp = rb_ldp(c);
        p.rb_ucnt = reinterpret_cast<unsigned *>(hd->ws + hd->L.ucnt);
        p.ah_external = 1;
        void *args[] = {&p};
        HIP_TRY(hipLaunchKernel(dhbat::ah_kernel(B, c.K, c.r), dim3(dhbat::ah_grid(B, c.K, c.r)),
                                dim3(dhbat::threads()), args, 0, st),
                "launch A_H (matrix cores)");
        const void *fn = dhrb::kernel(p.lbase_bf16 != 0, L_final != nullptr, c.V, markov);
        if (c.flags & DOMINO_EXEC_PLAIN_LAUNCH)
            HIP_TRY(hipLaunchKernel(fn, dim3(hd->rb_grid), dim3(dhrb::threads()), args, 0, st),
                    "hipLaunchKernel(batched persistent)");
        else
            HIP_TRY(hipLaunchCooperativeKernel(fn, dim3(hd->rb_grid), dim3(dhrb::threads()), args, 0, st),
                    "hipLaunchCooperativeKernel(batched persistent)");
        return DOMINO_OK;
    }
    if (persistent) {
        void *args[] = {&p};
        const void *fn = resident ? (markov ? dhres::markov_kernel(B) : dhres::kernel(B)) : hd->kern.persistent;
        const dim3 grid(resident ? hd->res_grid : hd->persist_grid);
        const dim3 block(resident ? dhres::threads() : NT);
        const unsigned smem = static_cast<unsigned>(resident ? hd->res_smem : hd->persist_smem);
        if (c.flags & DOMINO_EXEC_PLAIN_LAUNCH)
            HIP_TRY(hipLaunchKernel(fn, grid, block, args, smem, st), "hipLaunchKernel(persistent)");
        else
            HIP_TRY(hipLaunchCooperativeKernel(fn, grid, block, args, smem, st), "hipLaunchCooperativeKernel(persistent)");
        return DOMINO_OK;
    }
    // stepwise: prologue, update(0), state(0), then per position w2 [, g], update, state.
    // With a teacher no state waits for an argmax: the chain runs first, writing u of
    // every position (to the caller's u_out or the workspace), and the W2 products of
    // all positions follow as one launch.
    const bool pos_batched = teacher != nullptr;
    if (pos_batched && !p.u_out)
        p.u_out = reinterpret_cast<float *>(hd->ws + hd->L.u_all);
    const int h3 = 3 * c.h;
    const int g_pro = std::max(B * c.r, (h3 + NWAVE - 1) / NWAVE);
    const int g_rows = (c.r + h3 + NWAVE - 1) / NWAVE;
    const int g_g = (h3 + NWAVE - 1) / NWAVE;
    const int g_w2 = (c.V + W2_STEP_ROWS - 1) / W2_STEP_ROWS;
    const int g_upd = (B * c.h + NT - 1) / NT;
    const size_t sm_small = sizeof(float) * smem_floats_small();
    const size_t sm_w2 = sizeof(float) * smem_floats_w2(c.r, lbuf_stride(c.V, g_w2));
    const size_t sm_state = sizeof(float) * smem_floats(c.r, c.h, 0);
    // larger batches of bf16 heads take the matrix-core state dots (S passed as bf16 hi/lo planes)
    const bool state_mfma = c.wdtype == DOMINO_BF16 && c.r % 32 == 0 && c.h % 32 == 0 && B > BC;
    if (state_mfma) {
        p.s_hl = reinterpret_cast<uint16_t *>(hd->ws + hd->L.s_hl);
        p.wst = reinterpret_cast<const uint16_t *>(hd->ws + hd->L.wst);  // state_mfma implies packed rows
        p.ldw = packed_ldw(c);
    }
    auto launch_state = [&](void **sargs) -> hipError_t {
        if (state_mfma)
            return hipLaunchKernel(dhbat::state_kernel(B, c.h), dim3(dhbat::state_grid(B, c.r, c.h)),
                                   dim3(dhbat::threads()), sargs, 0, st);
        return hipLaunchKernel(hd->kern.state, dim3(g_rows), dim3(NT), sargs, sm_state, st);
    };
    // larger batches of bf16 heads: A_H on the matrix cores (H rows x W1_H rows), its own launch
    const bool ah_mfma = c.wdtype == DOMINO_BF16 && c.d % 32 == 0 && c.r % 32 == 0 && B > BC;
    if (ah_mfma) {
        p.ah_external = 1;
        void *args[] = {&p};
        HIP_TRY(hipLaunchKernel(dhbat::ah_kernel(B, c.K, c.r), dim3(dhbat::ah_grid(B, c.K, c.r)), dim3(dhbat::threads()),
                                args, 0,
                                st),
                "launch A_H (matrix cores)");
    }
    // bf16 heads with r = 256 take the matrix-core W2 kernel
    // (its load offsets are 32-bit: V < 2^22).  Drafts of more than 8 rows give it u
    // as one bf16 operand (half the matrix-core work); at most 8 rows keep the
    // hi + lo split, so their logits equal the resident kernel's bit for bit
    const bool w2_mfma = c.wdtype == DOMINO_BF16 && c.r == dhbat::r_supported() && c.V < (1 << 22);
    const bool w2_u1 = B > BC;
    auto launch_w2 = [&](Params &pw, int rows, int pos) -> hipError_t {
        int groups = w2_mfma ? dhbat::w2_groups(rows) : 0;
        void *args[] = {&pw, &pos};
        void *margs[] = {&pw, &pos, &groups};
        if (w2_mfma)
            return hipLaunchKernel(dhbat::w2_kernel(rows, pw.lbase_bf16 != 0, pw.L_final != nullptr, w2_u1),
                                   dim3(dhbat::w2_grid(rows, hd->cus)),
                                   dim3(dhbat::w2_threads(rows)), margs, dhbat::w2_smem(), st);
        return hipLaunchKernel(hd->kern.w2, dim3(g_w2), dim3(NT), args, sm_w2, st);
    };
    if (markov) {
        // Markov head: the prologue (A_H unless computed above, key clearing), then per
        // position the u launch (table gather) and the W2 launch; with a teacher, u of
        // every position in one launch and the position-batched W2 launch
        void *args[] = {&p};
        HIP_TRY(hipLaunchKernel(hd->kern.prologue, dim3(ah_mfma ? 1 : B * c.r), dim3(NT), args, sm_small, st),
                "launch prologue");
        const int nu = pos_batched ? B * c.K * c.r : B * c.r;
        const dim3 gu(std::min((nu + NT - 1) / NT, 2048));
        if (pos_batched) {
            int q = -1;
            void *uargs[] = {&p, &q};
            HIP_TRY(hipLaunchKernel(reinterpret_cast<const void *>(&k_markov_u), gu, dim3(NT), uargs, 0, st),
                    "launch Markov u (all positions)");
        } else {
            for (int pos = 0; pos < c.K; ++pos) {
                int q = pos;
                void *uargs[] = {&p, &q};
                HIP_TRY(hipLaunchKernel(reinterpret_cast<const void *>(&k_markov_u), gu, dim3(NT), uargs, 0, st),
                        "launch Markov u");
                HIP_TRY(launch_w2(p, B, pos), "launch w2");
            }
        }
    } else {
        void *args[] = {&p};
        // with A_H from its own launch the prologue only covers the 3h rows of q_0 (and g_0)
        const int g = ah_mfma ? (h3 + NWAVE - 1) / NWAVE : g_pro;
        HIP_TRY(hipLaunchKernel(hd->kern.prologue, dim3(g), dim3(NT), args, sm_small, st), "launch prologue");
        int q = 0;
        void *sargs[] = {&p, &q};
        HIP_TRY(hipLaunchKernel(reinterpret_cast<const void *>(&k_step_update), dim3(g_upd), dim3(NT), sargs,
                                sm_small, st), "launch update");
        HIP_TRY(launch_state(sargs), "launch state");
        for (int pos = 0; pos < c.K; ++pos) {
            if (!pos_batched)
                HIP_TRY(launch_w2(p, B, pos), "launch w2");
            if (pos + 1 < c.K) {
                int q = pos + 1;
                void *gargs[] = {&p, &q};
                if (!p.P)
                    HIP_TRY(hipLaunchKernel(hd->kern.g, dim3(g_g), dim3(NT), gargs, sm_small, st), "launch g");
                HIP_TRY(hipLaunchKernel(reinterpret_cast<const void *>(&k_step_update), dim3(g_upd), dim3(NT), gargs,
                                        sm_small, st), "launch update");
                HIP_TRY(launch_state(gargs), "launch state");
            }
        }
    }
    if (pos_batched) {
        // one W2 launch over the B K rows (b, pos): with K = 1 and B K rows the L_base,
        // L_final and u layouts [B, K, *] are those of B K single-position rows, and the
        // partial keys of row i sit at keys[g * B K + i]
        const int rows = B * c.K;
        Params pw = p;
        pw.B = pw.maxB = rows;
        pw.K = 1;
        pw.u_buf = p.u_out;
        pw.u_out = nullptr;
        pw.S_out = nullptr;
        const int nk = NG * rows;
        hipLaunchKernelGGL(k_keys_zero, dim3(std::min((nk + NT - 1) / NT, 1024)), dim3(NT), 0, st, p.keys, nk);
        HIP_TRY(hipGetLastError(), "launch key clear");
        HIP_TRY(launch_w2(pw, rows, 0), "launch w2 (all positions)");
        void *args[] = {&p};
        HIP_TRY(hipLaunchKernel(reinterpret_cast<const void *>(&k_rows_tokens), dim3(std::min((rows + NT - 1) / NT, 1024)),
                                dim3(NT), args, 0, st),
                "launch tokens");
    } else {
        void *args[] = {&p};
        HIP_TRY(hipLaunchKernel(reinterpret_cast<const void *>(&k_step_final), dim3(1), dim3(NT), args, 0, st),
                "launch final");
    }
    return DOMINO_OK;
}

int domino_accept_len(int32_t B, int32_t K, const int32_t *draft, const int32_t *target, int32_t *out_len,
                      void *stream)
{
    if (B < 0)
        return fail(DOMINO_EINVAL, "B=%d < 0", B);
    if (K < 1 || K > MAXK)
        return fail(DOMINO_EINVAL, "K=%d outside [1, %d]", K, MAXK);
    if (B == 0)
        return DOMINO_OK;
    if (!draft || !target || !out_len)
        return fail(DOMINO_EINVAL, "NULL pointer");
    if (!aligned16(draft) || !aligned16(target) || !aligned16(out_len))
        return fail(DOMINO_EINVAL, "pointers must be 16-byte aligned");
    hipLaunchKernelGGL(k_accept_len, dim3((B + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), B, K,
                       draft, target, out_len);
    HIP_TRY(hipGetLastError(), "launch k_accept_len");
    return DOMINO_OK;
}

static int verify_args(int32_t B, int32_t K, int32_t V)
{
    if (B < 0)
        return fail(DOMINO_EINVAL, "B=%d < 0", B);
    if (K < 1 || K > MAXK)
        return fail(DOMINO_EINVAL, "K=%d outside [1, %d]", K, MAXK);
    if (V < 1)
        return fail(DOMINO_EINVAL, "V=%d < 1", V);
    if (static_cast<long long>(B) * (K + 1) * dhverify::chunks(B, K, V) > 0x7FFFFFFFll)
        return fail(DOMINO_EUNSUPPORTED, "B=%d too large for one launch", B);
    return DOMINO_OK;
}

int domino_verify_workspace_size(int32_t B, int32_t K, int32_t V, size_t *bytes)
{
    const int rc = verify_args(B, K, V);
    if (rc)
        return rc;
    if (!bytes)
        return fail(DOMINO_EINVAL, "bytes is NULL");
    *bytes = B ? dhverify::workspace_bytes(B, K, V) : 0;
    return DOMINO_OK;
}

int domino_verify(int32_t B, int32_t K, int32_t V, const float *logits, const int32_t *draft, void *workspace,
                  size_t workspace_bytes, int32_t *target, int32_t *accept, int32_t *next, void *stream)
{
    const int rc = verify_args(B, K, V);
    if (rc)
        return rc;
    if (B == 0)
        return DOMINO_OK;
    if (!logits || !draft || !workspace || !accept || !next)
        return fail(DOMINO_EINVAL, "NULL pointer");
    if (!aligned16(logits) || !aligned16(draft) || !aligned16(workspace) || !aligned16(accept) ||
        !aligned16(next) || (target && !aligned16(target)))
        return fail(DOMINO_EINVAL, "pointers must be 16-byte aligned");
    const size_t need = dhverify::workspace_bytes(B, K, V);
    if (workspace_bytes < need)
        return fail(DOMINO_EWORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    HIP_TRY(dhverify::launch(B, K, V, logits, draft, static_cast<uint64_t *>(workspace), target, accept, next,
                             static_cast<hipStream_t>(stream)),
            "launch verify");
    return DOMINO_OK;
}

int domino_verify_noalloc(int32_t B, int32_t K, int32_t V, const float *logits, const int32_t *draft,
                          int32_t *target, int32_t *accept, int32_t *next, void *stream)
{
    const int rc = verify_args(B, K, V);
    if (rc)
        return rc;
    if (B == 0)
        return DOMINO_OK;
    if (!logits || !draft || !accept || !next)
        return fail(DOMINO_EINVAL, "NULL pointer");
    if (!aligned16(logits) || !aligned16(draft) || !aligned16(accept) || !aligned16(next) ||
        (target && !aligned16(target)))
        return fail(DOMINO_EINVAL, "pointers must be 16-byte aligned");
    const size_t need = dhverify::workspace_bytes(B, K, V);
    if (need > dhverify::SCRATCH_BYTES)
        return fail(DOMINO_EUNSUPPORTED, "B=%d, K=%d, V=%d needs %zu bytes of scratch; the static buffer holds %zu "
                    "(use domino_verify with a workspace)", B, K, V, need, dhverify::SCRATCH_BYTES);
    void *ws = nullptr;
    HIP_TRY(dhverify::scratch_address(&ws), "hipGetSymbolAddress(scratch)");
    HIP_TRY(dhverify::launch(B, K, V, logits, draft, static_cast<uint64_t *>(ws), target, accept, next,
                             static_cast<hipStream_t>(stream)),
            "launch verify");
    return DOMINO_OK;
}

int domino_head_exec_info(domino_head_t hd, int32_t B, int32_t *persistent, int32_t *w2_resident, int32_t *grid)
{
    if (!hd)
        return fail(DOMINO_EINVAL, "handle is NULL");
    if (B < 1 || B > hd->cfg.max_batch)
        return fail(DOMINO_EINVAL, "B=%d outside [1, max_batch=%d]", B, hd->cfg.max_batch);
    bool pers, res, bat;
    if (!choose_launch(hd, B, &pers, &res, &bat))
        return fail(DOMINO_EUNSUPPORTED, "persistent launch needs B <= %d, or a bf16 head with r = %d, the folded "
                    "table and B <= %d, and one resident block per compute unit", BC, dhrb::r_supported(),
                    dhrb::max_batch());
    if (persistent)
        *persistent = pers;
    if (w2_resident)
        *w2_resident = res;
    if (grid)
        *grid = !pers ? 0 : bat ? hd->rb_grid : res ? hd->res_grid : hd->persist_grid;
    return DOMINO_OK;
}

int domino_head_set_spin_limit(domino_head_t hd, uint32_t limit)
{
    if (!hd)
        return fail(DOMINO_EINVAL, "handle is NULL");
    hd->spin_limit = limit;
    return DOMINO_OK;
}

int domino_head_check_error(domino_head_t hd, uint32_t *device_flags)
{
    if (!hd)
        return fail(DOMINO_EINVAL, "handle is NULL");
    uint32_t f = 0;
    if (hd->state_ready) {
        // every stream: drafts may also have run as replays of a captured graph on a
        // stream other than the one of the last eager call
        HIP_TRY(hipDeviceSynchronize(), "hipDeviceSynchronize");
        HIP_TRY(hipMemcpy(&f, hd->ws + hd->L.flags, sizeof f, hipMemcpyDeviceToHost), "hipMemcpy(flags)");
        // the next draft clears barrier words and flags before it runs
        hd->state_ready = false;
    }
    if (device_flags)
        *device_flags = f;
    if (f)
        return fail(DOMINO_EDEVICE, "device flags 0x%x (bit0: token id outside [0,V); bit1: grid barrier timeout)", f);
    return DOMINO_OK;
}

}  // extern "C"
