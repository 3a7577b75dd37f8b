// Device-side building blocks of the Domino head kernels (gfx950, wave64).
//
// Storage types, 16-byte chunk unpacking, block reductions, the packed argmax
// key and the grid barrier used by the persistent launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Threads per block and the namespace of the device code built for it: the
// library compiles these headers twice, 512 threads (namespace dh) and 256
// threads (namespace dh256, for the kernel that keeps W2 in registers).
#ifndef DH_NT
#define DH_NT 512
#endif
#ifndef DH_NS
#define DH_NS dh
#endif

// Optional instrumentation: a translation unit may define DH_TRACE(slot) before
// including these headers to record timestamps at the marked points of the
// resident persistent kernels (slot = 32 * position + point, -16..-12 for the
// anchor step, 508..511 for the prologue).  The default is a no-op.
#ifndef DH_TRACE
#define DH_TRACE(slot) ((void)(slot))
#endif
// DH_TRACE_LANDED(slot): the same mark taken once the thread's loads in flight
// have landed (an instrumented build waits for them there; the default is a no-op)
#ifndef DH_TRACE_LANDED
#define DH_TRACE_LANDED(slot) ((void)(slot))
#endif

namespace DH_NS {

constexpr int NT = DH_NT;         // threads per block
constexpr int NWAVE = NT / 64;
constexpr int NG = 16;            // barrier groups = partial argmax slots per position
constexpr int MAXK = 16;          // largest block size
constexpr int BC = 8;             // batch rows sharing one pass over W2
constexpr int BAR_STRIDE = 64;    // uints between barrier words (256 bytes: own cache line)

// Storage tag for bfloat16 (raw 16-bit patterns).
struct bf16s {
    uint16_t bits;
};

template <typename WT>
struct WT16;

template <>
struct WT16<float> {
    static constexpr int EPC = 4;  // elements per 16-byte chunk
    __device__ static inline void unpack(const uint4 &q, float *o)
    {
        o[0] = __uint_as_float(q.x);
        o[1] = __uint_as_float(q.y);
        o[2] = __uint_as_float(q.z);
        o[3] = __uint_as_float(q.w);
    }
    __device__ static inline float one(const void *base, size_t i) { return static_cast<const float *>(base)[i]; }
};

template <>
struct WT16<bf16s> {
    static constexpr int EPC = 8;
    __device__ static inline void unpack(const uint4 &q, float *o)
    {
        o[0] = __uint_as_float(q.x << 16);
        o[1] = __uint_as_float(q.x & 0xFFFF0000u);
        o[2] = __uint_as_float(q.y << 16);
        o[3] = __uint_as_float(q.y & 0xFFFF0000u);
        o[4] = __uint_as_float(q.z << 16);
        o[5] = __uint_as_float(q.z & 0xFFFF0000u);
        o[6] = __uint_as_float(q.w << 16);
        o[7] = __uint_as_float(q.w & 0xFFFF0000u);
    }
    __device__ static inline float one(const void *base, size_t i)
    {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(base)[i]) << 16);
    }
};

// 16-byte load of the chunk starting at element `elem` of a WT array.
template <typename WT>
__device__ inline uint4 ld16(const void *base, size_t elem)
{
    return *reinterpret_cast<const uint4 *>(static_cast<const char *>(base) + elem * sizeof(WT));
}

// acc + sum_e w[e] * x[e] over one chunk, in element order.
template <typename WT>
__device__ inline float dot_chunk(const uint4 &q, const float *x, float acc)
{
    float w[WT16<WT>::EPC];
    WT16<WT>::unpack(q, w);
#pragma unroll
    for (int e = 0; e < WT16<WT>::EPC; ++e)
        acc = fmaf(w[e], x[e], acc);
    return acc;
}

// fp32 chunk of EPC consecutive floats (EPC = 4 or 8) from global memory.
template <int EPC>
__device__ inline void ld_f32(const float *p, float *o)
{
    const float4 a = *reinterpret_cast<const float4 *>(p);
    o[0] = a.x;
    o[1] = a.y;
    o[2] = a.z;
    o[3] = a.w;
    if constexpr (EPC == 8) {
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        o[4] = b.x;
        o[5] = b.y;
        o[6] = b.z;
        o[7] = b.w;
    }
}

// ---- cross-lane exchange without LDS traffic --------------------------------
// DPP lane permutations (within 16-lane rows) and the gfx950 row-swap
// instructions.  Lane layouts, for lane i:
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]: reads lane i ^ 1
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]: reads lane i ^ 2
constexpr int DPP_HALF_MIRROR = 0x141;  // reads lane 7 - i within each group of 8
constexpr int DPP_ROW_MIRROR = 0x140;   // reads lane 15 - i within each row of 16

template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t v)
{
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ inline float dpp_f32(float v) { return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v))); }
template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v)
{
    return (static_cast<uint64_t>(dpp_u32<CTRL>(static_cast<uint32_t>(v >> 32))) << 32) |
           dpp_u32<CTRL>(static_cast<uint32_t>(v));
}

// v_permlane16_swap with both operands v: every lane of the row pair {0,1}
// (and {2,3}) gets the value of the even row in `even` and of the odd row in `odd`.
__device__ inline void row_pair_values(uint32_t v, uint32_t &even, uint32_t &odd)
{
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    even = s[0];
    odd = s[1];
}
// v_permlane32_swap with both operands v: every lane gets the value of its
// lane in the lower half (`lo`) and in the upper half (`hi`).
__device__ inline void half_values(uint32_t v, uint32_t &lo, uint32_t &hi)
{
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    lo = s[0];
    hi = s[1];
}

// Sum over the 2^k lanes of aligned groups (GROUP = 2, 4, 8 or 16 lanes).
// Every lane of a group gets bit-identical sums: each step adds two partial
// sums that a lane and its partner hold in swapped order.
template <int GROUP>
__device__ inline float group_sum(float v)
{
    static_assert(GROUP == 1 || GROUP == 2 || GROUP == 4 || GROUP == 8 || GROUP == 16, "group of 1..16 lanes");
    if constexpr (GROUP >= 2)
        v += dpp_f32<DPP_QUAD_XOR1>(v);
    if constexpr (GROUP >= 4)
        v += dpp_f32<DPP_QUAD_XOR2>(v);
    if constexpr (GROUP >= 8)
        v += dpp_f32<DPP_HALF_MIRROR>(v);
    if constexpr (GROUP >= 16)
        v += dpp_f32<DPP_ROW_MIRROR>(v);
    return v;
}

// Sum over the wave, bit-identical in every lane.
__device__ inline float wave_sum(float v)
{
    v = group_sum<16>(v);
    uint32_t a, b;
    row_pair_values(__float_as_uint(v), a, b);
    v = __uint_as_float(a) + __uint_as_float(b);
    half_values(__float_as_uint(v), a, b);
    return __uint_as_float(a) + __uint_as_float(b);
}

__device__ inline uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Max over the four lanes i, i+16, i+32, i+48 (the same position in each row).
__device__ inline uint64_t rows_max_u64(uint64_t v)
{
    uint32_t el, ol, eh, oh;
    row_pair_values(static_cast<uint32_t>(v), el, ol);
    row_pair_values(static_cast<uint32_t>(v >> 32), eh, oh);
    v = max_u64((static_cast<uint64_t>(eh) << 32) | el, (static_cast<uint64_t>(oh) << 32) | ol);
    half_values(static_cast<uint32_t>(v), el, ol);
    half_values(static_cast<uint32_t>(v >> 32), eh, oh);
    return max_u64((static_cast<uint64_t>(eh) << 32) | el, (static_cast<uint64_t>(oh) << 32) | ol);
}

__device__ inline uint64_t wave_max_u64(uint64_t v)
{
    v = max_u64(v, dpp_u64<DPP_QUAD_XOR1>(v));
    v = max_u64(v, dpp_u64<DPP_QUAD_XOR2>(v));
    v = max_u64(v, dpp_u64<DPP_HALF_MIRROR>(v));
    v = max_u64(v, dpp_u64<DPP_ROW_MIRROR>(v));
    return rows_max_u64(v);
}

// bfloat16 bits of x, rounded to nearest even (finite x).
__device__ inline uint32_t bf16_rne_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Sums M per-thread values over the block in a fixed order.  Results land in
// red[NWAVE*M + m]; the caller syncs before reusing `red`.
template <int M>
__device__ inline void block_sum(float (&v)[M], float *red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < M; ++m)
        v[m] = wave_sum(v[m]);
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < M; ++m)
            red[wave * M + m] = v[m];
    }
    __syncthreads();
    if (threadIdx.x < M) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w)
            s += red[w * M + threadIdx.x];
        red[NWAVE * M + threadIdx.x] = s;
    }
    __syncthreads();
}

// The GRU and SiLU nonlinearities, on the hardware's base-2 exponential and
// reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp each) instead of the library's
// correctly rounded exp and IEEE division: errors of a few 1e-7, far inside the
// 1e-4 bound on S and u, in a fraction of the instructions.  Every kernel uses
// these, so the launch paths stay bitwise equal.
//   sigmoid x = 1 / (1 + 2^(-x log2 e))  (x -> +inf: 1; x -> -inf: 1 / inf = 0)
//   tanh x    = 1 - 2 / (1 + 2^(2 x log2 e))  (+inf: 1; -inf: 1 - 2 = -1)
__device__ inline float sigmoidf_(float x)
{
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}
__device__ inline float tanhf_(float x)
{
    return 1.f - 2.f * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * 2.88539008177792681f));
}

// Argmax key: larger key = better candidate.  High word orders the float
// (NaN above +inf, -0 folded into +0); low word prefers the lower index.
__device__ inline uint64_t argmax_key(float f, uint32_t idx)
{
    // selects only (no branches)
    const uint32_t bits = (f == 0.f) ? 0u : __float_as_uint(f);
    uint32_t ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
    ord = (f != f) ? 0xFFFFFFFFu : ord;
    return (static_cast<uint64_t>(ord) << 32) | (0xFFFFFFFFu - idx);
}

__device__ inline uint32_t key_index(uint64_t key) { return 0xFFFFFFFFu - static_cast<uint32_t>(key); }

// The exchange words live in global memory.  Accesses through a global-address-space
// pointer compile to global loads and stores, which count only against the vector
// memory counter; through a generic pointer they become flat accesses, which also count
// against the LDS counter, so every later wait for an LDS read would wait for them too
// (an agent-scope store then costs a memory round trip at the next LDS read).
template <typename T>
__device__ inline __attribute__((address_space(1))) T *gmem(T *p)
{
    return (__attribute__((address_space(1))) T *)p;
}
template <typename T>
__device__ inline const __attribute__((address_space(1))) T *gmem(const T *p)
{
    return (const __attribute__((address_space(1))) T *)p;
}

__device__ inline uint64_t ld_agent_u64(const uint64_t *p)
{
    return __hip_atomic_load(gmem(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Cross-block exchange.  Values handed from one block to another inside a
// persistent launch (activations, state products, argmax keys) are written
// and read with agent-scope atomic accesses, which bypass the per-XCD L2
// caches that are not coherent with each other.  The barrier below then only
// has to order completed accesses; it needs no L2 write-back or invalidate.
// ---------------------------------------------------------------------------
__device__ inline void xst(float *p, float v) { __hip_atomic_store(gmem(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float xld(const float *p)
{
    return __hip_atomic_load(gmem(const_cast<float *>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide failure flag of a persistent kernel (bounded waits that timed
// out).  Cleared once at kernel start (block_fail_init, before the first block
// sync) and never reset: a failure ends the kernel.  block_failed() costs one
// block sync instead of the three of __syncthreads_and.
__device__ inline int &block_fail_word()
{
    __shared__ int w;
    return w;
}
__device__ inline void block_fail_init()
{
    if (threadIdx.x == 0)
        block_fail_word() = 0;
    __syncthreads();
}
__device__ inline bool block_failed(int ok)
{
    if (!ok)
        block_fail_word() = 1;
    __syncthreads();
    return block_fail_word() != 0;
}

// ---------------------------------------------------------------------------
// Grid barrier for a cooperative launch (every block resident), in two halves
// so that loads of data published before the previous barrier can be issued
// between them.
// Arrival: every thread waits for its own memory operations to complete, the
// block syncs, and thread 0 writes the new generation into the block's own
// arrival slot.  Wait: every block polls every slot itself (thread i polls
// slots i, i + NT, ...) until each holds at least the new generation; there is
// no central block and no release word.  Layout of `bar` (uints): arrival
// slot of block b at BAR_SLOTS + b.  Generations only grow: a block starts a
// launch from the value of its own slot, and at the end of a launch writes its
// final generation there (barrier_finish), so every slot agrees at the next
// launch and the words need clearing only once.  Spins are bounded: a slot
// not reached after `spin_limit` polls sets DOMINO_FLAG_SYNC_TIMEOUT (bit 1)
// and the wait returns false in every thread of that block; the caller must
// then leave the kernel.
// ---------------------------------------------------------------------------
constexpr int BAR_SLOTS = NG * BAR_STRIDE;
constexpr int MAX_GRID = 1024;
constexpr int BAR_WORDS_ALL = BAR_SLOTS + MAX_GRID;

__device__ inline unsigned *bar_slots(unsigned *bar) { return bar + BAR_SLOTS; }

__device__ inline unsigned barrier_gen_init(unsigned *bar)
{
    return __hip_atomic_load(gmem(&bar_slots(bar)[blockIdx.x]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// End of a launch: record the block's final generation in its slot.
__device__ inline void barrier_finish(unsigned *bar, unsigned gen)
{
    if (threadIdx.x == 0)
        __hip_atomic_store(gmem(&bar_slots(bar)[blockIdx.x]), gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// `gen` is tracked identically by every thread of the block.
__device__ inline void grid_arrive(unsigned *bar, unsigned gen)
{
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(gmem(&bar_slots(bar)[blockIdx.x]), gen + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline bool grid_wait(unsigned *bar, unsigned &gen, unsigned spin_limit, unsigned *flags)
{
    const unsigned next = gen + 1;
    const unsigned *slots = bar_slots(bar);
    int ok = 1;
    for (int i = threadIdx.x; i < static_cast<int>(gridDim.x); i += NT) {
        unsigned spins = 0;
        while (static_cast<int>(__hip_atomic_load(gmem(const_cast<unsigned *>(&slots[i])), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT) - next) < 0) {
            if (++spins > spin_limit) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    gen = next;
    const bool failed = block_failed(ok);
    if (failed && threadIdx.x == 0)
        __hip_atomic_fetch_or(gmem(flags), 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return !failed;
}

__device__ inline bool grid_sync(unsigned *bar, unsigned &gen, unsigned spin_limit, unsigned *flags)
{
    grid_arrive(bar, gen);
    return grid_wait(bar, gen, spin_limit, flags);
}

// ---------------------------------------------------------------------------
// Barrier that also reduces the greedy argmax (persistent launch, V <= 2^18).
// Arrival: each block stores, for each of its nb batch rows, its local argmax
// key into its own 64-bit word, with the 14 spare high bits of the index
// field replaced by the generation (an index below 2^18 leaves the top 14 of
// its 32 bits unused).  Wait: every block reads every word until it
// carries the new generation and reduces the keys itself, leaving the tokens
// of this position in tok[0..nb) (visible to the whole block on return).  Generations compare modulo 2^14 (a word is
// ready when it is at most 2^13 ahead).  The words of even and odd generations
// are kept apart: a block may arrive at the next argmax barrier while a slower
// one still reads the words of this one (nothing between two argmax barriers
// waits for every block), but it cannot arrive at the one after before every
// block has arrived at the next, which each does only after its wait here.
// Arrival words: asy[(gen & 1) * MAX_GRID * BC + blk * BC + b].
// ---------------------------------------------------------------------------
constexpr int ASYNC_WORDS = 2 * MAX_GRID * BC;

__device__ inline size_t argmax_word(unsigned gen, int blk, int b)
{
    return static_cast<size_t>(gen & 1u) * (MAX_GRID * BC) + static_cast<size_t>(blk) * BC + b;
}
constexpr uint64_t KEY_ORD_MASK = 0xFFFFFFFF00000000ull;
constexpr uint64_t KEY_IDX_MASK = 0x3FFFFull;

__device__ inline uint64_t argmax_key18(float f, uint32_t idx)
{
    return (argmax_key(f, 0) & KEY_ORD_MASK) | (KEY_IDX_MASK - idx);
}

// local_key[b] must have been written by thread b, or before a block sync.
// Arrival also publishes the block's earlier stores (like grid_arrive): after
// the wait every block sees them.
__device__ inline void argmax_arrive(uint64_t *asy, unsigned gen, const uint64_t *local_key, int nb)
{
    const uint64_t g14 = static_cast<uint64_t>((gen + 1) & 0x3FFFu) << 18;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    // the words of rows nb..BC-1 get the generation too (with key 0): every word
    // is then at most one generation old, and a later launch with more rows never
    // takes one written many launches ago for a current one
    if (threadIdx.x < BC) {
        const uint64_t k = threadIdx.x < nb ? local_key[threadIdx.x] & (KEY_ORD_MASK | KEY_IDX_MASK) : 0;
        __hip_atomic_store(gmem(&asy[argmax_word(gen + 1, blockIdx.x, threadIdx.x)]), k | g14, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ inline bool argmax_wait(const uint64_t *asy, unsigned &gen, int nb, int *tok, unsigned spin_limit,
                                   unsigned *flags)
{
    __shared__ uint64_t s_red[NWAVE * BC];
    const unsigned next = gen + 1;
    const unsigned g14 = next & 0x3FFFu;
    const int total = static_cast<int>(gridDim.x) * nb;
    uint64_t best[BC];
#pragma unroll
    for (int b = 0; b < BC; ++b)
        best[b] = 0;
    int ok = 1;
    for (int e = threadIdx.x; e < total; e += NT) {
        const int blk = e / nb, b = e % nb;
        const uint64_t *wp = &asy[argmax_word(next, blk, b)];
        uint64_t w;
        unsigned spins = 0;
        for (;;) {
            w = __hip_atomic_load(gmem(const_cast<uint64_t *>(wp)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (((static_cast<unsigned>(w >> 18) - g14) & 0x3FFFu) < 0x2000u)
                break;
            if (++spins > spin_limit) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const uint64_t k = w & (KEY_ORD_MASK | KEY_IDX_MASK);
#pragma unroll
        for (int bb = 0; bb < BC; ++bb)
            if (bb == b)
                best[bb] = max_u64(best[bb], k);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int b = 0; b < BC; ++b) {
        if (b < nb) {
            const uint64_t m = wave_max_u64(best[b]);
            if (lane == 0)
                s_red[wave * BC + b] = m;
        }
    }
    gen = next;
    const bool failed = block_failed(ok);  // also the sync after the s_red writes
    if (threadIdx.x < nb) {
        uint64_t m = 0;
        for (int w = 0; w < NWAVE; ++w)
            m = max_u64(m, s_red[w * BC + threadIdx.x]);
        tok[threadIdx.x] = m ? static_cast<int>(KEY_IDX_MASK - (m & KEY_IDX_MASK)) : 0;
    }
    if (failed && threadIdx.x == 0)
        __hip_atomic_fetch_or(gmem(flags), 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();  // tok visible to the block
    return !failed;
}

__device__ inline bool grid_argmax_sync(uint64_t *asy, unsigned &gen, const uint64_t *local_key, int nb, int *tok,
                                        unsigned spin_limit, unsigned *flags)
{
    argmax_arrive(asy, gen, local_key, nb);
    return argmax_wait(asy, gen, nb, tok, spin_limit, flags);
}

}  // namespace DH_NS
