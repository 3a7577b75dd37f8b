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

__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

__device__ inline uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o);
        uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o);
        uint64_t w = (static_cast<uint64_t>(hi) << 32) | lo;
        v = w > v ? w : v;
    }
    return v;
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

__device__ inline float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }

// Argmax key: larger key = better candidate.  High word orders the float
// (NaN above +inf, -0 folded into +0); low word prefers the lower index.
__device__ inline uint64_t argmax_key(float f, uint32_t idx)
{
    uint32_t ord;
    if (f != f) {
        ord = 0xFFFFFFFFu;
    } else {
        uint32_t bits = (f == 0.f) ? 0u : __float_as_uint(f);
        ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
    }
    return (static_cast<uint64_t>(ord) << 32) | (0xFFFFFFFFu - idx);
}

__device__ inline uint32_t key_index(uint64_t key) { return 0xFFFFFFFFu - static_cast<uint32_t>(key); }

__device__ inline uint64_t ld_agent_u64(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Cross-block exchange.  Values handed from one block to another inside a
// persistent launch (activations, state products, argmax keys) are written
// and read with agent-scope atomic accesses, which bypass the per-XCD L2
// caches that are not coherent with each other.  The barrier below then only
// has to order completed accesses; it needs no L2 write-back or invalidate.
// ---------------------------------------------------------------------------
__device__ inline void xst(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float xld(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Grid barrier for a cooperative launch (one block per compute unit).
// Arrival: every thread waits for its own memory operations to complete, the
// block syncs, and thread 0 writes the new generation into the block's own
// arrival slot (no contended counter).  Block 0 polls all slots; when every
// block has arrived it writes the generation into NG release words (one per
// group of blocks, on separate cache lines) that the other blocks poll.
// Layout of `bar` (uints): release word g at g*BAR_STRIDE, arrival slots from
// BAR_SLOTS.  Generations only grow, so the words carry over between launches
// and need clearing only once.  Spins are bounded: past `spin_limit` polls the
// block sets DOMINO_FLAG_SYNC_TIMEOUT (bit 1) and grid_sync returns false in
// every thread of that block; the caller must then leave the kernel.
// ---------------------------------------------------------------------------
constexpr int BAR_SLOTS = NG * BAR_STRIDE;
constexpr int MAX_GRID = 1024;
constexpr int BAR_WORDS_ALL = BAR_SLOTS + MAX_GRID;

__device__ inline unsigned *bar_release(unsigned *bar, int g) { return bar + g * BAR_STRIDE; }

__device__ inline unsigned barrier_gen_init(unsigned *bar)
{
    return __hip_atomic_load(bar_release(bar, blockIdx.x % NG), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// `gen` is tracked identically by every thread of the block.
__device__ inline bool grid_sync(unsigned *bar, unsigned &gen, unsigned spin_limit, unsigned *flags)
{
    __shared__ int s_ok;
    const unsigned next = gen + 1;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    unsigned *slots = bar + BAR_SLOTS;
    if (threadIdx.x == 0)
        __hip_atomic_store(&slots[blockIdx.x], next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1;
    if (blockIdx.x == 0) {
        unsigned spins = 0;
        for (;;) {
            int mine = 1;
            for (int i = threadIdx.x; i < static_cast<int>(gridDim.x); i += blockDim.x)
                if (__hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != next)
                    mine = 0;
            if (__syncthreads_and(mine))
                break;
            if (++spins > spin_limit) {
                ok = 0;
                break;
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        if (threadIdx.x < NG)
            __hip_atomic_store(bar_release(bar, threadIdx.x), next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!ok && threadIdx.x == 0)
            __hip_atomic_fetch_or(flags, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0) {
        unsigned spins = 0;
        const unsigned *rel = bar_release(bar, blockIdx.x % NG);
        while (__hip_atomic_load(const_cast<unsigned *>(rel), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != next) {
            if (++spins > spin_limit) {
                __hip_atomic_fetch_or(flags, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        s_ok = ok;
    }
    gen = next;
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return s_ok != 0;
}

// ---------------------------------------------------------------------------
// Barrier that also reduces the greedy argmax (persistent launch, V <= 2^18).
// Each block arrives by storing, for each of its nb batch rows, its local
// argmax key into its own 64-bit arrival word, with the 14 spare high bits of
// the index field replaced by the generation (an index below 2^18 leaves the
// top 14 of its 32 bits unused).  Block 0 polls all arrival words; the poll
// that sees every word at the new generation also holds every partial key, so
// it reduces them directly and releases the barrier with 64-bit words
// {generation, token} (one per batch row and group).  Every block leaves with
// the tokens of this position in tok[0..nb).  Arrival words: aslot[blk*BC + b];
// release words: arel[g*ASYNC_STRIDE + b].
// ---------------------------------------------------------------------------
constexpr int ASYNC_STRIDE = 32;  // u64 per release group (256 bytes)
constexpr int ASYNC_WORDS = MAX_GRID * BC + NG * ASYNC_STRIDE;
constexpr uint64_t KEY_ORD_MASK = 0xFFFFFFFF00000000ull;
constexpr uint64_t KEY_IDX_MASK = 0x3FFFFull;

__device__ inline uint64_t argmax_key18(float f, uint32_t idx)
{
    return (argmax_key(f, 0) & KEY_ORD_MASK) | (KEY_IDX_MASK - idx);
}

__device__ inline bool grid_argmax_sync(uint64_t *asy, unsigned &gen, const uint64_t *local_key, int nb, int *tok,
                                        unsigned spin_limit, unsigned *flags)
{
    __shared__ int s_ok;
    __shared__ uint64_t s_red[NWAVE * BC];
    const unsigned next = gen + 1;
    const uint64_t g14 = static_cast<uint64_t>(next & 0x3FFFu) << 18;
    uint64_t *aslot = asy;
    uint64_t *arel = asy + MAX_GRID * BC;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x < nb) {
        const uint64_t k = local_key[threadIdx.x];
        __hip_atomic_store(&aslot[blockIdx.x * BC + threadIdx.x], (k & (KEY_ORD_MASK | KEY_IDX_MASK)) | g14,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    int ok = 1;
    if (blockIdx.x == 0) {
        const int total = static_cast<int>(gridDim.x) * nb;
        uint64_t best[BC];
        unsigned spins = 0;
        for (;;) {
            int mine = 1;
#pragma unroll
            for (int b = 0; b < BC; ++b)
                best[b] = 0;
            for (int e = threadIdx.x; e < total; e += blockDim.x) {
                const int blk = e / nb, b = e % nb;
                const uint64_t w = __hip_atomic_load(&aslot[blk * BC + b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (((w >> 18) & 0x3FFFu) != (next & 0x3FFFu))
                    mine = 0;
                const uint64_t k = w & (KEY_ORD_MASK | KEY_IDX_MASK);
#pragma unroll
                for (int bb = 0; bb < BC; ++bb)
                    if (bb == b && k > best[bb])
                        best[bb] = k;
            }
            if (__syncthreads_and(mine))
                break;
            if (++spins > spin_limit) {
                ok = 0;
                break;
            }
        }
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int b = 0; b < BC; ++b) {
            const uint64_t m = wave_max_u64(best[b]);
            if (lane == 0)
                s_red[wave * BC + b] = m;
        }
        __syncthreads();
        if (threadIdx.x < nb) {
            uint64_t m = 0;
            for (int w = 0; w < NWAVE; ++w)
                m = s_red[w * BC + threadIdx.x] > m ? s_red[w * BC + threadIdx.x] : m;
            const uint32_t t = m ? static_cast<uint32_t>(KEY_IDX_MASK - (m & KEY_IDX_MASK)) : 0u;
            const uint64_t rel = (static_cast<uint64_t>(next) << 32) | t;
            for (int g = 0; g < NG; ++g)
                __hip_atomic_store(&arel[g * ASYNC_STRIDE + threadIdx.x], rel, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (!ok && threadIdx.x == 0)
            __hip_atomic_fetch_or(flags, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0) {
        const int g = blockIdx.x % NG;
        unsigned spins = 0;
        for (;;) {
            int done = 1;
            for (int b = 0; b < nb; ++b) {
                const uint64_t w =
                    __hip_atomic_load(&arel[g * ASYNC_STRIDE + b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (static_cast<unsigned>(w >> 32) != next)
                    done = 0;
                else
                    tok[b] = static_cast<int>(static_cast<uint32_t>(w));
            }
            if (done)
                break;
            if (++spins > spin_limit) {
                __hip_atomic_fetch_or(flags, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        s_ok = ok;
    }
    gen = next;
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return s_ok != 0;
}

}  // namespace DH_NS
