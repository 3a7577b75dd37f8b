// Greedy verify step of speculative decoding on the device.
//
// The target model checks a whole drafted block in one parallel pass and keeps
// what it would have produced itself (paper.oopus.info review, section 一);
// every accepted token is the target's own (researchpapers.dev summary, 关键结果
// and 常见问题).  For B drafted blocks of K tokens and the target's logits rows
// [B, K+1, V] (row j scores the token after the context plus the first j draft
// tokens; row K follows the whole draft):
//     target[b][j] = argmax_v logits[b][j][v]     (lowest index on ties, a NaN
//                                                  above every number, -0 == +0)
//     accept[b]    = first j < K with draft[b][j] != target[b][j], else K
//     next[b]      = target[b][accept[b]]          (committed after the prefix)
//
// The argmax reads 4 V bytes per row once, so it is bound by HBM bandwidth.
// k_verify_rows splits each row into `nch` chunks, one 256-thread block per
// (row, chunk) so that even B = 1 fills the chip, keeps eight 16-byte
// non-temporal loads per thread in flight and writes one packed key per block
// to the workspace (nothing to clear: every key slot is written).
// k_verify_final reduces the keys of one batch row in one block.
#define DH_NT 256
#define DH_NS dhv
#include "dh_common.h"
#include "dh_verify.h"

#include <mutex>

namespace DH_NS {

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int VF_UNROLL = 8;          // 16-byte loads per thread in flight
constexpr int VF_MIN_CHUNK = 4096;    // floats per block at least (16 KiB)
constexpr int VF_TARGET_BLOCKS = 2048;

__global__ __launch_bounds__(NT) void k_verify_rows(const float *logits, int V, int nch, int chunk, uint64_t *keys)
{
    __shared__ uint64_t red[NWAVE];
    const int row = blockIdx.x / nch, c = blockIdx.x % nch;
    const int v0 = c * chunk, v1 = v0 + chunk < V ? v0 + chunk : V;
    const float *src = logits + static_cast<size_t>(row) * V;
    uint64_t best = 0;
    if ((V & 3) == 0) {
        // rows are 16-byte aligned and chunk is a multiple of 4, so every load
        // below lies inside [v0, v1)
        constexpr int STEP = NT * 4;
        for (int v = v0 + threadIdx.x * 4; v < v1; v += STEP * VF_UNROLL) {
            f4v x[VF_UNROLL];
#pragma unroll
            for (int u = 0; u < VF_UNROLL; ++u)
                if (v + u * STEP < v1)
                    x[u] = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(src + v + u * STEP));
#pragma unroll
            for (int u = 0; u < VF_UNROLL; ++u)
                if (v + u * STEP < v1) {
                    const uint32_t i = static_cast<uint32_t>(v + u * STEP);
                    best = max_u64(best, argmax_key(x[u].x, i));
                    best = max_u64(best, argmax_key(x[u].y, i + 1));
                    best = max_u64(best, argmax_key(x[u].z, i + 2));
                    best = max_u64(best, argmax_key(x[u].w, i + 3));
                }
        }
    } else {
        for (int v = v0 + threadIdx.x; v < v1; v += NT)
            best = max_u64(best, argmax_key(__builtin_nontemporal_load(src + v), static_cast<uint32_t>(v)));
    }
    best = wave_max_u64(best);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t m = red[0];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w)
            m = max_u64(m, red[w]);
        keys[blockIdx.x] = m;  // 0 only for a chunk past the end of the row
    }
}

// One block per batch row: every thread loads its share of the row's (K+1) nch
// keys at once and folds them into the K+1 LDS slots; then lane j of wave 0
// takes row j's token, and one ballot finds the first draft token that differs.
__global__ __launch_bounds__(NT) void k_verify_final(int K, int nch, const uint64_t *keys, const int32_t *draft,
                                                     int32_t *target, int32_t *accept, int32_t *next)
{
    __shared__ unsigned long long best[MAXK + 1];
    const int b = blockIdx.x, lane = threadIdx.x & 63;
    const int n = (K + 1) * nch;
    const uint64_t *kb = keys + static_cast<size_t>(b) * n;
    // the draft tokens go out with the key loads
    const int dj = (threadIdx.x < K) ? draft[static_cast<size_t>(b) * K + threadIdx.x] : 0;
    if (threadIdx.x <= K)
        best[threadIdx.x] = 0ull;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += NT)
        atomicMax(&best[e / nch], static_cast<unsigned long long>(kb[e]));
    __syncthreads();
    if (threadIdx.x >= 64)
        return;
    const int t = lane <= K ? static_cast<int>(key_index(best[lane])) : 0;
    if (target && lane <= K)
        target[static_cast<size_t>(b) * (K + 1) + lane] = t;
    const uint64_t differ = __ballot(lane < K && dj != t);
    const int a = differ ? __ffsll(static_cast<unsigned long long>(differ)) - 1 : K;
    const int nt = __shfl(t, a);
    if (lane == 0) {
        accept[b] = a;
        next[b] = nt;
    }
}

}  // namespace DH_NS

// Scratch of the allocation-free verify entry point: the argmax keys of one call
// live in this file-scope device array instead of a caller's workspace.  In host
// code its name is only a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress, once per device (each device holds its own copy).
static __device__ __align__(256) uint64_t scratch[dhverify::SCRATCH_BYTES / sizeof(uint64_t)];

namespace dhverify {

using namespace dhv;

hipError_t scratch_address(void **out)
{
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static void *addr[MAX_DEVICES];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

int chunks(int B, int K, int V)
{
    const long long rows = static_cast<long long>(B) * (K + 1);
    long long n = (VF_TARGET_BLOCKS + rows - 1) / (rows > 0 ? rows : 1);
    const long long cap = V / VF_MIN_CHUNK > 1 ? V / VF_MIN_CHUNK : 1;
    if (n > cap)
        n = cap;
    return n < 1 ? 1 : static_cast<int>(n);
}

size_t workspace_bytes(int B, int K, int V)
{
    return sizeof(uint64_t) * static_cast<size_t>(B) * (K + 1) * chunks(B, K, V);
}

hipError_t launch(int B, int K, int V, const float *logits, const int32_t *draft, uint64_t *keys, int32_t *target,
                  int32_t *accept, int32_t *next, hipStream_t st)
{
    const int nch = chunks(B, K, V);
    int chunk = (V + nch - 1) / nch;
    chunk = (chunk + 3) & ~3;
    const unsigned grid = static_cast<unsigned>(static_cast<size_t>(B) * (K + 1) * nch);
    hipLaunchKernelGGL(k_verify_rows, dim3(grid), dim3(NT), 0, st, logits, V, nch, chunk, keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_verify_final, dim3(B), dim3(NT), 0, st, K, nch, static_cast<const uint64_t *>(keys), draft,
                       target, accept, next);
    return hipGetLastError();
}

}  // namespace dhverify
