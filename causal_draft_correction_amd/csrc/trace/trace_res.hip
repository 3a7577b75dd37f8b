// The resident B <= 8 kernels with their DH_TRACE hooks recording into
// trace_res_buf (slot + 64: the anchor step's hooks use slots -16..-12).
#include "trace_buf.h"

__device__ unsigned long long trace_res_buf[TRACE_BLOCKS * TRACE_SLOTS];
#define DH_TRACE(slot) TRACE_MARK(trace_res_buf, 64, slot)
#define DH_TRACE_LANDED(slot)                                                                            \
    do {                                                                                                 \
        __builtin_amdgcn_s_waitcnt(0);                                                                   \
        TRACE_MARK(trace_res_buf, 64, slot);                                                             \
    } while (0)

#include "../domino_head_res.hip"

// Copies the whole buffer (TRACE_BLOCKS x TRACE_SLOTS u64, row per block) to `host`.
extern "C" int domino_trace_read_res(void *host)
{
    return static_cast<int>(hipMemcpyFromSymbol(host, HIP_SYMBOL(trace_res_buf), sizeof(trace_res_buf)));
}

// Zeroes the buffer (synchronous).
extern "C" int domino_trace_clear_res(void)
{
    static unsigned long long zero[TRACE_BLOCKS * TRACE_SLOTS];
    return static_cast<int>(hipMemcpyToSymbol(HIP_SYMBOL(trace_res_buf), zero, sizeof(zero)));
}
