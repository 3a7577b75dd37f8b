// The batched resident kernel with its RB_MARK hooks recording into trace_rb_buf.
#include "trace_buf.h"

__device__ unsigned long long trace_rb_buf[TRACE_BLOCKS * TRACE_SLOTS];
#define RB_MARK(slot) TRACE_MARK(trace_rb_buf, 0, slot)
#define RB_MARK_LANDED(slot)                                                                             \
    do {                                                                                                 \
        __builtin_amdgcn_s_waitcnt(0);                                                                   \
        TRACE_MARK(trace_rb_buf, 0, slot);                                                               \
    } while (0)
// the W2 phase's group points: kept in LDS while the phase runs, written to slots
// 64 pos + 8 + i afterwards
__shared__ unsigned long long trace_rb_gt[32];
#define RB_GMARK(i)                                                                                      \
    do {                                                                                                 \
        if (threadIdx.x == 0 && (i) < 32)                                                                \
            trace_rb_gt[(i)] = __builtin_amdgcn_s_memrealtime();                                         \
    } while (0)
#define RB_GFLUSH(pos, n)                                                                                \
    do {                                                                                                 \
        for (int i_ = 0; i_ < (n) && i_ < 32; ++i_)                                                      \
            TRACE_PUT(trace_rb_buf, 0, 64 * (pos) + 8 + i_, trace_rb_gt[i_]);                            \
    } while (0)

#include "../domino_head_rb.hip"

// Copies the whole buffer (TRACE_BLOCKS x TRACE_SLOTS u64, row per block) to `host`.
extern "C" int domino_trace_read_rb(void *host)
{
    return static_cast<int>(hipMemcpyFromSymbol(host, HIP_SYMBOL(trace_rb_buf), sizeof(trace_rb_buf)));
}

// Zeroes the buffer (synchronous).
extern "C" int domino_trace_clear_rb(void)
{
    static unsigned long long zero[TRACE_BLOCKS * TRACE_SLOTS];
    return static_cast<int>(hipMemcpyToSymbol(HIP_SYMBOL(trace_rb_buf), zero, sizeof(zero)));
}
