// Per-phase timestamps of the persistent kernels (instrumented build only; the
// product library defines no hooks and records nothing).
//
// Thread 0 of each block writes the 100 MHz constant-rate device clock
// (s_memrealtime) into its own row of a device buffer at every marked point:
// row = block (< TRACE_BLOCKS), column = the hook's slot + TRACE_BIAS.  Slots
// outside the row are dropped, so a hook can never write past the buffer.
// Each instrumented unit defines its own buffer and an exported reader.
#pragma once
#include <hip/hip_runtime.h>

#define TRACE_BLOCKS 256
#define TRACE_SLOTS 1024

#define TRACE_MARK(buf, bias, slot)                                                                      \
    do {                                                                                                 \
        const int s_ = (slot) + (bias);                                                                  \
        if (threadIdx.x == 0 && blockIdx.x < TRACE_BLOCKS && s_ >= 0 && s_ < TRACE_SLOTS)                \
            buf[blockIdx.x * TRACE_SLOTS + s_] = __builtin_amdgcn_s_memrealtime();                       \
    } while (0)

// the same with a given value (a time noted earlier)
#define TRACE_PUT(buf, bias, slot, value)                                                                \
    do {                                                                                                 \
        const int s_ = (slot) + (bias);                                                                  \
        if (threadIdx.x == 0 && blockIdx.x < TRACE_BLOCKS && s_ >= 0 && s_ < TRACE_SLOTS)                \
            buf[blockIdx.x * TRACE_SLOTS + s_] = (value);                                                \
    } while (0)
