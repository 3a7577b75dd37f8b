// Greedy verify step: launch shape and entry of the device code in domino_verify.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dhverify {

// Chunks each target row is split into (one block per row and chunk).
int chunks(int B, int K, int V);
// Workspace bytes for B blocks of K drafted tokens over a vocabulary of V:
// one 8-byte packed argmax key per (row, chunk).
size_t workspace_bytes(int B, int K, int V);
// Bytes of the file-scope device scratch the allocation-free entry point uses
// in place of a workspace (a call needs workspace_bytes(B, K, V) of it).
constexpr size_t SCRATCH_BYTES = size_t(1) << 20;
// Device address of that scratch on the current device (looked up on the first
// call per device, then cached).
hipError_t scratch_address(void **out);
// Both launches on `st`; target may be NULL.  Arguments were checked by the caller.
hipError_t launch(int B, int K, int V, const float *logits, const int32_t *draft, uint64_t *keys, int32_t *target,
                  int32_t *accept, int32_t *next, hipStream_t st);

}  // namespace dhverify
