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
// Both launches on `st`; target may be NULL.  Arguments were checked by the caller.
hipError_t launch(int B, int K, int V, const float *logits, const int32_t *draft, uint64_t *keys, int32_t *target,
                  int32_t *accept, int32_t *next, hipStream_t st);

}  // namespace dhverify
