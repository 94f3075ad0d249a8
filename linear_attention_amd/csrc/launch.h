// Kernel launchers behind the C ABI.  Arguments are already validated on the
// host; the kernels still clamp token ranges and check slot indices.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// Token-recurrent path: one workgroup per (request, head), state in registers.
// Request b covers tokens [cu_seqlens[b], cu_seqlens[b+1]) when cu_seqlens is
// non-null, else [b*tokens_per_req, (b+1)*tokens_per_req).  The final state
// goes to state_out[b] when state_out is non-null, else back to the pool slot.
hipError_t launch_recurrent(bool bf16, const void *q, const void *k, const void *v,
                            const int32_t *cu_seqlens, int tokens_per_req, int batch,
                            int num_heads, int64_t total_tokens, float *pool,
                            int64_t pool_slots, const int32_t *slot_idx, const float *slopes,
                            void *out, float *state_out, hipStream_t stream);

// Chunked bf16 MFMA prefill: one workgroup per (request, head, 32-column
// block of the state), chunks of 64 tokens.
hipError_t launch_prefill_chunked(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                  const int32_t *cu_seqlens, int batch, int num_heads,
                                  int64_t total_tokens, float *pool, int64_t pool_slots,
                                  const int32_t *slot_idx, const float *slopes, uint16_t *out,
                                  hipStream_t stream);

}  // namespace la
