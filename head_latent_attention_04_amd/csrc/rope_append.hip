// Standalone RoPE rotation and cache append: one work-group per (new token, group of 32 heads); the
// per-token work and its citations are in rope_device.h.
#include "rope_device.h"

namespace mla {

__global__ void __launch_bounds__(256) rope_append_kernel(CacheView cache, int n_heads, const int32_t* __restrict__ token_seq,
                                                           const int32_t* __restrict__ token_pos,
                                                           const uint16_t* __restrict__ c_kv,
                                                           const uint16_t* __restrict__ k_rope,
                                                           uint16_t* __restrict__ q_rope, double log2_theta) {
  __shared__ double s_cs[kDr];
  rope_token_group(cache, n_heads, blockIdx.x, blockIdx.y, token_seq, token_pos, c_kv, k_rope, q_rope, log2_theta,
                   nullptr, 0, s_cs);
}

hipError_t launch_rope_append(const CacheView& cache, int n_heads, int num_tokens, const int32_t* token_seq,
                              const int32_t* token_pos, const uint16_t* c_kv, const uint16_t* k_rope,
                              uint16_t* q_rope, float theta, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int groups = q_rope != nullptr ? rope_groups(n_heads) : 1;
  hipLaunchKernelGGL(rope_append_kernel, dim3(num_tokens, groups), dim3(256), 0, stream, cache, n_heads, token_seq,
                     token_pos, c_kv, k_rope, q_rope, log2((double)theta));
  return hipGetLastError();
}

}  // namespace mla
