// RoPE rotation of the decoupled key/query and append of the latent row to the paged cache.
//
// RoPE as on "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA與ROPE的融合": position m turns pair i by
// m * theta_i, theta_i = base^(-2i/d) with d = d_R (the decoupled part). Pairs are interleaved
// (x_{2i}, x_{2i+1}), matching the complex freqs_cis rotation the module of
// "论文复现工坊 No.4", section 2, takes as input. The row written is [c_KV | R_m k_R]
// (the split order of that module's wkv_a output).
//
// One work-group of 256 threads per new token. The angle m * theta_i is formed and turned in
// fp64 (positions reach 1.3e5 rad, where an fp32 angle would be off by ~1e-2 rad) and each result is
// rounded once to bf16.
#include "mla_internal.h"

namespace mla {

__global__ void __launch_bounds__(256) rope_append_kernel(CacheView cache, int n_heads, const int32_t* __restrict__ token_seq,
                                                           const int32_t* __restrict__ token_pos,
                                                           const uint16_t* __restrict__ c_kv,
                                                           const uint16_t* __restrict__ k_rope,
                                                           uint16_t* __restrict__ q_rope, double log2_theta) {
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int seq = token_seq[i];
  const int pos = token_pos[i];
  uint16_t* row = cache.data + row_offset(cache, seq, pos);

  __shared__ double s_cos[kDr / 2];
  __shared__ double s_sin[kDr / 2];
  if (tid < kDr / 2) {
    // theta_j = base^(-2j/d): exp2 of an exactly representable multiple of log2(base)
    double inv = exp2(-(2.0 * tid / kDr) * log2_theta);
    double s, c;
    sincos((double)pos * inv, &s, &c);
    s_cos[tid] = c;
    s_sin[tid] = s;
  }
  // c_KV: 512 bf16 = 64 x 16 bytes, copied unchanged
  if (tid < kDc / 8) {
    reinterpret_cast<uint4*>(row)[tid] = reinterpret_cast<const uint4*>(c_kv + (int64_t)i * kDc)[tid];
  }
  __syncthreads();
  if (tid >= 64 && tid < 64 + kDr / 2) {
    int j = tid - 64;
    const uint16_t* k = k_rope + (int64_t)i * kDr;
    double x0 = bf16_to_f32(k[2 * j]), x1 = bf16_to_f32(k[2 * j + 1]);
    double c = s_cos[j], s = s_sin[j];
    uint32_t packed = (uint32_t)f64_to_bf16(x0 * c - x1 * s) | ((uint32_t)f64_to_bf16(x0 * s + x1 * c) << 16);
    reinterpret_cast<uint32_t*>(row + kDc)[j] = packed;
  }
  if (q_rope != nullptr) {
    uint32_t* q = reinterpret_cast<uint32_t*>(q_rope + (int64_t)i * n_heads * kDr);
    for (int p = tid; p < n_heads * (kDr / 2); p += blockDim.x) {
      int j = p % (kDr / 2);
      uint32_t v = q[p];
      double x0 = bf16_to_f32((uint16_t)(v & 0xFFFFu)), x1 = bf16_to_f32((uint16_t)(v >> 16));
      double c = s_cos[j], s = s_sin[j];
      q[p] = (uint32_t)f64_to_bf16(x0 * c - x1 * s) | ((uint32_t)f64_to_bf16(x0 * s + x1 * c) << 16);
    }
  }
}

hipError_t launch_rope_append(const CacheView& cache, int n_heads, int num_tokens, const int32_t* token_seq,
                              const int32_t* token_pos, const uint16_t* c_kv, const uint16_t* k_rope,
                              uint16_t* q_rope, float theta, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_append_kernel, dim3(num_tokens), dim3(256), 0, stream, cache, n_heads, token_seq,
                     token_pos, c_kv, k_rope, q_rope, log2((double)theta));
  return hipGetLastError();
}

}  // namespace mla
