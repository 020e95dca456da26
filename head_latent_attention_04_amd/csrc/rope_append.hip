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

  // Every load of this token is issued before the first store (the query is rotated in place, so a
  // load after a store of the same array would wait for it), and the token's inputs before its
  // position, which only the angles and the destination row depend on.
  constexpr int kQPerThread = 16;  // n_heads * 32 pairs / 256 threads, for up to 128 heads per pass
  uint32_t* q = q_rope != nullptr ? reinterpret_cast<uint32_t*>(q_rope + (int64_t)i * n_heads * kDr) : nullptr;
  const int nq = n_heads * (kDr / 2);
  uint4 ckv = make_uint4(0, 0, 0, 0);
  if (tid < kDc / 8) ckv = reinterpret_cast<const uint4*>(c_kv + (int64_t)i * kDc)[tid];
  uint32_t kr = 0;
  if (tid < kDr / 2) kr = reinterpret_cast<const uint32_t*>(k_rope + (int64_t)i * kDr)[tid];
  uint32_t v0[kQPerThread];  // first pass of the query pairs
  if (q != nullptr) {
#pragma unroll
    for (int k = 0; k < kQPerThread; ++k) v0[k] = tid + 256 * k < nq ? q[tid + 256 * k] : 0u;
  }
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
  __syncthreads();
  // c_KV: 512 bf16 = 64 x 16 bytes, copied unchanged; k_R pair j rotated by angle j
  if (tid < kDc / 8) reinterpret_cast<uint4*>(row)[tid] = ckv;
  if (tid < kDr / 2) {
    const double x0 = bf16_to_f32((uint16_t)(kr & 0xFFFFu)), x1 = bf16_to_f32((uint16_t)(kr >> 16));
    const double c = s_cos[tid], s = s_sin[tid];
    reinterpret_cast<uint32_t*>(row + kDc)[tid] =
        (uint32_t)f64_to_bf16(x0 * c - x1 * s) | ((uint32_t)f64_to_bf16(x0 * s + x1 * c) << 16);
  }
  if (q != nullptr) {
    // pair p = tid + 256 k of the token's [n_heads, 32] pairs; its angle index is p % 32 = tid % 32
    const double c = s_cos[tid % (kDr / 2)], s = s_sin[tid % (kDr / 2)];
    for (int base = 0; base < nq; base += 256 * kQPerThread) {
      uint32_t v[kQPerThread];
#pragma unroll
      for (int k = 0; k < kQPerThread; ++k) {
        const int p = base + tid + 256 * k;
        v[k] = base == 0 ? v0[k] : (p < nq ? q[p] : 0u);
      }
#pragma unroll
      for (int k = 0; k < kQPerThread; ++k) {
        const int p = base + tid + 256 * k;
        const double x0 = bf16_to_f32((uint16_t)(v[k] & 0xFFFFu)), x1 = bf16_to_f32((uint16_t)(v[k] >> 16));
        if (p < nq) q[p] = (uint32_t)f64_to_bf16(x0 * c - x1 * s) | ((uint32_t)f64_to_bf16(x0 * s + x1 * c) << 16);
      }
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
