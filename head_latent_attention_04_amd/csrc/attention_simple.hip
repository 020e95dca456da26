// Straightforward causal prefill attention over the latent cache: one wave per (query row, head).
//
// This is the plain formulation of the absorbed scores and the latent reduction
// ("论文复现工坊 No.4", sections 2 and 4; "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA的數學原理"):
//   s_t = scale * (q_abs . c_t + q_R . kR_t),  online softmax over t,  o_lat = sum_t p_t c_t.
// The wave scores the tokens of a 64-token chunk one at a time with coalesced row reads, keeps the
// running max and sum, and lane l accumulates latent columns l, l+64, ..., l+448.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Attend one query (576 floats in LDS) over tokens [t0, t1) of sequence `seq`.
// Returns per-lane o[8] (unnormalised, latent columns lane + 64k), running max m (log2 units) and sum l.
__device__ void attend_range(const CacheView& cache, int seq, int t0, int t1, const float* q, float scale_log2,
                             float o[8], float& m, float& l) {
  const int lane = threadIdx.x;
  m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.f;
  __shared__ float p_s[64];
  float qv[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) qv[k] = q[lane + 64 * k];
  for (int c0 = t0; c0 < t1; c0 += 64) {
    const int t = c0 + lane;
    const int n = min(64, t1 - c0);
    float s = -INFINITY;
    // the wave scores one token at a time with coalesced row reads; lane j keeps token j's score
    for (int j = 0; j < n; ++j) {
      const uint16_t* row = cache.data + row_offset(cache, seq, c0 + j);
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < 9; ++k) part = fmaf(qv[k], bf16_to_f32(row[lane + 64 * k]), part);
      part = wave_sum(part);
      if (lane == j) s = part * scale_log2;
    }
    float cmax = wave_max(s);
    float m_new = fmaxf(m, cmax);
    float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
    float p = (t < t1) ? exp2f(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
    m = m_new;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= alpha;
    p_s[lane] = p;
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      const uint16_t* row = cache.data + row_offset(cache, seq, c0 + j);
      float pj = p_s[j];
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = fmaf(pj, bf16_to_f32(row[lane + 64 * k]), o[k]);
    }
    __syncthreads();
  }
}

}  // namespace

// grid (n_heads, total_q), block 64: query row j sees keys 0..pos_j.
__global__ void __launch_bounds__(64) prefill_simple_kernel(CacheView cache, int batch, int n_heads,
                                                            const int32_t* __restrict__ seq_lens,
                                                            const int32_t* __restrict__ cu_q_lens,
                                                            const uint16_t* __restrict__ q_abs, float scale_log2,
                                                            float* __restrict__ o_lat, float* __restrict__ lse) {
  const int h = blockIdx.x, j = blockIdx.y;
  const int lane = threadIdx.x;
  int b = 0;
  while (b + 1 < batch && cu_q_lens[b + 1] <= j) ++b;
  const int qlen = cu_q_lens[b + 1] - cu_q_lens[b];
  const int pos = seq_lens[b] - qlen + (j - cu_q_lens[b]);
  __shared__ float q[kRow];
  const uint16_t* qa = q_abs + ((int64_t)j * n_heads + h) * kRow;
  for (int k = lane; k < kRow; k += 64) q[k] = bf16_to_f32(qa[k]);
  __syncthreads();
  float o[8], m, l;
  attend_range(cache, b, 0, pos + 1, q, scale_log2, o, m, l);
  const int64_t r = (int64_t)j * n_heads + h;
  float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) o_lat[r * kDc + lane + 64 * k] = o[k] * inv;
  if (lane == 0) lse[r] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
}

hipError_t launch_prefill_attention(const CacheView& cache, int batch, int n_heads, const int32_t* seq_lens,
                                    const int32_t* cu_q_lens, int total_q, int max_q_len, const uint16_t* q_abs,
                                    float scale, float* o_lat, float* lse, hipStream_t stream) {
  (void)max_q_len;
  if (total_q == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_simple_kernel, dim3(n_heads, total_q), dim3(64), 0, stream, cache, batch, n_heads,
                     seq_lens, cu_q_lens, q_abs, scale * kLog2e, o_lat, lse);
  return hipGetLastError();
}

}  // namespace mla
