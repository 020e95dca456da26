// Split-KV combine and value up-projection.
//
// The partials of one (sequence, head) are merged with their log-sum-exps (the same softmax,
// taken in pieces): lse = ln sum_s exp(lse_s), o_lat = sum_s exp(lse_s - lse) o_s. The merged
// latent is then up-projected, out[h] = W_UV[h] o_lat: the value side is never expanded per
// token ("论文复现工坊 No.4", section 1; "Multi-Head Latent Attention: DeepSeek V2/V3 工程视角",
// section 四: the W_UV up-projection or its absorbed equivalent).
//
// One work-group per (head, 16 sequences): the merged latents go to LDS in fp32, and each thread
// produces one output column for 8 sequences, reading W_UV[h] once per work-group.
#include "mla_internal.h"

namespace mla {

constexpr int kCombRows = 16;

__global__ void __launch_bounds__(256) combine_simple_kernel(int batch, int n_heads, int num_splits,
                                                             const float* __restrict__ o_partial,
                                                             const float* __restrict__ lse_partial,
                                                             const uint16_t* __restrict__ w_uv,
                                                             uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * kCombRows;
  const int tid = threadIdx.x;
  __shared__ float olat[kCombRows][kDc];
  for (int rr = 0; rr < kCombRows; ++rr) {
    const int b = b0 + rr;
    if (b >= batch) {
      for (int c = tid; c < kDc; c += 256) olat[rr][c] = 0.f;
      continue;
    }
    const int64_t base = ((int64_t)b * n_heads + h) * num_splits;
    // max and sum of exp over splits (every thread computes the same scalars)
    float m = -INFINITY;
    for (int s = 0; s < num_splits; ++s) m = fmaxf(m, lse_partial[base + s]);
    float z = 0.f;
    if (m != -INFINITY)
      for (int s = 0; s < num_splits; ++s) z += expf(lse_partial[base + s] - m);
    if (tid == 0 && lse_out) lse_out[(int64_t)b * n_heads + h] = (m == -INFINITY) ? -INFINITY : m + logf(z);
    for (int c = tid; c < kDc; c += 256) {
      float acc = 0.f;
      if (m != -INFINITY) {
        for (int s = 0; s < num_splits; ++s) {
          float ls = lse_partial[base + s];
          if (ls != -INFINITY) acc = fmaf(expf(ls - m) / z, o_partial[(base + s) * kDc + c], acc);
        }
      }
      olat[rr][c] = acc;
    }
  }
  __syncthreads();
  const int v = tid % kDv;
  const int half = tid / kDv;  // sequences half*8 .. half*8+7
  const uint16_t* w = w_uv + ((int64_t)h * kDv + v) * kDc;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int c = 0; c < kDc; ++c) {
    float wv = bf16_to_f32(w[c]);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(wv, olat[half * 8 + k][c], acc[k]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    int b = b0 + half * 8 + k;
    if (b < batch) out[((int64_t)b * n_heads + h) * kDv + v] = f32_to_bf16(acc[k]);
  }
}

hipError_t launch_combine(int batch, int n_heads, int num_splits, const float* o_partial, const float* lse_partial,
                          const uint16_t* w_uv, uint16_t* out, float* lse_out, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  dim3 grid(n_heads, (batch + kCombRows - 1) / kCombRows);
  hipLaunchKernelGGL(combine_simple_kernel, grid, dim3(256), 0, stream, batch, n_heads, num_splits, o_partial,
                     lse_partial, w_uv, out, lse_out);
  return hipGetLastError();
}

}  // namespace mla
