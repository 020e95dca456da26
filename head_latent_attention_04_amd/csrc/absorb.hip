// Query absorption: q_abs[r, h, :] = W_UK[h]^T q_nope[r, h, :], joined to the rotated RoPE query.
//
// "论文复现工坊 No.4", section 4: the key up-projection W_UK is folded into the query
// (Q_absorbed = Q W_UK^T) and the product is scored directly against the cached latent c^KV;
// "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA的數學原理": x_t (W_q W_k^T) c_i^T.
//
// Output row layout [r, h, 0:576] = [q_abs (512) | q_rope (64)], bf16, i.e. the query side of a
// 576-wide dot product with a cache row [c_KV | k_R].
//
// One work-group per (head, 32 rows): W_UK[h] (128 x 512) is streamed once per group of rows and
// each of the 256 threads owns two latent columns for all 32 rows (fp32 accumulation).
#include "mla_internal.h"

namespace mla {

constexpr int kAbsRows = 32;

__global__ void __launch_bounds__(256) absorb_kernel(int rows, int n_heads, const uint16_t* __restrict__ q_nope,
                                                      const uint16_t* __restrict__ q_rope,
                                                      const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_abs) {
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * kAbsRows;
  const int tid = threadIdx.x;
  __shared__ float qs[kAbsRows][kDnope];
  for (int i = tid; i < kAbsRows * kDnope; i += 256) {
    int rr = i / kDnope, d = i % kDnope;
    int r = r0 + rr;
    qs[rr][d] = (r < rows) ? bf16_to_f32(q_nope[((int64_t)r * n_heads + h) * kDnope + d]) : 0.f;
  }
  __syncthreads();
  float acc0[kAbsRows], acc1[kAbsRows];
#pragma unroll
  for (int rr = 0; rr < kAbsRows; ++rr) { acc0[rr] = 0.f; acc1[rr] = 0.f; }
  const uint16_t* w = w_uk + (int64_t)h * kDnope * kDc;
  for (int d = 0; d < kDnope; ++d) {
    float w0 = bf16_to_f32(w[d * kDc + tid]);
    float w1 = bf16_to_f32(w[d * kDc + tid + 256]);
#pragma unroll
    for (int rr = 0; rr < kAbsRows; ++rr) {
      acc0[rr] = fmaf(qs[rr][d], w0, acc0[rr]);
      acc1[rr] = fmaf(qs[rr][d], w1, acc1[rr]);
    }
  }
#pragma unroll
  for (int rr = 0; rr < kAbsRows; ++rr) {
    int r = r0 + rr;
    if (r < rows) {
      uint16_t* o = q_abs + ((int64_t)r * n_heads + h) * kRow;
      o[tid] = f32_to_bf16(acc0[rr]);
      o[tid + 256] = f32_to_bf16(acc1[rr]);
      if (tid < kDr) o[kDc + tid] = q_rope[((int64_t)r * n_heads + h) * kDr + tid];
    }
  }
}

hipError_t launch_absorb(int rows, int n_heads, const uint16_t* q_nope, const uint16_t* q_rope,
                         const uint16_t* w_uk, uint16_t* q_abs, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  dim3 grid(n_heads, (rows + kAbsRows - 1) / kAbsRows);
  hipLaunchKernelGGL(absorb_kernel, grid, dim3(256), 0, stream, rows, n_heads, q_nope, q_rope, w_uk, q_abs);
  return hipGetLastError();
}

}  // namespace mla
