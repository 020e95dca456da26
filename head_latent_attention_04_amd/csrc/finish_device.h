// Per-token finishing steps of the two down-projections that read the hidden state: the sum of the
// split-K partials, the projection's bf16 rounding, the RMSNorm, and the RoPE work of each path
// ("论文复现工坊 No.4", section 2: wkv_a's output split into the latent part, which goes through
// kv_norm, and the decoupled RoPE key; wq_a's output through q_norm). One 256-thread work-group per
// token; `part` points at the token's first partial column and rows are `ld` floats apart, so the
// same code serves partials of one projection and of both projections side by side.
#pragma once

#include "rope_device.h"

namespace mla {

constexpr int kKvRowOut = kDc + kDr;  // 576 outputs of the KV down-projection per token

// c_q in MFMA operand order for 32-token blocks: token t, element k at
//   (((t / 32) * (q_rank / 16) + k / 16) * 64 + t % 32 + 32 ((k / 8) % 2)) * 8 + k % 8.
__host__ __device__ inline int64_t cq_offset(int t, int k, int q_rank) {
  return (((int64_t)(t / 32) * (q_rank / 16) + k / 16) * 64 + t % 32 + 32 * ((k / 8) & 1)) * 8 + k % 8;
}

// KV side of token i: kv = sum of the splits, rounded to bf16; the latent part normalised (fp32 mean of
// squares, eps, kv_norm's weight) and rounded; k_R turned by the token's position (fp64 angles, one
// rounding, as the plain append); the row [c_KV | R_p k_R] written to the cache slot of the token.
// Thread t < 144 owns columns 4t .. 4t + 3: 128 threads the latent part, 16 the RoPE key (two pairs
// each). All split partials are loaded before the first add (one memory latency), then added in
// split order. s_sum: 4 floats of LDS.
__device__ __forceinline__ void kv_finish_token(const CacheView& cache, int i, int num_tokens, int nsplit,
                                                const int32_t* __restrict__ token_seq,
                                                const int32_t* __restrict__ token_pos,
                                                const float* __restrict__ part, int ld,
                                                const uint16_t* __restrict__ gamma, float eps, double log2_theta,
                                                float* s_sum) {
  const int tid = threadIdx.x;
  const bool live = tid < kKvRowOut / 4;
  const int seq = token_seq[i], pos = token_pos[i];
  const float4* p4 = reinterpret_cast<const float4*>(part) + (int64_t)i * (ld / 4) + tid;
  const int64_t split_stride = (int64_t)num_tokens * (ld / 4);
  float4 v[kGemmMaxSplits];
#pragma unroll
  for (int s = 0; s < kGemmMaxSplits; ++s)
    v[s] = (live && s < nsplit) ? p4[s * split_stride] : make_float4(0.f, 0.f, 0.f, 0.f);
  // the RoPE threads take their angles (fp64) while the partials are on their way
  const bool rope_thread = live && tid >= kDc / 4;
  const int j = 2 * (tid - kDc / 4);
  double rc[2] = {1.0, 1.0}, rs[2] = {0.0, 0.0};
  if (rope_thread) {
#pragma unroll
    for (int e = 0; e < 2; ++e) rope_cos_sin(pos, j + e, log2_theta, &rc[e], &rs[e]);
  }
  float kv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kGemmMaxSplits; ++s) {
    kv[0] += v[s].x;
    kv[1] += v[s].y;
    kv[2] += v[s].z;
    kv[3] += v[s].w;
  }
  // the projection's output rounded to bf16; mean of squares of the latent part in fp32
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kv[e] = bf16_to_f32(f32_to_bf16(kv[e]));
    ss += kv[e] * kv[e];
  }
  if (tid >= kDc / 4) ss = 0.f;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((tid & 63) == 0) s_sum[tid >> 6] = ss;
  __syncthreads();
  if (!live) return;
  uint16_t* row = cache.data + row_offset(cache, seq, pos);
  if (tid < kDc / 4) {
    const float r = 1.f / sqrtf((s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3]) / kDc + eps);
    uint16_t c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = f32_to_bf16(kv[e] * r * bf16_to_f32(gamma[4 * tid + e]));
    reinterpret_cast<uint2*>(row)[tid] =
        make_uint2((uint32_t)c[0] | ((uint32_t)c[1] << 16), (uint32_t)c[2] | ((uint32_t)c[3] << 16));
  } else {
    // k_R (rounded to bf16 above) turned by the token's position, pairs j and j + 1
    uint32_t w[2] = {(uint32_t)f32_to_bf16(kv[0]) | ((uint32_t)f32_to_bf16(kv[1]) << 16),
                     (uint32_t)f32_to_bf16(kv[2]) | ((uint32_t)f32_to_bf16(kv[3]) << 16)};
#pragma unroll
    for (int e = 0; e < 2; ++e) w[e] = rope_turn_pair(w[e], rc[e], rs[e]);
    reinterpret_cast<uint2*>(row + kDc)[tid - kDc / 4] = make_uint2(w[0], w[1]);
  }
}

// Query side of token i: c_q = bf16(RMSNorm(bf16(sum of the splits))) written in operand order, and the
// token's 32 RoPE cos/sin pairs (fp64) for the query kernel. Thread t owns columns 4 (t + 256 u) .. +3,
// u < 2 (q_rank <= 2048); all split loads are issued before the adds. s_sum: 4 floats of LDS.
__device__ __forceinline__ void cq_finish_token(int i, int num_tokens, int q_rank, int nsplit,
                                                const int32_t* __restrict__ token_pos,
                                                const float* __restrict__ part, int ld,
                                                const uint16_t* __restrict__ gamma, float eps, double log2_theta,
                                                uint16_t* __restrict__ c_q, double* __restrict__ cs, float* s_sum) {
  const int tid = threadIdx.x;
  const int n4 = q_rank / 4;  // float4 columns, <= 512
  float kv[2][4] = {};
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c4 = tid + 256 * u;
    if (c4 >= n4) continue;
    const float4* p4 = reinterpret_cast<const float4*>(part) + (int64_t)i * (ld / 4) + c4;
    float4 v[kGemmMaxSplits];
#pragma unroll
    for (int s = 0; s < kGemmMaxSplits; ++s)
      v[s] = s < nsplit ? p4[(int64_t)s * num_tokens * (ld / 4)] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < kGemmMaxSplits; ++s) {
      kv[u][0] += v[s].x;
      kv[u][1] += v[s].y;
      kv[u][2] += v[s].z;
      kv[u][3] += v[s].w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv[u][e] = bf16_to_f32(f32_to_bf16(kv[u][e]));  // wq_a's output dtype
      ss += kv[u][e] * kv[u][e];
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((tid & 63) == 0) s_sum[tid >> 6] = ss;
  // the token's RoPE angles (fp64), one pair per thread of the first 32
  if (tid < kDr / 2) {
    double c, s;
    rope_cos_sin(token_pos[i], tid, log2_theta, &c, &s);
    cs[((int64_t)i * (kDr / 2) + tid) * 2] = c;
    cs[((int64_t)i * (kDr / 2) + tid) * 2 + 1] = s;
  }
  __syncthreads();
  const float r = 1.f / sqrtf((s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3]) / q_rank + eps);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c4 = tid + 256 * u;
    if (c4 >= n4) continue;
    uint16_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(kv[u][e] * r * bf16_to_f32(gamma[4 * c4 + e]));
    *reinterpret_cast<uint2*>(c_q + cq_offset(i, 4 * c4, q_rank)) =
        make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
  }
}

}  // namespace mla
