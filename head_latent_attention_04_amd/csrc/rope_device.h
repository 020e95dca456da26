// RoPE rotation of one new token's decoupled key and query, and the append of its latent row to
// the paged cache, as one work-group's share of the work.
//
// RoPE as on "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA與ROPE的融合": position m turns pair j by
// m * theta_j, theta_j = base^(-2j/d) with d = d_R (the decoupled part). Pairs are interleaved
// (x_{2j}, x_{2j+1}), matching the complex freqs_cis rotation the module of
// "论文复现工坊 No.4", section 2, takes as input. The row written is [c_KV | R_m k_R]
// (the split order of that module's wkv_a output).
//
// Work-group (token i, head group g) rotates the query pairs of heads 32 g .. 32 g + 31; group 0
// also writes the token's cache row. The angle m * theta_j is formed and turned in fp64 (positions
// reach 1.3e5 rad, where an fp32 angle would be off by ~1e-2 rad) and each result is rounded once
// to bf16.
#pragma once

#include "mla_internal.h"

namespace mla {

constexpr int kRopeHeadsPerGroup = 32;  // heads per work-group: 8 threads per head, 4 pairs each

__host__ __device__ inline int rope_groups(int n_heads) { return (n_heads + kRopeHeadsPerGroup - 1) / kRopeHeadsPerGroup; }

// cos and sin of pair j's angle at position pos: theta_j = base^(-2j/d_R), formed as exp2 of an
// exactly representable multiple of log2(base), turned in fp64.
__device__ __forceinline__ void rope_cos_sin(int pos, int j, double log2_theta, double* c, double* s) {
  const double inv = exp2(-(2.0 * j / kDr) * log2_theta);
  sincos((double)pos * inv, s, c);
}

// One interleaved pair (x_2j in the low half, x_2j+1 in the high half of w) turned by (c, s), each
// result rounded once to bf16.
__device__ __forceinline__ uint32_t rope_turn_pair(uint32_t w, double c, double s) {
  const double x0 = bf16_to_f32((uint16_t)(w & 0xFFFFu)), x1 = bf16_to_f32((uint16_t)(w >> 16));
  return (uint32_t)f64_to_bf16(x0 * c - x1 * s) | ((uint32_t)f64_to_bf16(x0 * s + x1 * c) << 16);
}

// 256 threads. s_cs: 64 doubles of LDS (cos, sin of the 32 angles). If q_abs is not null the
// rotated query is also written into the RoPE part of the absorbed-query rows (operand order).
__device__ __forceinline__ void rope_token_group(const CacheView& cache, int n_heads, int i, int g,
                                                 const int32_t* __restrict__ token_seq,
                                                 const int32_t* __restrict__ token_pos,
                                                 const uint16_t* __restrict__ c_kv,
                                                 const uint16_t* __restrict__ k_rope, uint16_t* __restrict__ q_rope,
                                                 double log2_theta, uint16_t* __restrict__ q_abs, int tiles,
                                                 double* s_cs) {
  const int tid = threadIdx.x;
  // Every load is issued before the first store (the query is rotated in place) and the token's
  // inputs before its position, which only the angles and the destination row depend on.
  uint4 ckv = make_uint4(0, 0, 0, 0);
  uint32_t kr = 0;
  if (g == 0) {
    if (tid < kDc / 8) ckv = reinterpret_cast<const uint4*>(c_kv + (int64_t)i * kDc)[tid];
    if (tid < kDr / 2) kr = reinterpret_cast<const uint32_t*>(k_rope + (int64_t)i * kDr)[tid];
  }
  // query piece: head 32 g + tid / 8, pairs 4 (tid % 8) .. +3 (elements 8 (tid % 8) .. +7)
  const int h = kRopeHeadsPerGroup * g + (tid >> 3), pc = tid & 7;
  const bool qok = q_rope != nullptr && h < n_heads;
  uint4* qp = qok ? reinterpret_cast<uint4*>(q_rope + ((int64_t)i * n_heads + h) * kDr) + pc : nullptr;
  uint4 qv = make_uint4(0, 0, 0, 0);
  if (qok) qv = *qp;
  const int pos = token_pos[i];

  if (tid < kDr / 2) {
    double s, c;
    rope_cos_sin(pos, tid, log2_theta, &c, &s);
    s_cs[tid] = c;
    s_cs[kDr / 2 + tid] = s;
  }
  __syncthreads();

  if (g == 0) {
    uint16_t* row = cache.data + row_offset(cache, token_seq[i], pos);
    // c_KV: 512 bf16 = 64 x 16 bytes, copied unchanged; k_R pair j rotated by angle j
    if (tid < kDc / 8) reinterpret_cast<uint4*>(row)[tid] = ckv;
    if (tid < kDr / 2) reinterpret_cast<uint32_t*>(row + kDc)[tid] = rope_turn_pair(kr, s_cs[tid], s_cs[kDr / 2 + tid]);
  }
  if (qok) {
    uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = rope_turn_pair(w[e], s_cs[4 * pc + e], s_cs[kDr / 2 + 4 * pc + e]);
    const uint4 r = make_uint4(w[0], w[1], w[2], w[3]);
    *qp = r;
    if (q_abs != nullptr) *reinterpret_cast<uint4*>(q_abs + q_perm_offset(i, tiles, h, kDc + 8 * pc)) = r;
  }
}

}  // namespace mla
