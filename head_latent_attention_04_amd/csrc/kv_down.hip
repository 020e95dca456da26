// KV down-projection of new tokens, fused with the RoPE rotation and the append: the step right
// ahead of the cache ("论文复现工坊 No.4", section 2: kv_combined = wkv_a(x) is split into the latent
// part and the decoupled RoPE key, and the latent part goes through kv_norm, an RMSNorm; section 4:
// that RMSNorm sits right after the W_DKV projection).
//
// Two kernels:
//   1. kv = x . W_DKV^T with bf16 MFMA, fp32 accumulation, as fp32 partials over splits of the input
//      dimension. From 256 tokens on, the tiled GEMM of gemm_bt.hip; below, its split-K kernel,
//      split so that the weight (d_c + d_R rows of `dim`) streams through many work-groups.
//      Work-group (column tile of 32, split s, block of 32 tokens): wave w takes a quarter of the
//      split's K range; the four partial tiles are added through LDS and written as fp32 partials
//      [split][token][576]. Both MFMA operands are K-contiguous in memory (x rows; W_DKV rows in the
//      nn.Linear layout), so they are loaded straight from global memory.
//   2. kv_down_finish_kernel: one work-group per token adds the split partials, rounds kv to bf16
//      (the projection's output dtype), normalises the latent part (fp32 mean of squares, the
//      caller's eps, kv_norm's weight) and rounds it, turns k_R by the token's position with the
//      RoPE helpers of rope_device.h (fp64 angles, one rounding, as the plain append), and writes
//      the cache row [c_KV | R_p k_R].
#include <algorithm>

#include "rope_device.h"

namespace mla {

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRowOut = kDc + kDr;  // 576 outputs per token
constexpr int kMaxSplits = kGemmMaxSplits;  // splits of the input dimension

// Token counts from here on take the tiled GEMM (128 x 192 tiles, operands through LDS); fewer
// tokens take the split-K kernel of gemm_bt.hip, which spreads the weight over many work-groups.
constexpr int kTiledMinTokens = 256;

inline bool kv_down_tiled(int num_tokens) { return num_tokens >= kTiledMinTokens; }

inline int kv_down_splits(int num_tokens, int dim) {
  if (kv_down_tiled(num_tokens)) return gemm_bt_splits(num_tokens, kRowOut, dim);
  return splitk_splits(num_tokens, kRowOut, dim);
}
}  // namespace

size_t kv_down_workspace_bytes(int num_tokens, int dim) {
  return (size_t)kv_down_splits(num_tokens, dim) * num_tokens * kRowOut * 4;
}

__global__ void __launch_bounds__(256) kv_down_finish_kernel(CacheView cache, int num_tokens, int nsplit,
                                                             const int32_t* __restrict__ token_seq,
                                                             const int32_t* __restrict__ token_pos,
                                                             const float* __restrict__ part,
                                                             const uint16_t* __restrict__ gamma, float eps,
                                                             double log2_theta) {
  __shared__ float s_sum[4];
  const int i = blockIdx.x, tid = threadIdx.x;
  // thread t < 144 owns columns 4t .. 4t + 3: 128 threads the latent part, 16 the RoPE key (two
  // pairs each). All split partials are loaded before the first add (one memory latency), then
  // added in split order.
  const bool live = tid < kRowOut / 4;
  const int seq = token_seq[i], pos = token_pos[i];
  const float4* p4 = reinterpret_cast<const float4*>(part) + (int64_t)i * (kRowOut / 4) + tid;
  const int64_t split_stride = (int64_t)num_tokens * (kRowOut / 4);
  float4 v[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
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
  for (int s = 0; s < kMaxSplits; ++s) {
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

hipError_t launch_kv_down(const CacheView& cache, int num_tokens, const int32_t* token_seq, const int32_t* token_pos,
                          const uint16_t* x, int dim, const uint16_t* w_dkv, const uint16_t* gamma, float eps,
                          float theta, void* workspace, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int ns = kv_down_splits(num_tokens, dim);
  const int tblocks = (num_tokens + 31) / 32;
  if (tblocks > 65535) return hipErrorInvalidValue;
  float* part = static_cast<float*>(workspace);
  hipError_t e;
  if (kv_down_tiled(num_tokens)) {
    e = launch_gemm_bt_partial(num_tokens, kRowOut, dim, ns, x, w_dkv, part, stream);
  } else {
    e = launch_splitk_gemm(num_tokens, kRowOut, dim, ns, x, w_dkv, part, stream);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_down_finish_kernel, dim3(num_tokens), dim3(256), 0, stream, cache, num_tokens, ns, token_seq,
                     token_pos, part, gamma, eps, log2((double)theta));
  return hipGetLastError();
}

}  // namespace mla
