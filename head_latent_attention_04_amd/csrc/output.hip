// The output side of the attention: wo on the flattened per-head outputs, and the variant with W_UV
// folded into wo per head, so that decode hands the merged latent straight to the output GEMM
// ("论文复现工坊 No.4", section 2: the heads' outputs flattened and projected by wo; section 4: a
// projection absorbed into its neighbour, here on the value side).
//
//   unfolded: out[t, h] = W_UV[h] o_lat[t, h] (the combine), y[t] = W_O flat(out[t])
//   folded:   W_OV[:, h] = W_O[:, h] W_UV[h] (once per weight set), y[t] = W_OV flat(o_lat[t])
//
// Kernels:
//   * merge_latent_kernel: the combine's log-sum-exp merge without W_UV: one wave per (row, head)
//     merges the split partials into the normalised latent o_lat (bf16).
//   * prepare_rows_kernel: a row-major weight [N, K] copied into MFMA operand order (as the query
//     path's weight): row n, element k at (((n / 32) (K / 16) + k / 16) 64 + n % 32 + 32 ((k / 8) % 2))
//     8 + k % 8, so a wave's operand for one K step of a 32-row tile is one contiguous 1 KB.
//   * fold_output_weights_kernel: W_OV in fp32 outer products over the 128 value rows of each head,
//     written in operand order.
//   * oo_splitk_gemm_kernel + reduce_bf16_kernel: y = act W^T for few rows and a long K (n_heads x
//     128 or n_heads x 512): work-group (split of K, four 32-column tiles, 32 rows); the split's
//     activations are staged in LDS once and each wave streams one tile's weight as contiguous 1 KB
//     operand loads; fp32 partials per split, then one pass adds them and rounds.
#include <algorithm>

#include "mla_internal.h"

namespace mla {

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kOutMaxSplits = 64;
constexpr int kOoChunk = 1024;               // K columns of activations per LDS fill
constexpr int kOoPitch = kOoChunk * 2 + 16;  // LDS row pitch (bytes): rows 4 banks apart

__host__ __device__ inline int64_t oo_offset(int n, int64_t k, int64_t K) {
  return (((int64_t)(n / 32) * (K / 16) + k / 16) * 64 + n % 32 + 32 * ((k / 8) & 1)) * 8 + k % 8;
}

struct OoSplit {
  int count;          // splits of K (one fp32 partial each)
  int64_t split_len;  // K columns per split, a multiple of kOoChunk
};

OoSplit oo_split(int M, int N, int64_t K) {
  // about 512 work-groups (two per compute unit), each split a whole number of LDS chunks
  const int64_t groups = (int64_t)((N / 32 + 3) / 4) * ((M + 31) / 32);
  const int64_t chunks = (K + kOoChunk - 1) / kOoChunk;
  int64_t per = std::max<int64_t>(1, (chunks * groups) / 512);
  per = std::max<int64_t>(per, (chunks + kOutMaxSplits - 1) / kOutMaxSplits);
  return OoSplit{(int)((chunks + per - 1) / per), per * kOoChunk};
}
}  // namespace

// ---- merged latent ---------------------------------------------------------------------------------
// Wave per (row, head): lane l owns latent columns 8 l .. +7. Weights exp(lse_s - lse*), the same for
// every lane, from the split log-sum-exps; splits with lse = -inf weigh nothing; a row with no
// visible key gives zeros and lse* = -inf.
__global__ void __launch_bounds__(256) merge_latent_kernel(int rows_heads, int num_splits,
                                                           const uint16_t* __restrict__ o_partial,
                                                           const float* __restrict__ lse_partial,
                                                           uint16_t* __restrict__ o_lat, float* __restrict__ lse_out) {
  const int rh = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (rh >= rows_heads) return;
  const float* ls = lse_partial + (int64_t)rh * num_splits;
  float m = -INFINITY;
  for (int s = 0; s < num_splits; ++s) m = fmaxf(m, ls[s]);
  float acc[8] = {};
  float z = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < num_splits; ++s) {
      const float l = ls[s];
      if (l == -INFINITY) continue;
      const float w = expf(l - m);
      z += w;
      const uint4 v = *reinterpret_cast<const uint4*>(o_partial + ((int64_t)rh * num_splits + s) * kDc + 8 * lane);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += w * bf16_to_f32((uint16_t)(u[e] & 0xFFFFu));
        acc[2 * e + 1] += w * bf16_to_f32((uint16_t)(u[e] >> 16));
      }
    }
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = (uint32_t)f32_to_bf16(acc[2 * e] * inv) | ((uint32_t)f32_to_bf16(acc[2 * e + 1] * inv) << 16);
  *reinterpret_cast<uint4*>(o_lat + (int64_t)rh * kDc + 8 * lane) = make_uint4(o[0], o[1], o[2], o[3]);
  if (lse_out != nullptr && lane == 0) lse_out[rh] = (m == -INFINITY) ? -INFINITY : m + logf(z);
}

// ---- weights in operand order -----------------------------------------------------------------------
__global__ void __launch_bounds__(256) prepare_rows_kernel(int N, int64_t K, const uint16_t* __restrict__ w,
                                                           uint16_t* __restrict__ w_op) {
  // thread: row n, elements 8 c .. 8 c + 7 (16 bytes in, 16 bytes out)
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = K / 8;
  if (idx >= (int64_t)N * per_row) return;
  const int n = (int)(idx / per_row);
  const int64_t k = 8 * (idx % per_row);
  *reinterpret_cast<uint4*>(w_op + oo_offset(n, k, K)) = *reinterpret_cast<const uint4*>(w + (int64_t)n * K + k);
}

// W_OV[n][h 512 + c] = sum_d W_O[n][h 128 + d] W_UV[h][d][c]. Work-group (head, 64 rows n, 64 columns c):
// thread (ty, tx) accumulates n = n0 + 4 ty .. +3, c = c0 + 4 tx .. +3; 16 rows d at a time in LDS.
__global__ void __launch_bounds__(256) fold_output_weights_kernel(int dim, int n_heads,
                                                                  const uint16_t* __restrict__ w_o,
                                                                  const uint16_t* __restrict__ w_uv,
                                                                  uint16_t* __restrict__ w_ov) {
  __shared__ float so[16][65], sv[16][64];
  const int h = blockIdx.x, n0 = 64 * blockIdx.y, c0 = 64 * blockIdx.z;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t kin = (int64_t)n_heads * kDv, kout = (int64_t)n_heads * kDc;
  float acc[4][4] = {};
  for (int d0 = 0; d0 < kDv; d0 += 16) {
    for (int e = tid; e < 16 * 64; e += 256) {
      const int nn = e >> 4, dd = e & 15;  // W_O: 16 consecutive d of row n0 + nn
      so[dd][nn] = bf16_to_f32(w_o[(int64_t)(n0 + nn) * kin + (int64_t)h * kDv + d0 + dd]);
      const int d2 = e >> 6, cc = e & 63;
      sv[d2][cc] = bf16_to_f32(w_uv[((int64_t)h * kDv + d0 + d2) * kDc + c0 + cc]);
    }
    __syncthreads();
#pragma unroll
    for (int dd = 0; dd < 16; ++dd) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = so[dd][4 * ty + i];
        b[i] = sv[dd][4 * tx + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint2 v = make_uint2((uint32_t)f32_to_bf16(acc[i][0]) | ((uint32_t)f32_to_bf16(acc[i][1]) << 16),
                               (uint32_t)f32_to_bf16(acc[i][2]) | ((uint32_t)f32_to_bf16(acc[i][3]) << 16));
    *reinterpret_cast<uint2*>(w_ov + oo_offset(n0 + 4 * ty + i, (int64_t)h * kDc + c0 + 4 * tx, kout)) = v;
  }
}

// ---- y = act W^T, split over K -------------------------------------------------------------------
// Work-group (split s, column group cg of 4 tiles, row block tb): the activations of rows
// 32 tb .. +31 over the split's K range are copied into LDS once, in chunks of kOoChunk columns; wave w
// then streams the operand-order weight of column tile 4 cg + w over the chunk (one contiguous 1 KB per
// K step, eight loads in flight) against LDS reads of the activations, and accumulates the whole split
// in one 32 x 32 fp32 tile. The weight is read exactly once; the activations (a few MB at most) come
// from L2 once per column group.
__global__ void __launch_bounds__(256) oo_splitk_gemm_kernel(int M, int N, int64_t K, int64_t split_len,
                                                             const uint16_t* __restrict__ act,
                                                             const uint16_t* __restrict__ w_op,
                                                             float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) char sa[32 * kOoPitch];
  const int s = blockIdx.x, cg = blockIdx.y, tb = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ct = 4 * cg + wave;
  const bool active = ct < N / 32;  // the last group may hold fewer than four tiles
  const int64_t kbeg = (int64_t)s * split_len, kend = std::min<int64_t>(K, kbeg + split_len);
  const uint16_t* pb = w_op + ((int64_t)(active ? ct : 0) * (K / 16)) * 512 + lane * 8;
  const char* arow = sa + (lane & 31) * kOoPitch + 16 * (lane >> 5);
  f32x16 acc = f32x16{};
  for (int64_t k0 = kbeg; k0 < kend; k0 += kOoChunk) {
    const int klen = (int)std::min<int64_t>(kOoChunk, kend - k0);  // a multiple of 16
    if (k0 != kbeg) __syncthreads();                              // the previous chunk is consumed
    auto stage_act = [&](int i, int cpr) {  // 16 bytes: row i / cpr, chunk i % cpr
      const int r = i / cpr, c = i % cpr;
      const int row = std::min(32 * tb + r, M - 1);
      *reinterpret_cast<uint4*>(sa + r * kOoPitch + 16 * c) =
          *reinterpret_cast<const uint4*>(act + (int64_t)row * K + k0 + 8 * c);
    };
    if (klen == kOoChunk) {
#pragma unroll 4
      for (int i = tid; i < 32 * (kOoChunk / 8); i += 256) stage_act(i, kOoChunk / 8);
    } else {
      for (int i = tid; i < 32 * (klen / 8); i += 256) stage_act(i, klen / 8);
    }
    __syncthreads();
    if (active) {
      const uint16_t* pk = pb + (k0 / 16) * 512;
      // eight weight fragments in flight; each is read by this wave only, hence the non-temporal hint
      auto batch = [&](int k) {
        bf16x8 b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          b[u] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(pk + (int64_t)(k + u) * 512));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 32 * (k + u));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[u], acc, 0, 0, 0);
        }
      };
      if (klen == kOoChunk) {  // a whole chunk: the step count is a constant and the loop unrolls
#pragma unroll
        for (int k = 0; k < kOoChunk / 16; k += 8) batch(k);
      } else {
        const int steps = klen / 16;
        int k = 0;
        for (; k + 8 <= steps; k += 8) batch(k);
        for (; k < steps; ++k) {
          const bf16x8 b = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(pk + (int64_t)k * 512));
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 32 * k);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
      }
    }
  }
  if (!active) return;
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
  // D: lane holds row 8 (e / 4) + 4 (lane / 32) + e % 4 and column lane % 32 of the tile
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int t = 32 * tb + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    if (t < M) part[((int64_t)s * M + t) * N + 32 * ct + (lane & 31)] = acc[e];
  }
}

__global__ void __launch_bounds__(256) reduce_bf16_kernel(int64_t count4, int nsplit, const float* __restrict__ part,
                                                          uint16_t* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 index
  if (i >= count4) return;
  float4 v[kOutMaxSplits > 16 ? 16 : kOutMaxSplits];
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += 16) {
#pragma unroll
    for (int s = 0; s < 16; ++s)
      v[s] = s0 + s < nsplit ? reinterpret_cast<const float4*>(part)[(int64_t)(s0 + s) * count4 + i]
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      a[0] += v[s].x;
      a[1] += v[s].y;
      a[2] += v[s].z;
      a[3] += v[s].w;
    }
  }
  reinterpret_cast<uint2*>(y)[i] = make_uint2((uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16),
                                              (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16));
}

// ---- launchers -------------------------------------------------------------------------------------
hipError_t launch_merge_latent(int rows, int n_heads, int num_splits, const uint16_t* o_partial,
                               const float* lse_partial, uint16_t* o_lat, float* lse_out, hipStream_t stream) {
  const int64_t rh = (int64_t)rows * n_heads;
  if (rh <= 0) return hipSuccess;
  if ((rh + 3) / 4 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_latent_kernel, dim3((unsigned)((rh + 3) / 4)), dim3(256), 0, stream, (int)rh, num_splits,
                     o_partial, lse_partial, o_lat, lse_out);
  return hipGetLastError();
}

hipError_t launch_prepare_rows(int N, int64_t K, const uint16_t* w, uint16_t* w_op, hipStream_t stream) {
  const int64_t threads = (int64_t)N * (K / 8);
  if (N % 32 != 0 || K % 16 != 0 || (threads + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prepare_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, N, K, w, w_op);
  return hipGetLastError();
}

hipError_t launch_fold_output_weights(int dim, int n_heads, const uint16_t* w_o, const uint16_t* w_uv,
                                      uint16_t* w_ov, hipStream_t stream) {
  if (dim % 64 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fold_output_weights_kernel, dim3(n_heads, dim / 64, kDc / 64), dim3(256), 0, stream, dim, n_heads,
                     w_o, w_uv, w_ov);
  return hipGetLastError();
}

size_t output_workspace_bytes(int M, int N, int64_t K) { return (size_t)oo_split(M, N, K).count * M * N * 4; }

hipError_t launch_output_gemm(int M, int N, int64_t K, const uint16_t* act, const uint16_t* w_op, void* workspace,
                              uint16_t* y, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (N % 32 != 0 || K % 64 != 0) return hipErrorInvalidValue;
  const OoSplit sp = oo_split(M, N, K);
  const int ns = sp.count;
  const int tblocks = (M + 31) / 32, groups = (N / 32 + 3) / 4;
  if (tblocks > 65535 || groups > 65535) return hipErrorInvalidValue;
  float* part = static_cast<float*>(workspace);
  hipLaunchKernelGGL(oo_splitk_gemm_kernel, dim3(ns, groups, tblocks), dim3(256), 0, stream, M, N, K, sp.split_len, act,
                     w_op, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t count4 = (int64_t)M * N / 4;
  hipLaunchKernelGGL(reduce_bf16_kernel, dim3((unsigned)((count4 + 255) / 256)), dim3(256), 0, stream, count4, ns, part,
                     y);
  return hipGetLastError();
}

}  // namespace mla
