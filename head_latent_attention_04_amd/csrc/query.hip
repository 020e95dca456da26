// The query path with the query and key projections multiplied ahead of time: the absorbed query
// rows the decode kernel scores come straight from the hidden state.
//
// ("论文复现工坊 No.4", section 2: wq_a, the RMSNorm q_norm over q_lora_rank values, wq_b whose
// per-head output is [q_nope | q_R]; section 4: the absorbed query is scored against c_KV directly.
// "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA的數學原理": the product of the query and key
// projections can be formed once, x_t (W_q W_k^T) c_i^T.)
//
//   W_UQK[h] = W_UK[h]^T W_UQ_nope[h]                  [d_c, q_rank], once per weight set
//   c_q      = q_norm(x W_DQ^T)                         [T, q_rank]
//   q_abs[t, h] = [W_UQK[h] c_q[t] | R_pos(t) (W_QR[h] c_q[t])]     [T, n_h, 576]
//
// Kernels:
//   * absorb_query_weights_kernel: the prepared weight, head h's 576 rows [W_UQK[h]; W_QR[h]] in MFMA
//     operand order (wq_offset); W_UQK in fp32 outer products over the 128 rows of W_UK[h] and
//     W_UQ_nope[h] (both read as whole rows), rounded once to bf16.
//   * c_q: the split-K GEMM of gemm_bt.hip, then cq_finish_kernel (one work-group per token: add the
//     splits, round, RMSNorm, round; and the token's 32 RoPE cos/sin pairs in fp64 for the query
//     kernel).
//   * query_gemm_kernel: work-group (32 tokens, head, 32 output columns of the head's 576): the
//     columns are rows 32 j .. +31 of the prepared weight; four waves split the K range (q_rank),
//     each operand load one contiguous 1 KB (both c_q and the weight are in operand order), and add
//     through LDS; each thread then owns 4 consecutive columns of one token, so the RoPE pairs are
//     rotated without lane exchanges. Written as bf16 rows [T, n_h, 576], the plain layout
//     mla_decode_absorbed takes.
#include <algorithm>

#include "finish_device.h"

namespace mla {

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQrankMax = 2048;

// Prepared query weight: head h's 576 rows (W_UQK[h] rows 0..511, then the q_R rows of W_UQ) in MFMA
// operand order: row n, element k at
//   (((h * 18 + n / 32) * (q_rank / 16) + k / 16) * 64 + n % 32 + 32 ((k / 8) % 2)) * 8 + k % 8,
// so the operand of one wave for one K step of a 32-row tile is one contiguous 1 KB.
__host__ __device__ inline int64_t wq_offset(int h, int n, int k, int q_rank) {
  return ((((int64_t)h * (kRow / 32) + n / 32) * (q_rank / 16) + k / 16) * 64 + n % 32 + 32 * ((k / 8) & 1)) * 8 + k % 8;
}
// c_q is in the same order for 32-token blocks (cq_offset, finish_device.h).

struct QueryWorkspace {
  size_t part, cq, cs, total;
};

QueryWorkspace query_layout(int num_tokens, int dim, int q_rank) {
  QueryWorkspace w;
  const size_t ns = (size_t)splitk_splits(num_tokens, q_rank, dim);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  w.part = 0;
  w.cq = al(ns * num_tokens * q_rank * 4);
  w.cs = w.cq + al((size_t)((num_tokens + 31) / 32) * 32 * q_rank * 2);
  w.total = w.cs + al((size_t)num_tokens * (kDr / 2) * 2 * sizeof(double));
  return w;
}
}  // namespace

// ---- prepared weight: W_UQK = W_UK^T W_UQ_nope per head, and the q_R rows of W_UQ ----------------------
// Work-group (head, 64 latent rows c, 64 rank columns r) for blockIdx.y < 8: thread (ty, tx)
// accumulates the 4 x 4 outputs c = c0 + 4 ty .. +3, r = r0 + 4 tx .. +3 over d < 128; rows d of
// W_UK[h] and W_UQ_nope[h] are staged in LDS 16 at a time. blockIdx.y == 8 copies the head's 64
// q_R rows (columns r0 .. r0 + 63) into their place.
__global__ void __launch_bounds__(256) absorb_query_weights_kernel(int q_rank, const uint16_t* __restrict__ w_uq,
                                                                   const uint16_t* __restrict__ w_uk,
                                                                   uint16_t* __restrict__ w_q) {
  __shared__ float sk[16][64], sq[16][64];
  const int h = blockIdx.x, c0 = 64 * blockIdx.y, r0 = 64 * blockIdx.z;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const uint16_t* uq = w_uq + (int64_t)h * (kDnope + kDr) * q_rank;  // head h's nope rows, then its q_R rows
  if (c0 >= kDc) {
    for (int e = tid; e < kDr * 16; e += 256) {  // 64 rows x 16 groups of 4 columns
      const int n = e >> 4, k = r0 + 4 * (e & 15);
      const uint2 v = *reinterpret_cast<const uint2*>(uq + (int64_t)(kDnope + n) * q_rank + k);
      *reinterpret_cast<uint2*>(w_q + wq_offset(h, kDc + n, k, q_rank)) = v;
    }
    return;
  }
  const uint16_t* uk = w_uk + (int64_t)h * kDnope * kDc;
  float acc[4][4] = {};
  for (int d0 = 0; d0 < kDnope; d0 += 16) {
    for (int e = tid; e < 16 * 64; e += 256) {
      const int dd = e >> 6, cc = e & 63;
      sk[dd][cc] = bf16_to_f32(uk[(int64_t)(d0 + dd) * kDc + c0 + cc]);
      sq[dd][cc] = bf16_to_f32(uq[(int64_t)(d0 + dd) * q_rank + r0 + cc]);
    }
    __syncthreads();
#pragma unroll
    for (int dd = 0; dd < 16; ++dd) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = sk[dd][4 * ty + i];
        b[i] = sq[dd][4 * tx + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  // 4 consecutive k (r0 + 4 tx .. +3) share one 8-byte piece of the operand order
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint2 v = make_uint2((uint32_t)f32_to_bf16(acc[i][0]) | ((uint32_t)f32_to_bf16(acc[i][1]) << 16),
                               (uint32_t)f32_to_bf16(acc[i][2]) | ((uint32_t)f32_to_bf16(acc[i][3]) << 16));
    *reinterpret_cast<uint2*>(w_q + wq_offset(h, c0 + 4 * ty + i, r0 + 4 * tx, q_rank)) = v;
  }
}

// ---- c_q: split sums, RMSNorm; RoPE angles (cq_finish_token, finish_device.h) ---------------------------
__global__ void __launch_bounds__(256) cq_finish_kernel(int num_tokens, int q_rank, int nsplit,
                                                        const int32_t* __restrict__ token_pos,
                                                        const float* __restrict__ part,
                                                        const uint16_t* __restrict__ gamma, float eps,
                                                        double log2_theta, uint16_t* __restrict__ c_q,
                                                        double* __restrict__ cs) {
  __shared__ float s_sum[4];
  cq_finish_token(blockIdx.x, num_tokens, q_rank, nsplit, token_pos, part, q_rank, gamma, eps, log2_theta, c_q, cs,
                  s_sum);
}

// ---- q_abs rows -----------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) query_gemm_kernel(int num_tokens, int n_heads, int q_rank,
                                                         const uint16_t* __restrict__ c_q,
                                                         const uint16_t* __restrict__ w_q,
                                                         const double* __restrict__ cs,
                                                         uint16_t* __restrict__ q_abs) {
  __shared__ float red[4 * 32 * 32];
  const int j = blockIdx.x, h = blockIdx.y, tb = blockIdx.z;  // j < 18: 32-column tile of the head's row
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ksteps = q_rank / 16, steps = ksteps / 4, ks0 = wave * steps;  // the wave's quarter of K
  // both operands in operand order: K step ks of the tile is the 1 KB at (tile * ksteps + ks) * 512
  const uint16_t* pa = c_q + ((int64_t)tb * ksteps + ks0) * 512 + lane * 8;
  const uint16_t* pb = w_q + (((int64_t)h * (kRow / 32) + j) * ksteps + ks0) * 512 + lane * 8;
  f32x16 acc = f32x16{};
  // the wave's K range (q_rank / 4 <= 512, up to 32 steps) in groups of 8 loads in flight
  for (int k = 0; k < steps; k += 8) {
    bf16x8 a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k + u < steps) {
        a[u] = *reinterpret_cast<const bf16x8*>(pa + (k + u) * 512);
        // the prepared weight is read once per call: non-temporal hint
        b[u] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(pb + (k + u) * 512));
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k + u < steps) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], acc, 0, 0, 0);
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
  // D: lane holds token 8 (e / 4) + 4 (lane / 32) + e % 4 and column lane % 32 of the tile
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int m = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    red[(wave * 32 + m) * 32 + (lane & 31)] = acc[e];
  }
  __syncthreads();
  // thread: token m = tid / 8, columns 4 (tid % 8) .. +3 of the tile
  const int m = threadIdx.x >> 3, c4 = threadIdx.x & 7;
  const int t = 32 * tb + m;
  if (t >= num_tokens) return;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = m * 32 + 4 * c4 + e;
    v[e] = bf16_to_f32(f32_to_bf16(red[idx] + red[1024 + idx] + red[2048 + idx] + red[3072 + idx]));
  }
  uint32_t w0, w1;
  if (j < kDc / 32) {
    w0 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    w1 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  } else {
    // q_R pairs (2 p, 2 p + 1), p = 16 (j - 16) + 2 c4 + {0, 1}: turned by the token's angles
    const int p = 16 * (j - kDc / 32) + 2 * c4;
    const double* a = cs + ((int64_t)t * (kDr / 2) + p) * 2;
    w0 = rope_turn_pair((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16), a[0], a[1]);
    w1 = rope_turn_pair((uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16), a[2], a[3]);
  }
  *reinterpret_cast<uint2*>(q_abs + ((int64_t)t * n_heads + h) * kRow + 32 * j + 4 * c4) = make_uint2(w0, w1);
}

size_t query_workspace_bytes(int num_tokens, int dim, int q_rank) { return query_layout(num_tokens, dim, q_rank).total; }

namespace {
hipError_t launch_query_rows(int n_heads, int num_tokens, int q_rank, const uint16_t* c_q, const uint16_t* w_q,
                             const double* cs, uint16_t* q_abs, hipStream_t stream) {
  const int tblocks = (num_tokens + 31) / 32;
  if (tblocks > 65535 || n_heads > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(query_gemm_kernel, dim3(kRow / 32, n_heads, tblocks), dim3(256), 0, stream, num_tokens, n_heads,
                     q_rank, c_q, w_q, cs, q_abs);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_absorb_query_weights(int n_heads, int q_rank, const uint16_t* w_uq, const uint16_t* w_uk,
                                       uint16_t* w_q, hipStream_t stream) {
  if (q_rank % 64 != 0 || q_rank > kQrankMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(absorb_query_weights_kernel, dim3(n_heads, kDc / 64 + 1, q_rank / 64), dim3(256), 0, stream,
                     q_rank, w_uq, w_uk, w_q);
  return hipGetLastError();
}

hipError_t launch_query_absorbed(int n_heads, int num_tokens, const int32_t* token_pos, const uint16_t* x, int dim,
                                 const uint16_t* w_dq, const uint16_t* gamma_q, float eps, int q_rank,
                                 const uint16_t* w_q, float theta, void* workspace, uint16_t* q_abs,
                                 hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  if (q_rank % 64 != 0 || q_rank > kQrankMax || dim % 64 != 0) return hipErrorInvalidValue;
  const QueryWorkspace lay = query_layout(num_tokens, dim, q_rank);
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + lay.part);
  uint16_t* c_q = reinterpret_cast<uint16_t*>(ws + lay.cq);
  double* cs = reinterpret_cast<double*>(ws + lay.cs);
  const int ns = splitk_splits(num_tokens, q_rank, dim);
  hipError_t e = launch_splitk_gemm(num_tokens, q_rank, dim, ns, x, w_dq, part, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cq_finish_kernel, dim3(num_tokens), dim3(256), 0, stream, num_tokens, q_rank, ns, token_pos, part,
                     gamma_q, eps, log2((double)theta), c_q, cs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_query_rows(n_heads, num_tokens, q_rank, c_q, w_q, cs, q_abs, stream);
}

// ---- the KV down-projection and the absorbed query rows of the same tokens, launches shared -----------
// Both down-projections read x: one split-K GEMM over the stacked weights [W_DKV; W_DQ] (fp32 partials
// [split][token][576 + q_rank]), one finishing launch (work-groups 0 .. T-1 the KV side of token i,
// T .. 2T-1 its query side), then the query GEMM: three launches instead of five. The split count is
// the smaller of the two single-projection counts, so where those agree every result is bit for bit
// that of launch_kv_down followed by launch_query_absorbed. Token counts that take the tiled KV GEMM
// run the two paths one after the other.
__global__ void __launch_bounds__(256) kv_q_finish_kernel(CacheView cache, int num_tokens, int q_rank, int nsplit,
                                                          const int32_t* __restrict__ token_seq,
                                                          const int32_t* __restrict__ token_pos,
                                                          const float* __restrict__ part,
                                                          const uint16_t* __restrict__ gamma_kv, float eps_kv,
                                                          const uint16_t* __restrict__ gamma_q, float eps_q,
                                                          double log2_theta, uint16_t* __restrict__ c_q,
                                                          double* __restrict__ cs) {
  __shared__ float s_sum[4];
  const int ld = kKvRowOut + q_rank;
  if ((int)blockIdx.x < num_tokens)
    kv_finish_token(cache, blockIdx.x, num_tokens, nsplit, token_seq, token_pos, part, ld, gamma_kv, eps_kv,
                    log2_theta, s_sum);
  else
    cq_finish_token(blockIdx.x - num_tokens, num_tokens, q_rank, nsplit, token_pos, part + kKvRowOut, ld, gamma_q,
                    eps_q, log2_theta, c_q, cs, s_sum);
}

namespace {
int kvq_splits(int num_tokens, int dim, int q_rank) {
  return std::min(splitk_splits(num_tokens, kKvRowOut, dim), splitk_splits(num_tokens, q_rank, dim));
}

QueryWorkspace kvq_layout(int num_tokens, int dim, int q_rank) {
  QueryWorkspace w;
  const size_t ns = (size_t)kvq_splits(num_tokens, dim, q_rank);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  w.part = 0;
  w.cq = al(ns * num_tokens * (kKvRowOut + q_rank) * 4);
  w.cs = w.cq + al((size_t)((num_tokens + 31) / 32) * 32 * q_rank * 2);
  w.total = w.cs + al((size_t)num_tokens * (kDr / 2) * 2 * sizeof(double));
  return w;
}

size_t aligned256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

size_t kv_down_query_workspace_bytes(int num_tokens, int dim, int q_rank) {
  if (kv_down_tiled_path(num_tokens))
    return aligned256(kv_down_workspace_bytes(num_tokens, dim)) + query_workspace_bytes(num_tokens, dim, q_rank);
  return kvq_layout(num_tokens, dim, q_rank).total;
}

hipError_t launch_kv_down_query(const CacheView& cache, int n_heads, int num_tokens, const int32_t* token_seq,
                                const int32_t* token_pos, const uint16_t* x, int dim, const uint16_t* w_dkv,
                                const uint16_t* gamma_kv, float eps_kv, const uint16_t* w_dq, const uint16_t* gamma_q,
                                float eps_q, int q_rank, const uint16_t* w_q, float theta, void* workspace,
                                uint16_t* q_abs, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  if (q_rank % 64 != 0 || q_rank > kQrankMax || dim % 64 != 0) return hipErrorInvalidValue;
  char* ws = static_cast<char*>(workspace);
  if (kv_down_tiled_path(num_tokens)) {
    hipError_t e = launch_kv_down(cache, num_tokens, token_seq, token_pos, x, dim, w_dkv, gamma_kv, eps_kv, theta, ws,
                                  stream);
    if (e != hipSuccess) return e;
    return launch_query_absorbed(n_heads, num_tokens, token_pos, x, dim, w_dq, gamma_q, eps_q, q_rank, w_q, theta,
                                 ws + aligned256(kv_down_workspace_bytes(num_tokens, dim)), q_abs, stream);
  }
  const QueryWorkspace lay = kvq_layout(num_tokens, dim, q_rank);
  float* part = reinterpret_cast<float*>(ws + lay.part);
  uint16_t* c_q = reinterpret_cast<uint16_t*>(ws + lay.cq);
  double* cs = reinterpret_cast<double*>(ws + lay.cs);
  const int ns = kvq_splits(num_tokens, dim, q_rank);
  hipError_t e = launch_splitk_gemm2(num_tokens, kKvRowOut, q_rank, dim, ns, x, w_dkv, w_dq, part, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_q_finish_kernel, dim3(2 * num_tokens), dim3(256), 0, stream, cache, num_tokens, q_rank, ns,
                     token_seq, token_pos, part, gamma_kv, eps_kv, gamma_q, eps_q, log2((double)theta), c_q, cs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_query_rows(n_heads, num_tokens, q_rank, c_q, w_q, cs, q_abs, stream);
}

}  // namespace mla
