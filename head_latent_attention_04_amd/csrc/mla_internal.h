// Internal declarations shared by the kernels and the C-ABI layer of the MLA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// The one shape the kernels are written for (DeepSeek-V2 dimensions: "Multi-Head Latent Attention:
// DeepSeek V2/V3 工程视角", section 一; module defaults of "论文复现工坊 No.4", section 2).
constexpr int kDc = 512;            // latent c_KV width
constexpr int kDr = 64;             // decoupled RoPE width
constexpr int kRow = kDc + kDr;     // 576 elements per cached token
constexpr int kRowBytes = kRow * 2; // 1152 bytes in bf16
constexpr int kDnope = 128;
constexpr int kDv = 128;
constexpr int kBlock = 64;          // tokens per cache block

struct CacheView {
  uint16_t* data;
  const int32_t* table;  // nullptr: contiguous
  int32_t max_blocks;
};

// ---- bf16 helpers -------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// two floats -> packed bf16 pair (low half = a), round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// double -> bf16, round to nearest even: first to float rounding toward zero with a sticky
// low bit (round-to-odd), which keeps the exact tie information, then float -> bf16 RNE.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  float t = __double2float_rz(x);
  uint32_t u = __float_as_uint(t);
  if ((double)t != x) u |= 1u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ int64_t row_offset(const CacheView& c, int seq, int pos) {
  int blk = pos / kBlock;
  int64_t phys = c.table ? (int64_t)c.table[(int64_t)seq * c.max_blocks + blk]
                         : (int64_t)seq * c.max_blocks + blk;
  return (phys * kBlock + (pos % kBlock)) * (int64_t)kRow;
}

// ---- absorbed-query layout between the absorb and attention kernels ------------------------------
// Heads are grouped in tiles of 32 (the last tile padded with zero queries). Within (row, tile) the
// 576 elements are stored in the order the score MFMA consumes them: element (h, d) sits at
//   [d / 16][32 * ((d / 8) % 2) + h % 32][d % 8],
// so operand step d/16 of a whole wave is one contiguous 1 KB load (lane = 32 * half + head).
constexpr int kQTileElems = 32 * kRow;  // 18432 elements = 36 KB per (row, head tile)

__host__ __device__ inline int q_tiles(int n_heads) { return (n_heads + 31) / 32; }

__host__ __device__ inline int64_t q_perm_offset(int64_t row, int tiles, int h, int d) {
  return ((row * tiles + (h >> 5)) * (kRow / 16) + (d >> 4)) * 512 + ((((d >> 3) & 1) << 5) + (h & 31)) * 8 + (d & 7);
}

// ---- launchers (each returns the launch status) ---------------------------------------------------
hipError_t launch_rope_append(const CacheView& cache, int n_heads, int num_tokens, const int32_t* token_seq,
                              const int32_t* token_pos, const uint16_t* c_kv, const uint16_t* k_rope,
                              uint16_t* q_rope, float theta, hipStream_t stream);

// q_abs(r, h, 0:512) = W_UK[h]^T q_nope[r, h]; q_abs(r, h, 512:576) = q_rope[r, h] (bf16), r < rows,
// written in the operand-order layout above (padding heads zero), or, if plain, as [rows, n_heads, 576].
hipError_t launch_absorb(int rows, int n_heads, const uint16_t* q_nope, const uint16_t* q_rope,
                         const uint16_t* w_uk, uint16_t* q_abs, bool plain, hipStream_t stream);

// launch_rope_append (with the query) and launch_absorb of the same num_tokens rows in one launch:
// row i of q_abs is token i, its RoPE part the query launch_rope_append rotates in place.
hipError_t launch_rope_absorb(const CacheView& cache, int n_heads, int num_tokens, const int32_t* token_seq,
                              const int32_t* token_pos, const uint16_t* c_kv, const uint16_t* k_rope, uint16_t* q_rope,
                              float theta, const uint16_t* q_nope, const uint16_t* w_uk, uint16_t* q_abs,
                              hipStream_t stream);

// Split-KV attention over the latent cache with bf16 MFMA. Row r of the work is one query token:
// decode (cu_q_lens == nullptr): row r is sequence r and sees its seq_lens[r] tokens; prefill: row j
// is query token j (sequence located through cu_q_lens[0..batch]) and sees tokens 0..its position.
// q_abs is in the operand-order layout (q_operand_order) or plain [rows, n_heads, 576].
// Writes per (row, head, split) the normalised latent partial (bf16, [rows, n_heads, splits, 512])
// and its log-sum-exp (fp32, natural log).
hipError_t launch_attention(const CacheView& cache, int rows, int n_heads, const int32_t* seq_lens,
                            const int32_t* cu_q_lens, int batch, const uint16_t* q_abs, bool q_operand_order,
                            float scale, int split_tokens, int num_splits, uint16_t* o_partial, float* lse_partial,
                            hipStream_t stream);

// Tiled bf16 GEMM, fp32 partials over K splits: part[s][m][n] = sum_{k in split s} A[m][k] B[n][k].
// A [M, K], B [N, K] row-major bf16; N % kGemmBN == 0, K % 64 == 0, 1 <= nsplit <= K / 64.
constexpr int kGemmBM = 128, kGemmBN = 192, kGemmMaxSplits = 16;
int gemm_bt_splits(int M, int N, int K);
hipError_t launch_gemm_bt_partial(int M, int N, int K, int nsplit, const uint16_t* A, const uint16_t* B, float* part,
                                  hipStream_t stream);

// Split-K GEMM for few rows, fp32 partials: part[s][m][n] = sum_{k in split s} A[m][k] B[n][k]
// (A [M, K], B [N, K] row-major bf16; N % 32 == 0, K % 64 == 0, nsplit divides K / 64).
int splitk_splits(int M, int N, int K);
hipError_t launch_splitk_gemm(int M, int N, int K, int nsplit, const uint16_t* A, const uint16_t* B, float* part,
                              hipStream_t stream);
// The same over two weights stacked by rows: columns n < N1 from B [N1, K], the rest from B2 [N2, K]
// (N1, N2 multiples of 32); part[s][m][N1 + N2].
hipError_t launch_splitk_gemm2(int M, int N1, int N2, int K, int nsplit, const uint16_t* A, const uint16_t* B,
                               const uint16_t* B2, float* part, hipStream_t stream);

// Query path with W_UQ W_UK absorbed ahead of time: the prepared weight w_q = head h's rows
// [W_UQK[h] = W_UK[h]^T W_UQ_nope[h] (512 rows); W_QR[h] (64 rows)] in MFMA operand order
// ([n_heads, 576, q_rank] elements), from wq_b's weight W_UQ [n_heads (128 + 64), q_rank] and W_UK;
// then the absorbed query rows [T, n_heads, 576] (plain layout) from x [T, dim]:
// c_q = RMSNorm(x W_DQ^T), [W_UQK[h] c_q | RoPE(W_QR[h] c_q)].
hipError_t launch_absorb_query_weights(int n_heads, int q_rank, const uint16_t* w_uq, const uint16_t* w_uk,
                                       uint16_t* w_q, hipStream_t stream);
size_t query_workspace_bytes(int num_tokens, int dim, int q_rank);
hipError_t launch_query_absorbed(int n_heads, int num_tokens, const int32_t* token_pos, const uint16_t* x, int dim,
                                 const uint16_t* w_dq, const uint16_t* gamma_q, float eps, int q_rank,
                                 const uint16_t* w_q, float theta, void* workspace, uint16_t* q_abs,
                                 hipStream_t stream);

// Output side. merge: the split partials of mla_decode_attend merged into the normalised latent
// o_lat [rows, n_heads, 512] bf16 (no W_UV). Weights in MFMA operand order (prepare_rows: any
// row-major [N, K]; fold: W_OV = W_O W_UV per head, [dim, n_heads 512]). output_gemm: y [M, N] bf16
// = act [M, K] times the prepared weight's rows, split over K (workspace: fp32 partials).
hipError_t launch_merge_latent(int rows, int n_heads, int num_splits, const uint16_t* o_partial,
                               const float* lse_partial, uint16_t* o_lat, float* lse_out, hipStream_t stream);
hipError_t launch_prepare_rows(int N, int64_t K, const uint16_t* w, uint16_t* w_op, hipStream_t stream);
hipError_t launch_fold_output_weights(int dim, int n_heads, const uint16_t* w_o, const uint16_t* w_uv,
                                      uint16_t* w_ov, hipStream_t stream);
size_t output_workspace_bytes(int M, int N, int64_t K);
hipError_t launch_output_gemm(int M, int N, int64_t K, const uint16_t* act, const uint16_t* w_op, void* workspace,
                              uint16_t* y, hipStream_t stream);

// Expanded-form chunked prefill: up-projected keys and values ([batch, n_heads, lpad, 128] each,
// lpad = max_seq_len rounded up to 128, in the workspace), then causal attention with 192-wide keys.
size_t prefill_expanded_kv_bytes(int batch, int n_heads, int max_seq_len);
hipError_t launch_prefill_expanded(const CacheView& cache, int batch, int n_heads, const int32_t* seq_lens,
                                   const int32_t* cu_q_lens, int max_q_len, int max_seq_len, const uint16_t* q_nope,
                                   const uint16_t* q_rope, const uint16_t* w_uk, const uint16_t* w_uv, float scale,
                                   void* workspace, uint16_t* out, float* lse_out, hipStream_t stream);

// KV down-projection of num_tokens tokens (x [T, dim] . W_DKV^T, W_DKV [576, dim]), RMSNorm of the latent
// part (eps, weight gamma [512]), then the RoPE rotation of k_R and the append, as launch_rope_append.
// workspace: kv_down_workspace_bytes(num_tokens, dim) bytes (fp32 split partials).
size_t kv_down_workspace_bytes(int num_tokens, int dim);
bool kv_down_tiled_path(int num_tokens);  // true where the tiled GEMM (not the split-K one) runs

// launch_kv_down and launch_query_absorbed of the same tokens with shared launches (see query.hip).
size_t kv_down_query_workspace_bytes(int num_tokens, int dim, int q_rank);
hipError_t launch_kv_down_query(const CacheView& cache, int n_heads, int num_tokens, const int32_t* token_seq,
                                const int32_t* token_pos, const uint16_t* x, int dim, const uint16_t* w_dkv,
                                const uint16_t* gamma_kv, float eps_kv, const uint16_t* w_dq, const uint16_t* gamma_q,
                                float eps_q, int q_rank, const uint16_t* w_q, float theta, void* workspace,
                                uint16_t* q_abs, hipStream_t stream);
hipError_t launch_kv_down(const CacheView& cache, int num_tokens, const int32_t* token_seq, const int32_t* token_pos,
                          const uint16_t* x, int dim, const uint16_t* w_dkv, const uint16_t* gamma, float eps,
                          float theta, void* workspace, hipStream_t stream);

// Check of the caller's device-resident index data (one work-group): *error_word = OR of the kCheck*
// bits of the rules broken, 0 when none. table == nullptr: the contiguous layout; cu_q_lens == nullptr:
// decode (no chunk offsets).
constexpr int kCheckBadLength = 1, kCheckBadBlock = 2, kCheckBadOffsets = 4, kCheckChunkTooLong = 8;
hipError_t launch_check_inputs(int batch, const int32_t* seq_lens, const int32_t* table, int max_blocks,
                               int64_t num_blocks, int block_size, const int32_t* cu_q_lens, int total_q,
                               int32_t* error_word, hipStream_t stream);

// LSE merge over splits + W_UV up-projection.
hipError_t launch_combine(int batch, int n_heads, int num_splits, const uint16_t* o_partial,
                          const float* lse_partial, const uint16_t* w_uv, uint16_t* out, float* lse_out,
                          hipStream_t stream);

}  // namespace mla
