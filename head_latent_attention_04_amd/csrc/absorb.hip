// Query absorption: q_abs[r, h, :] = W_UK[h]^T q_nope[r, h, :], joined to the rotated RoPE query.
//
// "论文复现工坊 No.4", section 4: the key up-projection W_UK is folded into the query
// (Q_absorbed = Q W_UK^T) and the product is scored directly against the cached latent c^KV;
// "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA的數學原理": x_t (W_q W_k^T) c_i^T.
//
// Output element (r, h, 0:576) = [q_abs (512) | q_rope (64)], bf16, i.e. the query side of a
// 576-wide dot product with a cache row [c_KV | k_R], stored in the attention kernel's operand order
// (q_perm_offset; the padding heads of the last 32-head tile are written as zeros).
//
// Per head this is a small GEMM, computed transposed with bf16 MFMA:
//   q_abs^T[c, r] = sum_d W_UK[h][d][c] q_nope[r, h, d]     (M = c, N = r, K = d)
// One work-group per (head, half of the 512 latent columns, a range of 32-row blocks), ordered so that
// the 8 heads whose pieces share an output line run on one XCD (absorb_coords). The 128 x 256
// slice of W_UK[h] is staged in LDS once (rows padded to 544 bytes so the transposed reads of 4 rows hit
// different banks) and read with ds_read_b64_tr_b16 as the d-contiguous A operand; q_nope rows are
// the B operand straight from global memory. fp32 accumulation, one bf16 rounding.
//
// rope_absorb_kernel runs the RoPE rotation and cache append of the same tokens (rope_device.h) in
// the same launch, on work-groups of their own.
#include <algorithm>

#include "rope_device.h"

namespace mla {

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kCols = 256;                 // latent columns per work-group
constexpr int kPitch = kCols * 2 + 32;     // LDS row pitch in bytes (544)

__device__ __forceinline__ i16x4 lds_tr16(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}
}  // namespace

constexpr int kAbsorbLds = kDnope * kPitch;  // bytes of LDS one absorption work-group uses

// Work-group (head h, column half ch, rows rbase .. rbase + rows_per_wg - 1). q_rope == nullptr: the
// RoPE part of the rows is written by someone else (the fused RoPE work-groups). kPlain: write the
// rows as plain [rows, n_heads, 576] (whole 16-byte runs of one row per lane pair, so a work-group
// fills whole lines: the layout for many rows) instead of the attention kernel's operand order
// (whose lines mix 32 heads, so a work-group writes 16-byte pieces of lines other work-groups share).
template <bool kPlain>
__device__ __forceinline__ void absorb_tile(int h, int ch, int rbase, int rows, int n_heads, int rows_per_wg,
                                            const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
                                            const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_abs,
                                            char* w_lds) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, kh = lane >> 5;
  const int tiles = q_tiles(n_heads);
  lds_char* lds = (lds_char*)w_lds;

  // element (r, d) of this head in the output layout
  auto out_off = [&](int64_t r, int d) -> int64_t {
    if constexpr (kPlain) return (r * n_heads + h) * kRow + d;
    return q_perm_offset(r, tiles, h, d);
  };
  if (h >= n_heads) {  // padding head of the last tile: zero query (columns of this half, RoPE part in half 0)
    if constexpr (kPlain) return;  // no padding heads in the plain layout
    const int cols = ch == 0 ? kCols + kDr : kCols;
    for (int i = tid; i < rows_per_wg * (cols / 8); i += 256) {
      const int r = rbase + i / (cols / 8), c8 = i % (cols / 8);
      const int d = c8 * 8 < kCols ? ch * kCols + c8 * 8 : kDc + (c8 * 8 - kCols);
      if (r < rows) *reinterpret_cast<uint4*>(q_abs + out_off(r, d)) = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  // The query rows of this work-group's first block of 32 are loaded up front with W_UK, so both
  // latencies overlap; each later block's rows are loaded while the previous block computes.
  // B operand: q_nope[r][h][16 ks + 8 kh .. +7], r = r0 + (lane & 31).
  bf16x8 qb[8], qn[8];
  auto load_q = [&](bf16x8* dst, int r0) {
    const int r = r0 + (lane & 31);
    const uint4* qsrc = reinterpret_cast<const uint4*>(q_nope + ((int64_t)min(r, rows - 1) * n_heads + h) * kDnope);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) dst[ks] = __builtin_bit_cast(bf16x8, qsrc[2 * ks + kh]);
  };
  load_q(qb, rbase);
  // stage W_UK[h][:, ch*256 : ch*256 + 256]; each slice is read by one work-group, so the loads carry
  // the non-temporal hint (0.3 us of 7.5 in an A/B; outputs identical)
  const uint16_t* wsrc = w_uk + (int64_t)h * kDnope * kDc + ch * kCols;
  {
    constexpr int kPer = kDnope * (kCols / 8) / 256;  // 16 loads per thread, all issued before any store
    u32x4 v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + 256 * k, d = i / (kCols / 8), c8 = i % (kCols / 8);
      v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc + (int64_t)d * kDc + c8 * 8));
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + 256 * k, d = i / (kCols / 8), c8 = i % (kCols / 8);
      *reinterpret_cast<u32x4*>(w_lds + d * kPitch + c8 * 16) = v[k];
    }
  }
  // the RoPE part of the row is copied unchanged (column half 0 does it)
  if (ch == 0 && q_rope != nullptr) {
    for (int i = tid; i < rows_per_wg * (kDr / 8); i += 256) {
      const int r = rbase + i / (kDr / 8), c8 = i % (kDr / 8);
      if (r < rows)
        *reinterpret_cast<uint4*>(q_abs + out_off(r, kDc + 8 * c8)) =
            reinterpret_cast<const uint4*>(q_rope + ((int64_t)r * n_heads + h) * kDr)[c8];
    }
  }
  __syncthreads();

  // A operand (W^T, d-contiguous): in 16-lane group g, lane i supplies row d0 + i/4 at column
  // c0 + 4 (i%4); lane then holds W[d0 + j][c0 + i], j = 0..3.
  const int i16 = lane & 15, g = lane >> 4;
  const uint32_t abase = ((i16 >> 2) + 8 * kh) * kPitch + (16 * (g & 1) + 4 * (i16 & 3)) * 2;

  const int rend = min(rows, rbase + rows_per_wg);
  for (int r0 = rbase; r0 < rend; r0 += 32) {
    const int r = r0 + (lane & 31);  // rows past the end compute from the last row and are not stored
    if (r0 + 32 < rend) load_q(qn, r0 + 32);
#pragma unroll
    for (int cbi = 0; cbi < 2; ++cbi) {
      const int cb = (wave * 2 + cbi) * 32;  // column block within the half
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const lds_char* p = lds + abase + (16 * ks) * kPitch + cb * 2;
        const i16x4 lo = lds_tr16(p);
        const i16x4 hi = lds_tr16(p + 4 * kPitch);
        const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qb[ks], acc, 0, 0, 0);
      }
      // Lane (row, kh) holds columns 8 q + 4 kh .. +3 of its row. For each pair of groups (q, q+1) the
      // lanes l and l ^ 32 trade halves so that the low lane writes group q and the high lane group
      // q+1 as whole 16-byte pieces (8 consecutive columns, one operand-order chunk). v_permlane32_swap
      // (x, y) leaves the low lane its own x and the high lane's x, and the high lane the low lane's y
      // and its own y, so with x = group q and y = group q+1 both lanes read their piece in the same
      // order.
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[2 * q] = (uint32_t)f32_to_bf16(acc[4 * q]) | ((uint32_t)f32_to_bf16(acc[4 * q + 1]) << 16);
        w[2 * q + 1] = (uint32_t)f32_to_bf16(acc[4 * q + 2]) | ((uint32_t)f32_to_bf16(acc[4 * q + 3]) << 16);
      }
#pragma unroll
      for (int q = 0; q < 4; q += 2) {
        const auto r0 = __builtin_amdgcn_permlane32_swap(w[2 * q], w[2 * q + 2], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(w[2 * q + 1], w[2 * q + 3], false, false);
        const uint4 v = make_uint4(r0[0], r1[0], r0[1], r1[1]);
        const int d = ch * kCols + cb + 8 * (q + kh);
        if (r < rows) *reinterpret_cast<uint4*>(q_abs + out_off(r, d)) = v;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[ks] = qn[ks];
  }
}

// Absorption work-group a (0 <= a < 8 * n_units, in launch order) -> (head, column half, first row).
// A unit is 8 consecutive heads with the same column half and row block: the 16-byte pieces its
// work-groups write make up whole 128-byte lines of the operand-order output (a line holds one
// 8-element chunk of 8 heads). Work-groups are dealt to the 8 XCDs round-robin by launch index, so
// unit u takes the launch indices 64 (u / 8) + 8 e + u % 8 (e = 0..7, its heads): all of a unit runs
// on one XCD, whose L2 merges the pieces into whole lines before they are written back (pieces of
// one line from eight XCDs would be written back one by one). Units past the last multiple of 8
// keep the plain order. (Any assignment is correct; this one is about the write traffic.)
__device__ __forceinline__ void absorb_coords(int a, int hp, int zb, int rows_per_wg, int* h, int* ch, int* r0) {
  const int octets = hp / 8;
  const int n_units = octets * (kDc / kCols) * zb;
  const int full = n_units & ~7;
  int u, e;
  if (a < 8 * full) {
    u = (a & 7) + 8 * (a >> 6);
    e = (a >> 3) & 7;
  } else {
    u = full + ((a - 8 * full) >> 3);
    e = (a - 8 * full) & 7;
  }
  *h = 8 * (u % octets) + e;
  *ch = (u / octets) % (kDc / kCols);
  *r0 = (u / (octets * (kDc / kCols))) * rows_per_wg;
}

template <bool kPlain>
__global__ void __launch_bounds__(256) absorb_mfma_kernel(int rows, int n_heads, int rows_per_wg, int zb,
                                                          const uint16_t* __restrict__ q_nope,
                                                          const uint16_t* __restrict__ q_rope,
                                                          const uint16_t* __restrict__ w_uk,
                                                          uint16_t* __restrict__ q_abs) {
  __shared__ __attribute__((aligned(16))) char w_lds[kAbsorbLds];
  int h, ch, r0;
  absorb_coords(blockIdx.x, 32 * q_tiles(n_heads), zb, rows_per_wg, &h, &ch, &r0);
  absorb_tile<kPlain>(h, ch, r0, rows, n_heads, rows_per_wg, q_nope, q_rope, w_uk, q_abs, w_lds);
}

// RoPE + append and absorption in one launch: the first n_rope work-groups are (token, head group)
// RoPE work-groups that also write the rotated query into the RoPE part of the absorbed rows (row i
// is token i); the rest are the absorption's (head, column half, row range) work-groups, which leave
// that part alone. The two sets touch disjoint outputs and run side by side. n_rope_slots (a multiple
// of 8, >= n_rope) keeps the absorption's launch indices aligned to the XCD rotation; RoPE slots past
// n_rope do nothing.
__global__ void __launch_bounds__(256) rope_absorb_kernel(CacheView cache, int n_heads, const int32_t* __restrict__ token_seq,
                                                          const int32_t* __restrict__ token_pos,
                                                          const uint16_t* __restrict__ c_kv,
                                                          const uint16_t* __restrict__ k_rope,
                                                          uint16_t* __restrict__ q_rope, double log2_theta, int n_rope,
                                                          int n_rope_slots, int rows, int rows_per_wg, int zb,
                                                          const uint16_t* __restrict__ q_nope,
                                                          const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_abs) {
  __shared__ __attribute__((aligned(16))) char smem[kAbsorbLds];
  const int tiles = q_tiles(n_heads);
  if ((int)blockIdx.x < n_rope_slots) {
    if ((int)blockIdx.x >= n_rope) return;
    const int groups = rope_groups(n_heads);
    rope_token_group(cache, n_heads, blockIdx.x / groups, blockIdx.x % groups, token_seq, token_pos, c_kv, k_rope,
                     q_rope, log2_theta, q_abs, tiles, reinterpret_cast<double*>(smem));
    return;
  }
  int h, ch, r0;
  absorb_coords(blockIdx.x - n_rope_slots, 32 * tiles, zb, rows_per_wg, &h, &ch, &r0);
  absorb_tile<false>(h, ch, r0, rows, n_heads, rows_per_wg, q_nope, nullptr, w_uk, q_abs, smem);
}

namespace {
// blocks of 32 rows per work-group: one for small batches, more when there are many rows, so that
// about 1024 work-groups each stage their W_UK slice once
int absorb_rows_per_wg(int rows, int n_heads) {
  const int hp = 32 * q_tiles(n_heads);
  const int64_t nrb = (rows + 31) / 32;
  const int64_t bpw = std::max<int64_t>(1, (nrb * hp * 2 + 1023) / 1024);
  return (int)std::min<int64_t>(32 * bpw, 32 * nrb);
}
}  // namespace

hipError_t launch_absorb(int rows, int n_heads, const uint16_t* q_nope, const uint16_t* q_rope,
                         const uint16_t* w_uk, uint16_t* q_abs, bool plain, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int hp = 32 * q_tiles(n_heads);
  const int rows_per_wg = absorb_rows_per_wg(rows, n_heads);
  const int zb = (rows + rows_per_wg - 1) / rows_per_wg;
  const int64_t nwg = (int64_t)hp * (kDc / kCols) * zb;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (plain)
    hipLaunchKernelGGL(absorb_mfma_kernel<true>, dim3((unsigned)nwg), dim3(256), 0, stream, rows, n_heads, rows_per_wg,
                       zb, q_nope, q_rope, w_uk, q_abs);
  else
    hipLaunchKernelGGL(absorb_mfma_kernel<false>, dim3((unsigned)nwg), dim3(256), 0, stream, rows, n_heads, rows_per_wg,
                       zb, q_nope, q_rope, w_uk, q_abs);
  return hipGetLastError();
}

hipError_t launch_rope_absorb(const CacheView& cache, int n_heads, int num_tokens, const int32_t* token_seq,
                              const int32_t* token_pos, const uint16_t* c_kv, const uint16_t* k_rope, uint16_t* q_rope,
                              float theta, const uint16_t* q_nope, const uint16_t* w_uk, uint16_t* q_abs,
                              hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int hp = 32 * q_tiles(n_heads);
  const int rows_per_wg = absorb_rows_per_wg(num_tokens, n_heads);
  const int64_t zb = (num_tokens + rows_per_wg - 1) / rows_per_wg;
  const int64_t n_rope = (int64_t)num_tokens * rope_groups(n_heads);
  const int64_t n_rope_slots = (n_rope + 7) & ~(int64_t)7;
  const int64_t total = n_rope_slots + (int64_t)hp * (kDc / kCols) * zb;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_absorb_kernel, dim3((unsigned)total), dim3(256), 0, stream, cache, n_heads, token_seq, token_pos,
                     c_kv, k_rope, q_rope, log2((double)theta), (int)n_rope, (int)n_rope_slots, num_tokens, rows_per_wg,
                     (int)zb, q_nope, w_uk, q_abs);
  return hipGetLastError();
}

}  // namespace mla
