// Split-KV combine and value up-projection.
//
// The partials (bf16) of one (sequence, head) are merged with their log-sum-exps (the same softmax,
// taken in pieces): lse = ln sum_s exp(lse_s), o_lat = sum_s exp(lse_s - lse) o_s. The merged
// latent is then up-projected, out[h] = W_UV[h] o_lat: the value side is never expanded per
// token ("论文复现工坊 No.4", section 1; "Multi-Head Latent Attention: DeepSeek V2/V3 工程视角",
// section 四: the W_UV up-projection or its absorbed equivalent).
//
// One work-group per (head, range of 16-sequence blocks), 4 waves:
//   0. every load a block needs is issued before any is used: the log-sum-exps and the partials of
//      its first 8 splits, then (first block only) the wave's 32 rows of W_UV[h], kept in registers
//      across blocks; the merge waits only for the partials and overlaps W_UV's arrival;
//   1. merge: thread t merges latent columns [32 (t % 16), +32) of sequence t / 16 (fp32) and
//      stores them in LDS as a bf16 pair hi + lo (hi = bf16(o), lo = bf16(o - hi)), which carries
//      the merged latent to the MFMA with about 16 significant bits;
//   2. up-projection with bf16 MFMA (v_mfma_f32_16x16x32_bf16): out^T[v, b] = W_UV[h][v, :] . o_lat[b, :]
//      for the wave's 32 output columns v (two 16-row tiles, N = the block's 16 sequences, K = c),
//      hi and lo accumulated into the same fp32 tile.
#include <algorithm>

#include "mla_internal.h"

namespace mla {

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kRowsPerWg = 16;  // sequences per block (the 16 columns of the MFMA tile)
constexpr int kPitch = kDc * 2 + 16;  // bf16 row of 512 latent columns, padded (conflict-free b128 reads)
}  // namespace

// kChunk: splits whose partials are loaded together (1, 2, 4 or 8: the split count rounded up to a
// power of two, at most 8). With kChunk <= 2 the next block's partials are loaded while the current
// block is merged and projected, which matters when a work-group runs many blocks (prefill, S = 1).
// kGroups (1 or 4): thread groups that share one sequence's splits. With 4 (small batches with many
// splits: at most 4 sequences, each row slot of the block holds a quarter of a sequence's splits,
// s = g, g + 4, ...), the four partial merges meet in LDS, so a sequence's 64 splits take two load
// round trips instead of eight.
template <int kChunk, int kGroups>
__global__ void __launch_bounds__(256, 1) combine_mfma_kernel(int batch, int n_heads, int num_splits, int blocks_per_wg,
                                                           const uint16_t* __restrict__ o_partial,
                                                           const float* __restrict__ lse_partial,
                                                           const uint16_t* __restrict__ w_uv,
                                                           uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(16))) char hi_lds[kRowsPerWg * kPitch];
  __shared__ __attribute__((aligned(16))) char lo_lds[kRowsPerWg * kPitch];
  __shared__ float red_lds[kGroups > 1 ? kRowsPerWg * kDc : 1];  // per row slot: unnormalised sums
  __shared__ float stat_lds[2 * kRowsPerWg];                       // per row slot: max, sum of weights
  constexpr int kRows = kRowsPerWg / kGroups;                      // sequences per block
  const int h = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  const int nblk = (batch + kRows - 1) / kRows;
  const int blk_begin = blockIdx.y * blocks_per_wg;
  const int blk_end = min(nblk, blk_begin + blocks_per_wg);
  if (blk_begin >= blk_end) return;

  // Merge role: thread t owns row slot t / 16 and latent columns 32 (t % 16) .. +31 of a block; the
  // slot is sequence b0 + slot / kGroups, split group slot % kGroups, whose splits are g, g + kGroups, ...
  const int slot = tid >> 4;
  const int bl = slot / kGroups, grp = slot % kGroups;
  const int c0 = 32 * (tid & 15);
  const int n_my = num_splits > grp ? (num_splits - grp + kGroups - 1) / kGroups : 0;  // this group's splits
  auto sidx = [&](int j) { return grp + kGroups * j; };
  // The first kChunk splits of a block: log-sum-exps and partials issued together, without branches
  // (an index past the last split reads the last one and gets weight zero).
  constexpr bool kPrefetch = kChunk <= 2;
  float ls[kChunk], ls_next[kChunk];
  uint4 v[kChunk][4], v_next[kChunk][4];
  auto load_first_chunk = [&](int blk, float (&ls)[kChunk], uint4 (&v)[kChunk][4]) {
    const int b = blk * kRows + bl;
    if (b >= batch || n_my == 0) {  // a row past the batch (or a group without splits) loads nothing
#pragma unroll
      for (int q = 0; q < kChunk; ++q) {
        ls[q] = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[q][k] = make_uint4(0, 0, 0, 0);
      }
      return;
    }
    const int64_t base = ((int64_t)b * n_heads + h) * num_splits;
#pragma unroll
    for (int q = 0; q < kChunk; ++q) ls[q] = lse_partial[base + sidx(min(q, n_my - 1))];  // masked at use
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const uint4* src = reinterpret_cast<const uint4*>(o_partial + (base + sidx(min(q, n_my - 1))) * kDc + c0);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[q][k] = src[k];
    }
  };

  // W_UV rows of the up-projection (A operand of tile vt: row v = 32 wave + 16 vt + lane % 16,
  // columns 32 ks + 8 (lane / 16) .. +7), kept in registers across blocks
  bf16x8 wa[2][kDc / 32];
  auto load_wuv = [&]() {
#pragma unroll
    for (int vt = 0; vt < 2; ++vt) {
      const uint4* wrow = reinterpret_cast<const uint4*>(
          w_uv + ((int64_t)h * kDv + 32 * wave + 16 * vt + (lane & 15)) * kDc + 8 * (lane >> 4));
#pragma unroll
      for (int ks = 0; ks < kDc / 32; ++ks) wa[vt][ks] = __builtin_bit_cast(bf16x8, wrow[4 * ks]);
    }
  };

  auto process_block = [&](int blk) {
    const int b0 = blk * kRows;
    // ---- 1. merge the splits (fp32) and stage the merged latent as bf16 hi + lo
    {
      const int b = b0 + bl;
      const bool bok = b < batch && n_my > 0;
      const int64_t base = ((int64_t)(bok ? b : 0) * n_heads + h) * num_splits;
#pragma unroll
      for (int q = 0; q < kChunk; ++q) ls[q] = q < n_my ? ls[q] : -INFINITY;
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < kChunk; ++q) m = fmaxf(m, ls[q]);
      if (bok)
        for (int j = kChunk; j < n_my; ++j) m = fmaxf(m, lse_partial[base + sidx(j)]);
      float z = 0.f;
      if (bok && m != -INFINITY) {
#pragma unroll
        for (int q = 0; q < kChunk; ++q) z += ls[q] == -INFINITY ? 0.f : __expf(ls[q] - m);
        for (int j = kChunk; j < n_my; ++j) z += __expf(lse_partial[base + sidx(j)] - m);
      }
      if constexpr (kGroups == 1) {
        if ((tid & 15) == 0 && bok && lse_out)
          lse_out[(int64_t)b * n_heads + h] = (m == -INFINITY) ? -INFINITY : m + __logf(z);
      } else if ((tid & 15) == 0) {
        stat_lds[2 * slot] = m;
        stat_lds[2 * slot + 1] = z;
      }
      // one group: weights normalised here; several: sums relative to the group's own max, normalised
      // when the groups meet
      const float inv_z = (m == -INFINITY) ? 0.f : (kGroups == 1 ? 1.f / z : 1.f);
      float acc[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) acc[k] = 0.f;
      auto accumulate = [&](float wgt, const uint4 (&vq)[4]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t wv[4] = {vq[k].x, vq[k].y, vq[k].z, vq[k].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[8 * k + 2 * e] = fmaf(wgt, __uint_as_float(wv[e] << 16), acc[8 * k + 2 * e]);
            acc[8 * k + 2 * e + 1] = fmaf(wgt, __uint_as_float(wv[e] & 0xFFFF0000u), acc[8 * k + 2 * e + 1]);
          }
        }
      };
      if (bok && m != -INFINITY) {
        // an empty split (lse = -inf, zero partial) and an index past the last split get weight 0
#pragma unroll
        for (int q = 0; q < kChunk; ++q) accumulate(ls[q] == -INFINITY ? 0.f : __expf(ls[q] - m) * inv_z, v[q]);
        // further splits, kChunk at a time, every load of a chunk issued before the first multiply-add
        for (int j0 = kChunk; j0 < n_my; j0 += kChunk) {
#pragma unroll
          for (int q = 0; q < kChunk; ++q) {
            const int s = sidx(min(j0 + q, n_my - 1));
            const float l = lse_partial[base + s];
            ls[q] = j0 + q < n_my ? l : -INFINITY;
            const uint4* src = reinterpret_cast<const uint4*>(o_partial + (base + s) * kDc + c0);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[q][k] = src[k];
          }
#pragma unroll
          for (int q = 0; q < kChunk; ++q) accumulate(ls[q] == -INFINITY ? 0.f : __expf(ls[q] - m) * inv_z, v[q]);
        }
      }
      const int row = bl;  // the block row (MFMA column) this thread stages
      if constexpr (kGroups > 1) {
        // the groups of a sequence meet: group g's sums scaled by exp(m_g - M), divided by the total
        // weight; the group-0 slot of each sequence stages it (rows kRows .. 15 of the staging tile
        // feed MFMA columns that are never stored, and columns do not mix)
#pragma unroll
        for (int k = 0; k < 32; ++k) red_lds[slot * kDc + c0 + k] = acc[k];
        __syncthreads();
        if (grp == 0) {
          float mg[kGroups], M = -INFINITY;
#pragma unroll
          for (int g = 0; g < kGroups; ++g) M = fmaxf(M, mg[g] = stat_lds[2 * (slot + g)]);
          float wg[kGroups], Z = 0.f;
#pragma unroll
          for (int g = 0; g < kGroups; ++g) {
            wg[g] = mg[g] == -INFINITY ? 0.f : __expf(mg[g] - M);
            Z += wg[g] * stat_lds[2 * (slot + g) + 1];
          }
          const float iz = M == -INFINITY ? 0.f : 1.f / Z;
#pragma unroll
          for (int k = 0; k < 32; ++k) {
            float t = 0.f;
#pragma unroll
            for (int g = 0; g < kGroups; ++g) t = fmaf(wg[g], red_lds[(slot + g) * kDc + c0 + k], t);
            acc[k] = t * iz;
          }
          if ((tid & 15) == 0 && b < batch && lse_out)
            lse_out[(int64_t)b * n_heads + h] = (M == -INFINITY) ? -INFINITY : M + __logf(Z);
        }
      }
      char* hrow = hi_lds + row * kPitch + c0 * 2;
      char* lrow = lo_lds + row * kPitch + c0 * 2;
      if (kGroups == 1 || grp == 0)
#pragma unroll
      for (int k = 0; k < 32; k += 8) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          hw[e / 2] = pack_bf16x2(acc[k + e], acc[k + e + 1]);
          lw[e / 2] = pack_bf16x2(acc[k + e] - __uint_as_float(hw[e / 2] << 16),
                                  acc[k + e + 1] - __uint_as_float(hw[e / 2] & 0xFFFF0000u));
        }
        *reinterpret_cast<uint4*>(hrow + k * 2) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(lrow + k * 2) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
    }
    __syncthreads();

    // ---- 2. out^T[v, b] for v in [32 wave, 32 wave + 32) (tiles vt) and the block's 16 sequences:
    // A = W_UV rows (registers), B = merged latent (LDS, lane: sequence lane % 16, columns 32 ks + 8 (lane / 16))
    {
      const lds_char* hb = (lds_char*)hi_lds + (lane & 15) * kPitch + 16 * (lane >> 4);
      const lds_char* lb = (lds_char*)lo_lds + (lane & 15) * kPitch + 16 * (lane >> 4);
      f32x4 acc[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int ks = 0; ks < kDc / 32; ++ks) {
        const bf16x8 bh = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(hb + 64 * ks);
        const bf16x8 bq = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(lb + 64 * ks);
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
          acc[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[vt][ks], bh, acc[vt], 0, 0, 0);
          acc[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[vt][ks], bq, acc[vt], 0, 0, 0);
        }
      }
      // D of tile vt: lane holds sequence b0 + lane % 16 and output dims 32 wave + 16 vt + 4 (lane / 16) + (0..3)
      const int b = b0 + (lane & 15);
      if ((lane & 15) < kRows && b < batch) {
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
          uint16_t* dst = out + ((int64_t)b * n_heads + h) * kDv + 32 * wave + 16 * vt + 4 * (lane >> 4);
          *reinterpret_cast<uint2*>(dst) =
              make_uint2(pack_bf16x2(acc[vt][0], acc[vt][1]), pack_bf16x2(acc[vt][2], acc[vt][3]));
        }
      }
    }
    __syncthreads();  // the next block rewrites the merged rows
  };

  // First block: its partials go out first, W_UV behind them, so the merge runs while W_UV arrives.
  load_first_chunk(blk_begin, ls, v);
  load_wuv();
  for (int blk = blk_begin; blk < blk_end; ++blk) {
    if (blk > blk_begin) {
      if constexpr (kPrefetch) {
#pragma unroll
        for (int q = 0; q < kChunk; ++q) {
          ls[q] = ls_next[q];
#pragma unroll
          for (int k = 0; k < 4; ++k) v[q][k] = v_next[q][k];
        }
      } else {
        load_first_chunk(blk, ls, v);
      }
    }
    if constexpr (kPrefetch) {
      if (blk + 1 < blk_end) load_first_chunk(blk + 1, ls_next, v_next);  // in flight during this block
    }
    process_block(blk);
  }
}

hipError_t launch_combine(int batch, int n_heads, int num_splits, const uint16_t* o_partial,
                          const float* lse_partial, const uint16_t* w_uv, uint16_t* out, float* lse_out,
                          hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  // up to 4 sequences with 16 splits or more: four thread groups per sequence, one block
  if (batch <= kRowsPerWg / 4 && num_splits >= 16) {
    // chunks of 4 splits per group: with 8 the registers of the group merge spill
    hipLaunchKernelGGL((combine_mfma_kernel<4, 4>), dim3(n_heads, 1), dim3(256), 0, stream, batch, n_heads, num_splits,
                       1, o_partial, lse_partial, w_uv, out, lse_out);
    return hipGetLastError();
  }
  // 16-sequence blocks per work-group: one for small batches; with many rows (prefill) enough that
  // about 512 work-groups each load their W_UV rows once
  const int64_t nblk = (batch + kRowsPerWg - 1) / kRowsPerWg;
  const int64_t bpw = std::max<int64_t>(1, (nblk * n_heads + 511) / 512);
  const int64_t yb = (nblk + bpw - 1) / bpw;
  if (yb > 65535) return hipErrorInvalidValue;
#define MLA_LAUNCH_COMBINE(C_)                                                                                      \
  hipLaunchKernelGGL((combine_mfma_kernel<C_, 1>), dim3(n_heads, (unsigned)yb), dim3(256), 0, stream, batch, n_heads, \
                     num_splits, (int)bpw, o_partial, lse_partial, w_uv, out, lse_out)
  if (num_splits <= 1)
    MLA_LAUNCH_COMBINE(1);
  else if (num_splits == 2)
    MLA_LAUNCH_COMBINE(2);
  else if (num_splits <= 4)
    MLA_LAUNCH_COMBINE(4);
  else
    MLA_LAUNCH_COMBINE(8);
#undef MLA_LAUNCH_COMBINE
  return hipGetLastError();
}

}  // namespace mla
