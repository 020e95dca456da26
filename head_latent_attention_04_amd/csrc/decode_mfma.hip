// Split-KV absorbed-MLA attention over the latent cache with bf16 MFMA, heads as the MFMA N dimension.
//
// Math ("论文复现工坊 No.4", sections 2 and 4; "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA的數學原理"
// and "MLA與ROPE的融合"): for every head h and cached token t,
//   s[t, h] = scale * ([q_abs | q_R][h] . [c_t | kR_t])     (one 576-wide dot product: the score of the
//                                                            concatenated parts is the sum of the parts)
//   o_lat[h] = sum_t softmax_t(s[., h]) c_t                   (c_t serves as both key and value latent)
//
// Work decomposition (one work-group per (sequence, split, group of up to 128 heads)):
//   * The split's cache blocks (64 tokens x 1152 B each) stream HBM -> LDS with global_load_lds
//     dwordx4, double buffered: block i+1 is in flight while block i is consumed. Rows past the
//     sequence end are fetched from row 0 of the block instead, so no stale value reaches the MFMAs.
//   * Each wave owns 32 heads. Per 32-token sub-tile it computes S^T[token, head] =
//     K_tile (A, from LDS) x Q^T (B, in registers) with v_mfma_f32_32x32x16_bf16 over the 576-wide row.
//     The accumulator layout gives every lane one head and 16 tokens, so the softmax needs one
//     cross-lane exchange (lanes l and l^32 hold the same head).
//   * P^T goes straight from the score accumulators into the B operand of
//     O^T[d, head] += C^T (A, ds_read_b64_tr_b16 from the same LDS tile) x P^T, all 512 latent columns
//     accumulated in 16 32x32 fp32 tiles per wave (256 accumulator registers).
//   * Online softmax against a reference max taken from the first scored sub-tile; weights stay
//     below 2^64 and a split whose scores climb further restarts with a raised reference, so the
//     accumulators are never rescaled in the loop.
//   * The split writes its normalised latent partial and log-sum-exp; a separate kernel merges splits.
//
// LDS tile layout: chunk-major (see lds_off below), so that one DMA instruction moves one 16-byte
// column of all 64 rows and both operand read patterns are free of bank conflicts.
#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

constexpr int kTileTok = 64;
constexpr int kTileBytes = kTileTok * kRowBytes;  // 73728
constexpr int kUnits = kTileBytes / 1024;         // 72 wave-wide 1 KB DMA transfers per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxExcess = 64.0f;               // log2 units: softmax weights stay <= 2^64

// LDS tile layout, chunk-major: the 16-byte chunk c (of 72) of token row r (of 64) is stored at
//   c * 1024 + (r ^ (4 * (c & 1))) * 16.
// One 1 KB DMA instruction fills one chunk column for all 64 rows. The score operand (32 rows at
// one chunk) reads 512 contiguous bytes; the transposed value operand (4 rows x 2 adjacent chunks)
// hits two 64-byte runs that the row XOR puts in different banks.
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return chunk * 1024 + ((row ^ (4 * (chunk & 1))) << 4);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  if constexpr (N > 63) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  }
}

// Physical block of (seq, logical block), made wave-uniform so the copy's buffer descriptor lives in
// scalar registers.
__device__ __forceinline__ const uint16_t* block_ptr(const CacheView& c, int seq, int blk) {
  int phys32 = c.table ? c.table[(int64_t)seq * c.max_blocks + blk] : 0;
  phys32 = __builtin_amdgcn_readfirstlane(phys32);
  const int64_t phys = c.table ? (int64_t)phys32 : (int64_t)seq * c.max_blocks + blk;
  return c.data + phys * (int64_t)(kBlock * kRow);
}

// Start the HBM -> LDS copy of one 64-token block: buffer_load_dwordx4 ... lds, one chunk column
// (64 rows x 16 bytes) per wave instruction; rows >= valid are taken from row 0 of the block.
// The copy is issued from inline asm so the compiler does not make every later LDS read wait for
// it (it would insert vmcnt(0) before reads of the other buffer); completion is awaited explicitly
// with wait_vmcnt before the barrier that publishes the block. M0 holds the LDS destination; no
// compiler-generated code in this kernel uses M0.
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <int NW>
__device__ __forceinline__ void issue_tile(const uint16_t* src_blk, lds_char* dst, int valid, int wave, int lane) {
  const uint64_t a = reinterpret_cast<uint64_t>(src_blk);
  i32x4 rsrc;
  rsrc.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  rsrc.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  rsrc.z = kTileBytes;                                                // bytes addressable
  rsrc.w = 0x00020000;
  // source row of this lane for even / odd chunk columns
  const int r0 = lane, r1 = lane ^ 4;
  const uint32_t v0 = (r0 < valid ? r0 : 0) * kRowBytes;
  const uint32_t v1 = (r1 < valid ? r1 : 0) * kRowBytes;
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst + wave * 1024);
#pragma unroll
  for (int j = 0; j < kUnits / NW; ++j) {
    // chunk column c = j * NW + wave: global byte offset c*16 in soffset, LDS offset c*1024 in M0
    const int c = j * NW + wave;
    const uint32_t voff = (c & 1) ? v1 : v0;
    const uint32_t soff = __builtin_amdgcn_readfirstlane(c * 16);
    const uint32_t m0 = lds_base + j * NW * 1024;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(rsrc), "s"(m0),
                 "s"(soff)
                 : "memory", "m0");
#pragma clang diagnostic pop
  }
}

// Work-group barrier without the memory fence of __syncthreads(): that fence would also wait for
// the next block's copy (vmcnt 0) and serialise the prefetch. LDS accesses are complete on
// lgkmcnt(0); copies into LDS are waited for explicitly with vmcnt.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 lds_b128(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

__device__ __forceinline__ i16x4 lds_tr16(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

// Score MFMAs accumulate in arch VGPRs (inline asm pins the VGPR form) so that all 256 accumulation
// registers stay free for the 32 x 512 output tile. Back-to-back accumulation into the same
// registers needs no wait states; the VALU reads that follow wait on score_mfma_drain().
__device__ __forceinline__ void score_mfma_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_mfma_drain(f32x16& acc) {
  // more than the wait states a 16-pass XDL result needs before a VALU may read or overwrite it
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

// max of a value over the lane pair (l, l ^ 32), returned to both lanes (v_permlane32_swap, no LDS)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// XCD-aware work order: consecutive logical work items land on the same XCD (work-groups are
// dealt to the 8 XCDs round-robin by linear id), so the splits of one sequence share an L2.
__device__ __forceinline__ int logical_block(int id, int n) {
  const int per = n / 8, rem = n % 8;
  const int xcd = id % 8, k = id / 8;
  return xcd < rem ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
}

// Exact two-pass fallback for one wave's 32 heads over tokens [t0, t1): pass 1 finds the true max,
// pass 2 accumulates exp2(s - max) c_t in fp32. Each lane holds latent columns lane + 64k. Reads the
// cache rows from global memory; only used when the fast path's fixed reference max is exceeded.
__device__ __forceinline__ void exact_split_fallback(const CacheView& cache, int b, int t0, int t1, int n_heads, int h0,
                                                  const uint16_t* __restrict__ q_abs, float scale_log2,
                                                  int num_splits, int s, float* __restrict__ o_partial,
                                                  float* __restrict__ lse_partial, int lane) {
  for (int hh = 0; hh < 32; ++hh) {
    const int h = h0 + hh;
    if (h >= n_heads) break;
    const uint16_t* qa = q_abs + ((int64_t)b * n_heads + h) * kRow;
    float qv[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) qv[k] = bf16_to_f32(qa[lane + 64 * k]);
    float m = -INFINITY;
    for (int t = t0; t < t1; ++t) {
      const uint16_t* row = cache.data + row_offset(cache, b, t);
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < 9; ++k) part = fmaf(qv[k], bf16_to_f32(row[lane + 64 * k]), part);
      for (int x = 32; x > 0; x >>= 1) part += __shfl_xor(part, x);
      m = fmaxf(m, part * scale_log2);
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    for (int t = t0; t < t1; ++t) {
      const uint16_t* row = cache.data + row_offset(cache, b, t);
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < 9; ++k) part = fmaf(qv[k], bf16_to_f32(row[lane + 64 * k]), part);
      for (int x = 32; x > 0; x >>= 1) part += __shfl_xor(part, x);
      const float p = exp2f(part * scale_log2 - m);
      l += p;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(p, bf16_to_f32(row[lane + 64 * k]), acc[k]);
    }
    const int64_t prow = ((int64_t)b * n_heads + h) * num_splits + s;
#pragma unroll
    for (int k = 0; k < 8; ++k) o_partial[prow * kDc + lane + 64 * k] = acc[k] / l;
    if (lane == 0) lse_partial[prow] = (m + __log2f(l)) * kLn2;
  }
}

}  // namespace

template <int NW>
__global__ void __launch_bounds__(NW * 64, 1)
decode_mfma_kernel(CacheView cache, int n_heads, int n_head_groups, const int32_t* __restrict__ seq_lens,
                   const uint16_t* __restrict__ q_abs, float scale_log2, int split_tokens, int num_splits,
                   float* __restrict__ o_partial, float* __restrict__ lse_partial) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * kTileBytes];
  __shared__ int restart_flag;
  lds_char* lds = (lds_char*)smem_raw;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kh = lane >> 5;
  int w = logical_block(blockIdx.x, gridDim.x);
  const int hg = w % n_head_groups;
  w /= n_head_groups;
  const int s = w % num_splits;
  const int b = w / num_splits;

  const int head = hg * (32 * NW) + wave * 32 + (lane & 31);
  const bool hok = head < n_heads;
  const int L = seq_lens[b];
  const int t0 = s * split_tokens;
  const int t1 = min(L, t0 + split_tokens);

  if (t1 <= t0) {  // empty split: zero partial, lse = -inf
    const int h0 = hg * (32 * NW);
    for (int i = threadIdx.x; i < 32 * NW * (kDc / 4); i += NW * 64) {
      const int h = h0 + i / (kDc / 4);
      if (h < n_heads)
        reinterpret_cast<float4*>(o_partial + (((int64_t)b * n_heads + h) * num_splits + s) * kDc)[i % (kDc / 4)] =
            make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (threadIdx.x < 32 * NW && h0 + (int)threadIdx.x < n_heads)
      lse_partial[((int64_t)b * n_heads + h0 + threadIdx.x) * num_splits + s] = -INFINITY;
    return;
  }

  const int ntiles = (t1 - t0 + kTileTok - 1) / kTileTok;
  const int blk0 = t0 / kBlock;
  if (threadIdx.x == 0) restart_flag = 0;
  issue_tile<NW>(block_ptr(cache, b, blk0), lds, min(kTileTok, t1 - t0), wave, lane);

  // Q^T (B operand of the score MFMA): lane holds head `head`, dims 16*ks + 8*kh .. +7.
  bf16x8 qreg[36];
  {
    const uint4* qsrc =
        reinterpret_cast<const uint4*>(q_abs + ((int64_t)b * n_heads + (hok ? head : 0)) * kRow + 8 * kh);
    const uint32_t keep = hok ? 0xFFFFFFFFu : 0u;  // heads past n_heads score with a zero query
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      uint4 v = qsrc[2 * ks];
      v.x &= keep; v.y &= keep; v.z &= keep; v.w &= keep;
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Score operand: lane reads row 32*sub + (lane & 31), chunk 2*ks + kh (parity kh), i.e.
  // (2ks + kh)*1024 + ((32 sub + (lane&31)) ^ 4kh)*16: one per-lane base, ks and sub as immediates
  // (a second base 64 KB up keeps every immediate below 2^16).
  const uint32_t abase = kh * 1024 + (((lane & 31) ^ (4 * kh)) << 4);
  // Transposed value operand: in each 16-lane group g, lane r supplies token
  // 32 sub + 16 ksp + 8 half + 4 kh + r/4 and latent column 32 dblk + 16 (g&1) + 4 (r%4), i.e.
  // chunk 4 dblk + 2 (g&1) + ((r>>1)&1) at byte 8 (r&1); only kh and that chunk parity move the
  // row XOR, so one per-lane base plus immediates covers every read.
  const int r16 = lane & 15;
  const int tpar = (r16 >> 1) & 1;
  const uint32_t tbase = (2 * ((lane >> 4) & 1) + tpar) * 1024 + (((4 * kh) ^ (4 * tpar)) + (r16 >> 2)) * 16 +
                         8 * (r16 & 1);

  // Online softmax against a reference max m_ref (log2 units) fixed by the first scored sub-tile.
  // Weights are exp2(s - m_ref) <= 2^kMaxExcess, so the accumulators are never rescaled in the loop.
  // If a later sub-tile's max exceeds m_ref + kMaxExcess, every wave of the work-group discards its
  // accumulators and recomputes its heads with the exact fallback below (in practice never taken).
  float m_ref = -INFINITY;
  f32x16 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x16{};
  float lsum = 0.f;
  bool overflow = false;
  bool restart = false;
  for (int it = 0; it < ntiles; ++it) {
    const uint32_t bufoff = (it & 1) * kTileBytes;
    const int tok0 = t0 + it * kTileTok;
    const int valid = min(kTileTok, t1 - tok0);
    if (it + 1 < ntiles) {
      issue_tile<NW>(block_ptr(cache, b, blk0 + it + 1), lds + (((it + 1) & 1) * kTileBytes),
                     min(kTileTok, t1 - tok0 - kTileTok), wave, lane);
      wait_vmcnt<kUnits / NW>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();

    for (int sub = 0; sub < 2; ++sub) {
      if (sub * 32 >= valid) break;
      const uint32_t soff = bufoff + sub * 32 * 16;
      // ---- scores S^T[32 tokens x 32 heads]
      f32x16 sacc;
      const lds_char* a_lo = lds + (abase + soff);
      const lds_char* a_hi = lds + (abase + soff + 65536);
      auto a_ld = [&](int ks) { return ks < 32 ? lds_b128(a_lo + ks * 2048) : lds_b128(a_hi + (ks - 32) * 2048); };
      constexpr int kAhead = 4;  // operand loads issued this many MFMAs ahead
      bf16x8 a_buf[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) a_buf[i] = a_ld(i);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        const bf16x8 a = a_buf[ks % kAhead];
        if (ks + kAhead < 36) a_buf[ks % kAhead] = a_ld(ks + kAhead);
        if (ks == 0)
          score_mfma_first(sacc, a, qreg[0]);
        else
          score_mfma(sacc, a, qreg[ks]);
      }
      score_mfma_drain(sacc);
      // ---- softmax weights; element j is token 32*sub + 8*(j>>2) + 4*kh + (j&3)
      if (valid - 32 * sub < 32) {  // only the block's last, partly filled sub-tile needs a mask
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int tk = 32 * sub + 8 * (j >> 2) + 4 * kh + (j & 3);
          if (tk >= valid) sacc[j] = -INFINITY;
        }
      }
      float mx = sacc[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sacc[j]);
      mx = pair_max(mx) * scale_log2;  // scale > 0: the max commutes with it
      if (m_ref == -INFINITY) m_ref = mx;
      overflow |= mx > m_ref + kMaxExcess;
      uint32_t pw[8];
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        // raw v_exp_f32: weights below 2^-126 flush to zero, which a softmax weight can afford
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[j], scale_log2, -m_ref));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[j + 1], scale_log2, -m_ref));
        lsum += p0 + p1;
        pw[j >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
      }
      // ---- O^T[d, head] += C^T[d, token] P^T[token, head]; transposed reads one block ahead
#pragma unroll
      for (int ksp = 0; ksp < 2; ++ksp) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pw[4 * ksp], pw[4 * ksp + 1], pw[4 * ksp + 2],
                                                                  pw[4 * ksp + 3]));
        const lds_char* tb = lds + (tbase + soff + 16 * ksp * 16);
        i16x4 lo = lds_tr16(tb);
        i16x4 hi = lds_tr16(tb + 8 * 16);
#pragma unroll
        for (int dblk = 0; dblk < 16; ++dblk) {
          i16x4 lo_n = lo, hi_n = hi;
          if (dblk + 1 < 16) {
            lo_n = lds_tr16(tb + (dblk + 1) * 4096);
            hi_n = lds_tr16(tb + (dblk + 1) * 4096 + 8 * 16);
          }
          const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb, o[dblk], 0, 0, 0);
          lo = lo_n;
          hi = hi_n;
        }
      }
    }
    if (__any(overflow) && lane == 0) restart_flag = 1;
    wg_barrier();  // every wave is done with this buffer before the next copy into it
    // (the loop runs to its end either way: an early exit here costs the hot loop its registers)
    restart |= restart_flag != 0;
  }

  if (restart) {
    wait_vmcnt<0>();  // no copy may still be landing in LDS when the work-group ends
    exact_split_fallback(cache, b, t0, t1, n_heads, hg * (32 * NW) + wave * 32, q_abs, scale_log2, num_splits, s,
                         o_partial, lse_partial, lane);
    return;
  }

  lsum += __shfl_xor(lsum, 32);
  if (!hok) return;
  const float inv = 1.f / lsum;
  const int64_t prow = ((int64_t)b * n_heads + head) * num_splits + s;
  float* dst = o_partial + prow * kDc;
#pragma unroll
  for (int dblk = 0; dblk < 16; ++dblk) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dblk + 8 * g + 4 * kh;
      *reinterpret_cast<float4*>(dst + d) =
          make_float4(o[dblk][4 * g] * inv, o[dblk][4 * g + 1] * inv, o[dblk][4 * g + 2] * inv, o[dblk][4 * g + 3] * inv);
    }
  }
  if (kh == 0) lse_partial[prow] = (m_ref + __log2f(lsum)) * kLn2;
}

template <int NW>
static hipError_t launch_nw(const CacheView& cache, int batch, int n_heads, const int32_t* seq_lens,
                            const uint16_t* q_abs, float scale, int split_tokens, int num_splits, float* o_partial,
                            float* lse_partial, hipStream_t stream) {
  const int groups = (n_heads + 32 * NW - 1) / (32 * NW);
  const int64_t nwg = (int64_t)groups * num_splits * batch;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_mfma_kernel<NW>, dim3((unsigned)nwg, 1), dim3(NW * 64), 0, stream, cache, n_heads, groups,
                     seq_lens, q_abs, scale * kLog2e, split_tokens, num_splits, o_partial, lse_partial);
  return hipGetLastError();
}

hipError_t launch_decode_attention(const CacheView& cache, int batch, int n_heads, const int32_t* seq_lens,
                                   const uint16_t* q_abs, float scale, int split_tokens, int num_splits,
                                   float* o_partial, float* lse_partial, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (n_heads >= 128)
    return launch_nw<4>(cache, batch, n_heads, seq_lens, q_abs, scale, split_tokens, num_splits, o_partial,
                        lse_partial, stream);
  if (n_heads > 64)
    return launch_nw<3>(cache, batch, n_heads, seq_lens, q_abs, scale, split_tokens, num_splits, o_partial,
                        lse_partial, stream);
  if (n_heads > 32)
    return launch_nw<2>(cache, batch, n_heads, seq_lens, q_abs, scale, split_tokens, num_splits, o_partial,
                        lse_partial, stream);
  return launch_nw<1>(cache, batch, n_heads, seq_lens, q_abs, scale, split_tokens, num_splits, o_partial,
                      lse_partial, stream);
}

}  // namespace mla
