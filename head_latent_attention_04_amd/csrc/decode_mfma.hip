// Split-KV absorbed-MLA attention over the latent cache with bf16 MFMA, heads as the MFMA N dimension.
//
// Math ("论文复现工坊 No.4", sections 2 and 4; "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA的數學原理"
// and "MLA與ROPE的融合"): for every head h and cached token t,
//   s[t, h] = scale * ([q_abs | q_R][h] . [c_t | kR_t])     (one 576-wide dot product: the score of the
//                                                            concatenated parts is the sum of the parts)
//   o_lat[h] = sum_t softmax_t(s[., h]) c_t                   (c_t serves as both key and value latent)
//
// Work decomposition: one work-group of four waves per (query row, split, group of up to 128 heads).
//   * The split's cache rows stream HBM -> LDS with buffer_load ... lds in 32-token stages (36 KB),
//     four stage buffers deep: three stages are in flight while one is consumed. A stage is 36 tiles
//     of 8 rows x 128 bytes and one wave instruction moves one tile, i.e. eight whole 128-byte lines.
//     Rows past the sequence end are fetched from row 0 of the block instead, so no stale value
//     reaches the MFMAs.
//   * Scores: wave w owns head tile w (32 heads) and computes S^T[token, head] = K_tile (A, from LDS)
//     x Q^T (B, in registers) with v_mfma_f32_32x32x16_bf16 over the 576-wide row. The accumulator
//     layout gives every lane one head and 16 tokens, so the softmax needs one cross-lane exchange
//     (lanes l and l^32 hold the same head). The weights go to LDS as P[head][token] in bf16.
//   * Latent reduction: wave w owns latent columns [128 w, 128 w + 128) of O^T[d, head] for every head
//     of the group: A = C^T (ds_read_b64_tr_b16 from the stage), B = P^T (LDS). Splitting this product
//     by columns rather than by heads reads each stage's transposed tile once instead of once per
//     head tile (transposed reads run at half the LDS rate of plain 16-byte reads).
//   * Online softmax against a reference max taken from the first scored stage; weights stay
//     below 2^64 and a split whose scores climb further falls back to an exact recomputation, so
//     the accumulators are never rescaled in the loop.
//   * The split's normalised latent partial (bf16) is staged in LDS and written as whole 1 KB rows,
//     its log-sum-exp (fp32) beside it; a separate kernel merges splits.
#include <type_traits>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 4;                           // waves per work-group
constexpr int kStageTok = 32;                       // tokens per pipeline stage
constexpr int kStageBytes = kStageTok * kRowBytes;  // 36864
constexpr int kStages = 4;                          // stage buffers in LDS
constexpr int kBands = kRowBytes / 128;             // 9 bands of 128 bytes per cache row
constexpr int kGroupBytes = kBands * 1024;          // 8 rows x 9 bands = 9216
constexpr int kPHeadBytes = kStageTok * 2;          // one head's 32 bf16 weights
constexpr int kOutPitch = kDc * 2 + 16;             // staged output row (bytes)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxExcess = 64.0f;                 // log2 units: softmax weights stay <= 2^64

// LDS stage layout. Token row r (0..31) is in row group g = r / 8 at r8 = r % 8; its 16-byte chunk c
// (0..71) is in band c / 8. Tile (g, band) is 1 KB:
//   offset(r, c) = (9 g + c / 8) * 1024 + 128 r8 + 16 ((c % 8) ^ swz(r)),
//   swz(r) = rot(r8) ^ 2 (g % 2),  rot(x) = ((x & 3) << 1) | (x >> 2)   (a bijection of 0..7).
// Reads that fall in the same LDS cycle then hit distinct banks: the score operand (rows r..r+7 or
// r..r+15 at one chunk), the transposed value operand (4 consecutive rows x 2 adjacent chunks in a
// 16-lane group, two such groups on adjacent chunk pairs) and the 8-row copy itself (contiguous).
__device__ __forceinline__ int rot3(int x) { return ((x & 3) << 1) | (x >> 2); }
__device__ __forceinline__ int row_swz(int r) { return rot3(r & 7) ^ (2 * ((r >> 3) & 1)); }

// P layout: head h's 32 weights at h * 64, its 8-token slot s at 16 (s ^ p_swz(h)). With this swizzle
// both the operand reads (16 bytes per lane, lanes (h, half) reading slot 2 ksp + half) and the
// writes (16 bytes per lane, lanes (h, half) writing slots 2 half and 2 half + 1) are free of LDS bank
// conflicts on gfx950 (checked with the SQ_LDS_BANK_CONFLICT counter on kernels that issue exactly
// these accesses; an earlier swizzle, ((h >> 1) ^ (h >> 3)) & 3, was 2-way conflicted on the reads).
__device__ __forceinline__ int p_swz(int h) { return (h ^ (h >> 2)) & 3; }

// Lanes l and l ^ 32 hold the low and high 8 bytes of four 16-byte chunks: x[k] (k = 0..3) the halves
// of chunks 0 and 1 (x[0], x[1] chunk 0; x[2], x[3] chunk 1) and x[k + 4] those of chunks 2 and 3. After
// the exchange the low lane holds whole chunks 0 (c[0]) and 1 (c[1]), the high lane whole chunks 2 and
// 3: v_permlane32_swap hands the low lane the high lane's first operand and the high lane the low
// lane's second operand.
__device__ __forceinline__ void pair_chunks(const uint32_t (&x)[8], u32x4 (&c)[2]) {
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(x[k], x[k + 4], false, false);
    lo[k] = r[0];
    hi[k] = r[1];
  }
  c[0] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  c[1] = u32x4{lo[2], lo[3], hi[2], hi[3]};
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
// The table is read through the constant address space so the load is a scalar one (counted by
// lgkmcnt): a vector load would make its wait also drain the stage copies in flight.
__device__ __forceinline__ const uint16_t* block_ptr(const CacheView& c, int seq, int blk) {
  const __attribute__((address_space(4))) int32_t* tab = (const __attribute__((address_space(4))) int32_t*)c.table;
  int phys32 = c.table ? tab[(int64_t)seq * c.max_blocks + blk] : 0;
  phys32 = __builtin_amdgcn_readfirstlane(phys32);
  const int64_t phys = c.table ? (int64_t)phys32 : (int64_t)seq * c.max_blocks + blk;
  return c.data + phys * (int64_t)(kBlock * kRow);
}

// Start the HBM -> LDS copy of one 32-token stage (half `half` of a 64-token block). Wave w copies row
// group w (rows 8w..8w+7), one 1 KB tile per band: lane l fetches row 8w + l/8 at chunk
// 8 band + ((l % 8) ^ swz(row)), which lands at tile offset 16 l = 128 r8 + 16 slot. Rows >= valid
// are fetched from row 0 of the block. The copy is issued from inline asm so the compiler does not
// make later LDS reads wait for it (it would insert vmcnt(0) before reads of the other stages);
// completion is awaited explicitly with wait_vmcnt before the barrier that publishes the stage. M0
// holds the LDS destination; no compiler-generated code in this kernel uses M0.
struct StageCopy {
  i32x4 rsrc;       // buffer descriptor of the block
  uint32_t voff;    // per-lane byte offset in the block
  uint32_t m0base;  // LDS address of this wave's row group
  uint32_t sbase;   // byte offset of the half block
};

__device__ __forceinline__ StageCopy stage_copy(const uint16_t* src_blk, int half, uint32_t lds_stage, int valid,
                                                int wave, int lane) {
  StageCopy c;
  const uint64_t a = reinterpret_cast<uint64_t>(src_blk);
  c.rsrc.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  c.rsrc.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  c.rsrc.z = kBlock * kRowBytes;                                        // bytes addressable: the block
  c.rsrc.w = 0x00020000;
  const int row = 8 * wave + (lane >> 3);
  const int chunk = (lane & 7) ^ row_swz(row);
  c.voff = (uint32_t)((row < valid ? row : 0) * kRowBytes + chunk * 16);
  c.m0base = __builtin_amdgcn_readfirstlane(lds_stage + wave * kGroupBytes);
  c.sbase = __builtin_amdgcn_readfirstlane(half * kStageBytes);
  return c;
}

// One wave instruction of a stage copy: the tile of `band`. kNt: the rows are read by this work-group
// only (decode with one head group), so the load carries the non-temporal hint and the stream does not
// displace reused lines (queries, block table) from the caches; the prefill's rows are read by many
// work-groups and keep the default policy.
template <bool kNt>
__device__ __forceinline__ void stage_copy_band(const StageCopy& c, int band) {
  const uint32_t soff = c.sbase + band * 128;
  const uint32_t m0 = c.m0base + band * 1024;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (kNt)
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen nt lds" ::"v"(c.voff), "s"(c.rsrc),
                 "s"(m0), "s"(soff)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(c.voff), "s"(c.rsrc), "s"(m0),
                 "s"(soff)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

template <bool kNt>
__device__ __forceinline__ void issue_stage(const uint16_t* src_blk, int half, uint32_t lds_stage, int valid, int wave,
                                            int lane) {
  const StageCopy c = stage_copy(src_blk, half, lds_stage, valid, wave, lane);
#pragma unroll
  for (int band = 0; band < kBands; ++band) stage_copy_band<kNt>(c, band);
}

// for (I = B; I < E; ++I) f(I) with I a compile-time constant in every call: the register arrays the
// body indexes (queries, accumulators, operands) stay in registers whatever the unroller decides.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
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

template <bool kOperandOrder>
__device__ __forceinline__ float q_elem(const uint16_t* __restrict__ q, int tiles, int n_heads, int row, int h, int d) {
  if constexpr (kOperandOrder) return bf16_to_f32(q[q_perm_offset(row, tiles, h, d)]);
  return bf16_to_f32(q[((int64_t)row * n_heads + h) * kRow + d]);
}

// Exact two-pass fallback for one head over tokens [t0, t1): pass 1 finds the true max, pass 2
// accumulates exp2(s - max) c_t in fp32. Each lane holds latent columns lane + 64k. Reads the cache
// rows from global memory; only used for a head whose scores outgrew the fast path's fixed
// reference max.
template <bool kOperandOrder>
__device__ __forceinline__ void exact_head_fallback(const CacheView& cache, int b, int qrow, int t0, int t1,
                                                    int n_heads, int h, const uint16_t* __restrict__ q_abs,
                                                    float scale_log2, int num_splits, int s,
                                                    uint16_t* __restrict__ o_partial, float* __restrict__ lse_partial,
                                                    int lane) {
  const int tiles = q_tiles(n_heads);
  float qv[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) qv[k] = q_elem<kOperandOrder>(q_abs, tiles, n_heads, qrow, h, lane + 64 * k);
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
  const int64_t prow = ((int64_t)qrow * n_heads + h) * num_splits + s;
#pragma unroll
  for (int k = 0; k < 8; ++k) o_partial[prow * kDc + lane + 64 * k] = f32_to_bf16(acc[k] / l);
  if (lane == 0) lse_partial[prow] = (m + __log2f(l)) * kLn2;
}

}  // namespace

template <int HT>
constexpr int kPBytesOf = HT * 32 * kPHeadBytes;  // weights P of one stage

// The work of one attention work-group (blockIdx.x: its logical block). HT: head tiles of 32 per
// work-group (1..4); kOperandOrder: layout of q_abs (see mla_internal.h); kNt: the cache rows are
// read once (stage_copy_band). smem_raw: the stage buffers (kStages * kStageBytes, 1 KB aligned);
// p_raw: P of two stages (2 * kPBytesOf<HT>).
template <int HT, bool kOperandOrder, bool kNt>
__device__ __forceinline__ void attend_tile(const CacheView& cache, int n_heads, int n_groups,
                                            const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q_lens,
                                            int batch, const uint16_t* __restrict__ q_abs, float scale_log2,
                                            int split_tokens, int num_splits, uint16_t* __restrict__ o_partial,
                                            float* __restrict__ lse_partial, char* smem_raw, char* p_raw) {
  constexpr int kPBytes = kPBytesOf<HT>;
  lds_char* lds = (lds_char*)smem_raw;
  lds_char* pl = (lds_char*)p_raw;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kh = lane >> 5;
  const int n = lane & 31;
  int w = logical_block(blockIdx.x, gridDim.x);
  const int hg = w % n_groups;
  w /= n_groups;
  const int s = w % num_splits;
  const int qrow = w / num_splits;  // query row: a sequence (decode) or a query token (prefill)

  // Decode: row qrow is sequence qrow and sees its seq_len tokens. Prefill: row j is query token j of
  // sequence b (cu_q_lens[b] <= j < cu_q_lens[b+1]) at position p = L_b - q_len_b + (j - cu_q_lens[b])
  // and sees tokens 0..p (masked self-attention).
  int b = qrow, L;
  if (cu_q_lens == nullptr) {
    L = seq_lens[b];
  } else {
    int lo = 0, hi = batch - 1;  // last b with cu_q_lens[b] <= qrow
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu_q_lens[mid] <= qrow) lo = mid; else hi = mid - 1;
    }
    b = lo;
    L = seq_lens[b] - (cu_q_lens[b + 1] - cu_q_lens[b]) + (qrow - cu_q_lens[b]) + 1;
  }
  b = __builtin_amdgcn_readfirstlane(b);
  L = __builtin_amdgcn_readfirstlane(L);
  const int tiles_total = q_tiles(n_heads);
  const int tiles_here = min(HT, tiles_total - 4 * hg);  // head tiles of this group (wave-uniform)
  const int h0 = 128 * hg;                               // first head of the group
  const bool qk_wave = wave < tiles_here;                // this wave owns head tile `wave`
  const int head = h0 + 32 * wave + n;                   // the lane's scored head
  const bool hok = qk_wave && head < n_heads;
  const int t0 = s * split_tokens;
  const int t1 = min(L, t0 + split_tokens);

  if (t1 <= t0) {  // empty split: zero partial, lse = -inf
    for (int i = threadIdx.x; i < 32 * HT * (kDc / 8); i += kWaves * 64) {
      const int h = h0 + i / (kDc / 8);
      if (h < n_heads)
        reinterpret_cast<uint4*>(o_partial + (((int64_t)qrow * n_heads + h) * num_splits + s) * kDc)[i % (kDc / 8)] =
            make_uint4(0, 0, 0, 0);
    }
    if (threadIdx.x < 32 * HT && h0 + (int)threadIdx.x < n_heads)
      lse_partial[((int64_t)qrow * n_heads + h0 + threadIdx.x) * num_splits + s] = -INFINITY;
    return;
  }

  // Q^T (B operand of the score MFMA): lane holds head tile `wave`, head n, dims 16 ks + 8 kh .. +7.
  // Waves without a head tile load a valid tile and never use it.
  bf16x8 qreg[36];
  {
    const int tile = min(4 * hg + wave, tiles_total - 1);
    if constexpr (kOperandOrder) {
      const uint4* src = reinterpret_cast<const uint4*>(q_abs + ((int64_t)qrow * tiles_total + tile) * kQTileElems) + lane;
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, src[64 * ks]);
    } else {
      const int hq = min(32 * tile + n, n_heads - 1);
      const uint4* src = reinterpret_cast<const uint4*>(q_abs + ((int64_t)qrow * n_heads + hq) * kRow + 8 * kh);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, src[2 * ks]);
    }
  }

  // stage k covers tokens t0 + 32k .. +31: half (k & 1) of block blk0 + k/2 (t0 is block aligned)
  const int nstages = (t1 - t0 + kStageTok - 1) / kStageTok;
  const int blk0 = t0 / kBlock;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  // Stage 0 goes out right behind the query loads. The empty asm below reads the last query
  // register, so the compiler waits for every load here (the query, and stage 0 with it, which the
  // first step needs anyway) and knows the query is resident inside the loop; otherwise it would
  // guard each score MFMA with a wait that also drains the copies in flight. Stage 1 follows.
  issue_stage<kNt>(block_ptr(cache, b, blk0), 0, lds0, min(kStageTok, t1 - t0), wave, lane);
  asm volatile("" ::"v"(qreg[35]));
  if (nstages > 1)
    issue_stage<kNt>(block_ptr(cache, b, blk0), 1, lds0 + kStageBytes, min(kStageTok, t1 - t0 - kStageTok), wave,
                     lane);

  // Score operand: lane reads token row n at chunk 2 ks + kh, i.e. band ks/4 and slot
  // (2 (ks%4) + kh) ^ swz(n) = 2 (ks%4) ^ (kh ^ swz(n)): one per-lane base per ks % 4.
  uint32_t qk_base[4];
  {
    const int x = kh ^ row_swz(n);
#pragma unroll
    for (int m = 0; m < 4; ++m) qk_base[m] = (n >> 3) * kGroupBytes + (n & 7) * 128 + 16 * ((2 * m) ^ x);
  }
  // Transposed value operand (32 latent columns x 16 tokens per MFMA): in 16-lane group g, lane r
  // supplies token 8 (g >> 1) + r/4 (+4 for the second read) of the k step and latent column
  // 128 wave + 32 dt + 16 (g & 1) + 4 (r % 4), i.e. band 2 wave + dt/2 at chunk position
  // 4 (dt & 1) + 2 (g & 1) + (r/2) % 2, byte 8 (r % 2). One per-lane base per (dt parity, read).
  uint32_t pv_base[2][2];
  {
    const int g16 = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int tok = 8 * (g16 >> 1) + (r16 >> 2) + 4 * rd;
        const int cpos = 4 * p + 2 * (g16 & 1) + ((r16 >> 1) & 1);
        pv_base[p][rd] = (tok >> 3) * kGroupBytes + 2 * wave * 1024 + (tok & 7) * 128 + 16 * (cpos ^ row_swz(tok)) +
                         8 * (r16 & 1);
      }
  }
  // Weight operand P^T (16 tokens x 32 heads): lane reads head n of the tile, tokens 16 ksp + 8 kh .. +7.
  uint32_t pb_base[2];
#pragma unroll
  for (int ksp = 0; ksp < 2; ++ksp) pb_base[ksp] = n * kPHeadBytes + 16 * ((2 * ksp + kh) ^ p_swz(n));
  const int hl = 32 * wave + n;  // the lane's scored head within the group

  // Online softmax against a reference max m_ref (log2 units) fixed by the first scored stage.
  // Weights are exp2(s - m_ref) <= 2^kMaxExcess, so the accumulators are never rescaled in the loop.
  // A head whose later scores exceed m_ref + kMaxExcess is flagged; its column of the accumulators
  // is left alone (the MFMA keeps columns apart) and the head is recomputed by the exact fallback
  // after the split's other heads are written (in practice never taken).
  float m_ref = -INFINITY;
  float lsum = 0.f;
  bool overflow = false;
  f32x16 o[4 * HT];  // O^T tiles: latent columns 128 wave + 32 dt, head tile ht -> o[dt * HT + ht]
#pragma unroll
  for (int i = 0; i < 4 * HT; ++i) o[i] = f32x16{};

  // ---- latent reduction of one stage as 8 HT MFMAs, i -> (ksp = i / (4 HT), dt = (i / HT) % 4,
  // ht = i % HT). P^T of k step 0 is loaded by pv_begin; the register of head tile ht is reloaded
  // with k step 1 right after its last k step 0 use (i = 3 HT + ht). The transposed C^T tile of each
  // (ksp, dt) group is loaded one group ahead.
  bf16x8 pb[HT];
  i16x4 tlo, thi;
  bf16x8 ta;
  auto tr_load = [&](const lds_char* stp, int g) {  // g = 4 ksp + dt
    const int off = (g >> 2) * 2 * kGroupBytes + ((g & 3) >> 1) * 1024;
    tlo = lds_tr16(stp + pv_base[g & 1][0] + off);
    thi = lds_tr16(stp + pv_base[g & 1][1] + off);
  };
  auto pv_begin = [&](const lds_char* stp, const lds_char* pp) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) pb[ht] = lds_b128(pp + pb_base[0] + ht * 32 * kPHeadBytes);
    tr_load(stp, 0);
  };
  auto pv_mfma = [&](const lds_char* stp, const lds_char* pp, int i) {
    const int ksp = i / (4 * HT), dt = (i / HT) % 4, ht = i % HT;
    if (ht == 0) {
      ta = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tlo, thi, 0, 1, 2, 3, 4, 5, 6, 7));
      if (i / HT + 1 < 8) tr_load(stp, i / HT + 1);
    }
    o[dt * HT + ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, pb[ht], o[dt * HT + ht], 0, 0, 0);
    if (ksp == 0 && dt == 3) pb[ht] = lds_b128(pp + pb_base[1] + ht * 32 * kPHeadBytes);
  };
  auto pv_all = [&](const lds_char* stp, const lds_char* pp) {
    pv_begin(stp, pp);
#pragma unroll
    for (int i = 0; i < 8 * HT; ++i) pv_mfma(stp, pp, i);
  };

  // The loop is software-pipelined by one stage: step k scores stage k and, interleaved with those
  // MFMAs and with the softmax that follows them, reduces stage k-1 with the weights P(k-1) written
  // at the end of step k-1 (P has two buffers, so one barrier per step suffices). Step 0 has no
  // previous stage and runs a copy of the body without the reduction (kReduce false). Step k also
  // copies stage k+2 into the buffer of stage k-2, one instruction every fourth score MFMA, so no
  // wave stalls on a burst of copy instructions.
  constexpr int kScorePv = 4 * HT;            // reduction MFMAs interleaved with the scores
  constexpr int kSoftPv = 8 * HT - kScorePv;  // the rest, spread over the softmax
  uint32_t pw[8];
  auto step = [&](const int k, auto REDUCE) {
    constexpr bool kReduce = decltype(REDUCE)::value;
    // stage k has landed once only the stage issued after it (if any) is outstanding
    if (k + 1 < nstages)
      wait_vmcnt<kBands>();
    else
      wait_vmcnt<0>();
    wg_barrier();  // publishes stage k and P(k-1); every wave is done with stage k-2 and P(k-2)
    const lds_char* st = lds + (k % kStages) * kStageBytes;
    const lds_char* stp = lds + ((k + kStages - 1) % kStages) * kStageBytes;  // stage k-1
    const lds_char* pp = pl + ((k + 1) & 1) * kPBytes;                        // P(k-1)
    const bool copy_next = k + 2 < nstages;
    // descriptor of stage k+2's copy, formed on every step (for a stage past the end it names the
    // split's last stage and is not issued), so it stays wave-uniform, in scalar registers
    const int kn = min(k + 2, nstages - 1);
    const StageCopy cp = stage_copy(block_ptr(cache, b, blk0 + (kn >> 1)), kn & 1, lds0 + (kn % kStages) * kStageBytes,
                                    min(kStageTok, t1 - t0 - kn * kStageTok), wave, lane);

    // every wave runs this body; a wave without a head tile scores a duplicate and drops it
    const int valid = min(kStageTok, t1 - t0 - k * kStageTok);
    if constexpr (kReduce) pv_begin(stp, pp);
    // ---- scores S^T[32 tokens x 32 heads]; half of stage k-1's reduction and the copy interleaved
    f32x16 sacc;
    {
      constexpr int kAhead = 3;  // operand loads issued this many MFMAs ahead
      bf16x8 a_buf[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) a_buf[i] = lds_b128(st + qk_base[i & 3] + (i >> 2) * 1024);
      static_for<0, 36>([&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        const bf16x8 a = a_buf[ks % kAhead];
        constexpr int kn = ks + kAhead;
        if constexpr (kn < 36) a_buf[ks % kAhead] = lds_b128(st + qk_base[kn & 3] + (kn >> 2) * 1024);
        if constexpr (ks == 0)
          score_mfma_first(sacc, a, qreg[0]);
        else
          score_mfma(sacc, a, qreg[ks]);
        if constexpr (kReduce)
          static_for<ks * kScorePv / 36, (ks + 1) * kScorePv / 36>([&](auto I) { pv_mfma(stp, pp, decltype(I)::value); });
        if constexpr ((ks & 3) == 1) {
          if (copy_next) stage_copy_band<kNt>(cp, ks >> 2);
        }
        // keep this order: the scheduler would otherwise hoist operand loads and run out of registers
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    score_mfma_drain(sacc);
    // ---- softmax weights; element j is token 8*(j>>2) + 4*kh + (j&3) of the stage. The other half
    // of stage k-1's reduction runs on the matrix cores meanwhile (12 slots).
    auto pv_slot = [&](auto SLOT) {
      constexpr int slot = decltype(SLOT)::value;
      if constexpr (kReduce)
        static_for<kScorePv + slot * kSoftPv / 12, kScorePv + (slot + 1) * kSoftPv / 12>(
            [&](auto I) { pv_mfma(stp, pp, decltype(I)::value); });
      __builtin_amdgcn_sched_barrier(0);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S11 = std::integral_constant<int, 11>;
    if (valid < kStageTok) {  // only the split's last, partly filled stage needs a mask
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int tk = 8 * (j >> 2) + 4 * kh + (j & 3);
        if (tk >= valid) sacc[j] = -INFINITY;
      }
    }
    pv_slot(S0{});
    float mx = sacc[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sacc[j]);
    pv_slot(S1{});
    mx = pair_max(mx) * scale_log2;  // scale > 0: the max commutes with it
    if (m_ref == -INFINITY) m_ref = mx;
    overflow |= mx > m_ref + kMaxExcess;
    pv_slot(S2{});
    static_for<0, 8>([&](auto JJ) {
      constexpr int j = 2 * decltype(JJ)::value;
      // raw v_exp_f32: weights below 2^-126 flush to zero, which a softmax weight can afford
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[j], scale_log2, -m_ref));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[j + 1], scale_log2, -m_ref));
      lsum += p0 + p1;
      pw[j >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
      asm volatile("" ::"v"(pw[j >> 1]));  // computed here, between the reduction MFMAs, not sunk to its store
      pv_slot(std::integral_constant<int, 3 + (j >> 1)>{});
    });
    pv_slot(S11{});
    if (qk_wave) {  // P(k)[head][tokens 8 q .. 8 q + 7] into the other buffer, whole 16-byte slots:
      // the lane holds tokens 8 q + 4 kh .. +3 as (pw[2q], pw[2q+1]); after the pair exchange lane kh
      // writes slots 2 kh and 2 kh + 1
      u32x4 chunk[2];
      pair_chunks(pw, chunk);
      const int ps = p_swz(n);
      lds_char* pk = pl + (k & 1) * kPBytes;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(pk + hl * kPHeadBytes + 16 * ((2 * kh + t) ^ ps)) =
            chunk[t];
    }
  };
  step(0, std::false_type{});
  for (int k = 1; k < nstages; ++k) step(k, std::true_type{});
  wg_barrier();  // publishes P of the last stage
  pv_all(lds + ((nstages - 1) % kStages) * kStageBytes, pl + ((nstages - 1) & 1) * kPBytes);
  wg_barrier();  // every wave is done with the stages and P
  // explicit wait states before the VALU reads the output accumulators (the count the compiler
  // derives from the instructions in between is not relied on)
#pragma unroll
  for (int i = 0; i < 4 * HT; ++i) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[i]));

  // 1/lsum of every head (negative: the head overflowed and is recomputed below), in P's space
  float* inv_lds = reinterpret_cast<float*>(p_raw);
  if (qk_wave) {
    lsum += __shfl_xor(lsum, 32);
    if (kh == 0) {
      inv_lds[hl] = overflow ? -1.f : 1.f / lsum;
      if (hok && !overflow)
        lse_partial[((int64_t)qrow * n_heads + head) * num_splits + s] = (m_ref + __log2f(lsum)) * kLn2;
    }
  }
  wg_barrier();  // publishes 1/lsum of every head

  // Scale by 1/lsum and stage as bf16 rows: element j of o[dt * HT + ht] is head 32 ht + n, latent
  // column 128 wave + 32 dt + 8 (j >> 2) + 4 kh + (j & 3). The lane pair (l, l ^ 32) trades halves so
  // that every store is a whole 16-byte piece of 8 columns (the 8-byte stores of the halves were 2-way
  // bank conflicted at this pitch; the 16-byte ones are not).
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const float iv = inv_lds[32 * ht + n];
    char* orow = smem_raw + (32 * ht + n) * kOutPitch + 2 * (128 * wave);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x2 v01 = {o[dt * HT + ht][4 * q] * iv, o[dt * HT + ht][4 * q + 1] * iv};
        const f32x2 v23 = {o[dt * HT + ht][4 * q + 2] * iv, o[dt * HT + ht][4 * q + 3] * iv};
        w[2 * q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v01, bf16x2));
        w[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, bf16x2));
      }
      u32x4 chunk[2];
      pair_chunks(w, chunk);
#pragma unroll
      for (int t = 0; t < 2; ++t) *reinterpret_cast<u32x4*>(orow + 2 * (32 * dt + 8 * (2 * kh + t))) = chunk[t];
    }
  }
  wg_barrier();
  // whole 1 KB rows out: wave w writes the group's heads w, w + 4, ... The stores are nontemporal:
  // the partials are read once, by the combine kernel on other XCDs, so they are not kept in this
  // XCD's L2 (which would otherwise write them back when the kernel ends).
#pragma unroll 4
  for (int i = 0; i < 8 * HT; ++i) {
    const int r = 4 * i + wave;
    if (r < 32 * tiles_here && h0 + r < n_heads && inv_lds[r] >= 0.f) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem_raw + r * kOutPitch + 16 * lane);
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4*>(o_partial + (((int64_t)qrow * n_heads + h0 + r) * num_splits + s) * kDc) + lane);
    }
  }
  // heads whose scores outgrew the reference max: exact recomputation by the wave that scored them
  if (qk_wave) {
    uint64_t todo = __ballot(overflow && kh == 0 && hok);
    while (todo) {
      const int hh = __builtin_ctzll(todo);
      todo &= todo - 1;
      exact_head_fallback<kOperandOrder>(cache, b, qrow, t0, t1, n_heads, h0 + 32 * wave + hh, q_abs, scale_log2,
                                         num_splits, s, o_partial, lse_partial, lane);
    }
  }
}

template <int HT, bool kOperandOrder, bool kNt>
__global__ void __launch_bounds__(kWaves * 64, 1)
decode_mfma_kernel(CacheView cache, int n_heads, int n_groups, const int32_t* __restrict__ seq_lens,
                   const int32_t* __restrict__ cu_q_lens, int batch, const uint16_t* __restrict__ q_abs,
                   float scale_log2, int split_tokens, int num_splits, uint16_t* __restrict__ o_partial,
                   float* __restrict__ lse_partial) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kStages * kStageBytes];
  __shared__ __attribute__((aligned(16))) char p_raw[2 * kPBytesOf<HT>];
  attend_tile<HT, kOperandOrder, kNt>(cache, n_heads, n_groups, seq_lens, cu_q_lens, batch, q_abs, scale_log2,
                                      split_tokens, num_splits, o_partial, lse_partial, smem_raw, p_raw);
}


template <int HT, bool kOperandOrder>
static hipError_t launch_ht(const CacheView& cache, int rows, int n_heads, const int32_t* seq_lens,
                            const int32_t* cu_q_lens, int batch, const uint16_t* q_abs, float scale, int split_tokens,
                            int num_splits, uint16_t* o_partial, float* lse_partial, hipStream_t stream) {
  const int groups = (q_tiles(n_heads) + 3) / 4;
  const int64_t nwg = (int64_t)groups * num_splits * rows;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  // decode with one head group reads every cache row once; prefill rows and several head groups re-read
  if (cu_q_lens == nullptr && groups == 1)
    hipLaunchKernelGGL((decode_mfma_kernel<HT, kOperandOrder, true>), dim3((unsigned)nwg), dim3(kWaves * 64), 0, stream,
                       cache, n_heads, groups, seq_lens, cu_q_lens, batch, q_abs, scale * kLog2e, split_tokens,
                       num_splits, o_partial, lse_partial);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<HT, kOperandOrder, false>), dim3((unsigned)nwg), dim3(kWaves * 64), 0,
                       stream, cache, n_heads, groups, seq_lens, cu_q_lens, batch, q_abs, scale * kLog2e, split_tokens,
                       num_splits, o_partial, lse_partial);
  return hipGetLastError();
}

template <bool kOperandOrder>
static hipError_t launch_layout(const CacheView& cache, int rows, int n_heads, const int32_t* seq_lens,
                                const int32_t* cu_q_lens, int batch, const uint16_t* q_abs, float scale,
                                int split_tokens, int num_splits, uint16_t* o_partial, float* lse_partial,
                                hipStream_t stream) {
#define MLA_LAUNCH(HT_)                                                                                       \
  return launch_ht<HT_, kOperandOrder>(cache, rows, n_heads, seq_lens, cu_q_lens, batch, q_abs, scale,         \
                                       split_tokens, num_splits, o_partial, lse_partial, stream)
  const int tiles = q_tiles(n_heads);
  if (tiles >= 4) MLA_LAUNCH(4);
  if (tiles == 3) MLA_LAUNCH(3);
  if (tiles == 2) MLA_LAUNCH(2);
  MLA_LAUNCH(1);
#undef MLA_LAUNCH
}

hipError_t launch_attention(const CacheView& cache, int rows, int n_heads, const int32_t* seq_lens,
                            const int32_t* cu_q_lens, int batch, const uint16_t* q_abs, bool q_operand_order,
                            float scale, int split_tokens, int num_splits, uint16_t* o_partial, float* lse_partial,
                            hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (q_operand_order)
    return launch_layout<true>(cache, rows, n_heads, seq_lens, cu_q_lens, batch, q_abs, scale, split_tokens,
                               num_splits, o_partial, lse_partial, stream);
  return launch_layout<false>(cache, rows, n_heads, seq_lens, cu_q_lens, batch, q_abs, scale, split_tokens,
                              num_splits, o_partial, lse_partial, stream);
}

}  // namespace mla
