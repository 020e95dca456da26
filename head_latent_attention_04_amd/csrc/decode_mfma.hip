// Split-KV absorbed-MLA attention over the latent cache with bf16 MFMA, heads as the MFMA N dimension.
//
// Math ("论文复现工坊 No.4", sections 2 and 4; "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA的數學原理"
// and "MLA與ROPE的融合"): for every head h and cached token t,
//   s[t, h] = scale * ([q_abs | q_R][h] . [c_t | kR_t])     (one 576-wide dot product: the score of the
//                                                            concatenated parts is the sum of the parts)
//   o_lat[h] = sum_t softmax_t(s[., h]) c_t                   (c_t serves as both key and value latent)
//
// Work decomposition (one work-group per (sequence, split, group of up to 128 heads)):
//   * The split's cache rows stream HBM -> LDS with buffer_load ... lds in 32-token stages (36 KB),
//     four stage buffers deep: three stages are in flight while one is consumed. Rows past the
//     sequence end are fetched from row 0 of the block instead, so no stale value reaches the MFMAs.
//   * Each wave owns 32 heads. Per stage it computes S^T[token, head] = K_tile (A, from LDS) x
//     Q^T (B, in registers) with v_mfma_f32_32x32x16_bf16 over the 576-wide row. The accumulator
//     layout gives every lane one head and 16 tokens, so the softmax needs one cross-lane exchange
//     (lanes l and l^32 hold the same head).
//   * P^T goes straight from the score accumulators into the B operand of
//     O^T[d, head] += C^T (A, ds_read_b64_tr_b16 from the same LDS stage) x P^T, all 512 latent
//     columns accumulated in 16 32x32 fp32 tiles per wave (256 accumulator registers).
//   * Online softmax against a reference max taken from the first scored stage; weights stay
//     below 2^64 and a split whose scores climb further falls back to an exact recomputation, so
//     the accumulators are never rescaled in the loop.
//   * The split writes its normalised latent partial (bf16) and log-sum-exp (fp32); a separate
//     kernel merges splits.
//
// LDS stage layout: chunk-major (see lds_off below), so that one DMA instruction moves two 16-byte
// columns of all 32 rows and both operand read patterns are free of bank conflicts.
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

constexpr int kStageTok = 32;                       // tokens per pipeline stage
constexpr int kStageBytes = kStageTok * kRowBytes;  // 36864
constexpr int kStages = 4;                          // stage buffers in LDS
constexpr int kStageUnits = kStageBytes / 1024;     // 36 wave-wide 1 KB DMA transfers per stage
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxExcess = 64.0f;                 // log2 units: softmax weights stay <= 2^64

// LDS stage layout, chunk-major: the 16-byte chunk c (of 72) of token row r (of 32) is stored at
//   c * 512 + (r ^ (4 * (c & 1))) * 16.
// The score operand (32 rows at one chunk) reads 512 contiguous bytes; the transposed value operand
// (4 rows x 2 adjacent chunks) hits two 64-byte runs that the row XOR puts in different banks.

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

// Start the HBM -> LDS copy of one 32-token stage (half `half` of a 64-token block): each wave
// instruction moves chunk columns 2u and 2u+1 of all 32 rows (lane l: column 2u + l/32, row l%32);
// rows >= valid are taken from row 0 of the block. The copy is issued from inline asm so the
// compiler does not make later LDS reads wait for it (it would insert vmcnt(0) before reads of the
// other stages); completion is awaited explicitly with wait_vmcnt before the barrier that publishes
// the stage. M0 holds the LDS destination; no compiler-generated code in this kernel uses M0.
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <int NW>
__device__ __forceinline__ void issue_stage(const uint16_t* src_blk, int half, lds_char* dst, int valid, int wave,
                                            int lane) {
  const uint64_t a = reinterpret_cast<uint64_t>(src_blk);
  i32x4 rsrc;
  rsrc.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  rsrc.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  rsrc.z = kBlock * kRowBytes;                                        // bytes addressable: the block
  rsrc.w = 0x00020000;
  const int odd = lane >> 5;
  const int row = (lane & 31) ^ (4 * odd);  // logical row stored at this lane's LDS slot
  const uint32_t voff = (uint32_t)((row < valid ? row : 0) * kRowBytes + odd * 16);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst + wave * 1024);
#pragma unroll
  for (int j = 0; j < kStageUnits / NW; ++j) {
    const int u = j * NW + wave;
    const uint32_t soff = __builtin_amdgcn_readfirstlane(half * kStageBytes + u * 32);
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
__device__ __forceinline__ void exact_split_fallback(const CacheView& cache, int b, int qrow, int t0, int t1,
                                                     int n_heads, int h0,
                                                  const uint16_t* __restrict__ q_abs, float scale_log2,
                                                  int num_splits, int s, uint16_t* __restrict__ o_partial,
                                                  float* __restrict__ lse_partial, int lane) {
  for (int hh = 0; hh < 32; ++hh) {
    const int h = h0 + hh;
    if (h >= n_heads) break;
    const uint16_t* qa = q_abs + ((int64_t)qrow * n_heads + h) * kRow;
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
    const int64_t prow = ((int64_t)qrow * n_heads + h) * num_splits + s;
#pragma unroll
    for (int k = 0; k < 8; ++k) o_partial[prow * kDc + lane + 64 * k] = f32_to_bf16(acc[k] / l);
    if (lane == 0) lse_partial[prow] = (m + __log2f(l)) * kLn2;
  }
}

}  // namespace

template <int NW>
__global__ void __launch_bounds__(NW * 64, 1)
decode_mfma_kernel(CacheView cache, int n_heads, int n_head_groups, const int32_t* __restrict__ seq_lens,
                   const int32_t* __restrict__ cu_q_lens, int batch, const uint16_t* __restrict__ q_abs,
                   float scale_log2, int split_tokens, int num_splits, uint16_t* __restrict__ o_partial,
                   float* __restrict__ lse_partial) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kStages * kStageBytes];
  __shared__ int restart_flag;
  lds_char* lds = (lds_char*)smem_raw;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kh = lane >> 5;
  int w = logical_block(blockIdx.x, gridDim.x);
  const int hg = w % n_head_groups;
  w /= n_head_groups;
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
  const int head = hg * (32 * NW) + wave * 32 + (lane & 31);
  const bool hok = head < n_heads;
  const int t0 = s * split_tokens;
  const int t1 = min(L, t0 + split_tokens);

  if (t1 <= t0) {  // empty split: zero partial, lse = -inf
    const int h0 = hg * (32 * NW);
    for (int i = threadIdx.x; i < 32 * NW * (kDc / 8); i += NW * 64) {
      const int h = h0 + i / (kDc / 8);
      if (h < n_heads)
        reinterpret_cast<uint4*>(o_partial + (((int64_t)qrow * n_heads + h) * num_splits + s) * kDc)[i % (kDc / 8)] =
            make_uint4(0, 0, 0, 0);
    }
    if (threadIdx.x < 32 * NW && h0 + (int)threadIdx.x < n_heads)
      lse_partial[((int64_t)qrow * n_heads + h0 + threadIdx.x) * num_splits + s] = -INFINITY;
    return;
  }

  // Q^T (B operand of the score MFMA): lane holds head `head`, dims 16*ks + 8*kh .. +7.
  bf16x8 qreg[36];
  {
    const uint4* qsrc =
        reinterpret_cast<const uint4*>(q_abs + ((int64_t)qrow * n_heads + (hok ? head : 0)) * kRow + 8 * kh);
    // Heads past n_heads score with head 0's query: their columns are computed and dropped (no
    // value is masked here, so nothing waits on these loads before the first copies go out).
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, qsrc[2 * ks]);
  }

  // stage k covers tokens t0 + 32k .. +31: half (k & 1) of block blk0 + k/2 (t0 is block aligned)
  const int nstages = (t1 - t0 + kStageTok - 1) / kStageTok;
  const int blk0 = t0 / kBlock;
  if (threadIdx.x == 0) restart_flag = 0;
  // Stage 0 goes out right behind the query loads. The empty asm below reads the last query
  // register, so the compiler waits for every load here (the query, and stage 0 with it, which the
  // first step needs anyway) and knows the query is resident inside the loop; otherwise it would
  // guard each score MFMA with a wait that also drains the copies in flight. Stages 1 and 2 follow.
  issue_stage<NW>(block_ptr(cache, b, blk0), 0, lds, min(kStageTok, t1 - t0), wave, lane);
  asm volatile("" ::"v"(qreg[35]));
#pragma unroll
  for (int k = 1; k < kStages - 1; ++k)
    if (k < nstages)
      issue_stage<NW>(block_ptr(cache, b, blk0 + (k >> 1)), k & 1, lds + k * kStageBytes,
                      min(kStageTok, t1 - t0 - k * kStageTok), wave, lane);

  // Score operand: lane reads row (lane & 31), chunk 2*ks + kh (parity kh): one per-lane base,
  // ks * 1024 as an immediate.
  const uint32_t abase = kh * 512 + (((lane & 31) ^ (4 * kh)) << 4);
  // Transposed value operand: in each 16-lane group g, lane r supplies row 16 ksp + 8 half + 4 kh + r/4
  // and latent column 32 dblk + 16 (g&1) + 4 (r%4), i.e. chunk 4 dblk + 2 (g&1) + ((r>>1)&1) at byte
  // 8 (r&1); only kh and that chunk parity move the row XOR: one per-lane base plus immediates.
  const int r16 = lane & 15;
  const int tpar = (r16 >> 1) & 1;
  const uint32_t tbase = (2 * ((lane >> 4) & 1) + tpar) * 512 + ((4 * (kh ^ tpar)) + (r16 >> 2)) * 16 + 8 * (r16 & 1);

  // Online softmax against a reference max m_ref (log2 units) fixed by the first scored stage.
  // Weights are exp2(s - m_ref) <= 2^kMaxExcess, so the accumulators are never rescaled in the loop.
  // If a later stage's max exceeds m_ref + kMaxExcess, every wave of the work-group discards its
  // accumulators and recomputes its heads with the exact fallback below (in practice never taken).
  float m_ref = -INFINITY;
  f32x16 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x16{};
  float lsum = 0.f;
  bool overflow = false;
  bool restart = false;
  for (int k = 0; k < nstages; ++k) {
    // stage k has landed once only the stages issued after it (at most two) are outstanding
    const int after = min(kStages - 2, nstages - 1 - k);
    if (after == 2)
      wait_vmcnt<2 * kStageUnits / NW>();
    else if (after == 1)
      wait_vmcnt<kStageUnits / NW>();
    else
      wait_vmcnt<0>();
    wg_barrier();  // publishes stage k; every wave is also done with stage k-1's buffer
    restart |= restart_flag != 0;
    if (k + kStages - 1 < nstages) {
      const int kn = k + kStages - 1;
      issue_stage<NW>(block_ptr(cache, b, blk0 + (kn >> 1)), kn & 1, lds + (kn % kStages) * kStageBytes,
                      min(kStageTok, t1 - t0 - kn * kStageTok), wave, lane);
    }
    const uint32_t soff = (k % kStages) * kStageBytes;
    const int valid = min(kStageTok, t1 - t0 - k * kStageTok);

    // ---- scores S^T[32 tokens x 32 heads]
    f32x16 sacc;
    {
      const lds_char* ab = lds + (abase + soff);
      constexpr int kAhead = 4;  // operand loads issued this many MFMAs ahead
      bf16x8 a_buf[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) a_buf[i] = lds_b128(ab + i * 1024);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        const bf16x8 a = a_buf[ks % kAhead];
        if (ks + kAhead < 36) a_buf[ks % kAhead] = lds_b128(ab + (ks + kAhead) * 1024);
        if (ks == 0)
          score_mfma_first(sacc, a, qreg[0]);
        else
          score_mfma(sacc, a, qreg[ks]);
      }
    }
    score_mfma_drain(sacc);
    // ---- softmax weights; element j is token 8*(j>>2) + 4*kh + (j&3) of the stage
    if (valid < kStageTok) {  // only the split's last, partly filled stage needs a mask
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int tk = 8 * (j >> 2) + 4 * kh + (j & 3);
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
          lo_n = lds_tr16(tb + (dblk + 1) * 2048);
          hi_n = lds_tr16(tb + (dblk + 1) * 2048 + 8 * 16);
        }
        const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb, o[dblk], 0, 0, 0);
        lo = lo_n;
        hi = hi_n;
      }
    }
    if (__any(overflow) && lane == 0) restart_flag = 1;
  }
  wg_barrier();
  restart |= restart_flag != 0;

  if (restart) {
    exact_split_fallback(cache, b, qrow, t0, t1, n_heads, hg * (32 * NW) + wave * 32, q_abs, scale_log2,
                         num_splits, s, o_partial, lse_partial, lane);
    return;
  }

  lsum += __shfl_xor(lsum, 32);
  if (!hok) return;
  const float inv = 1.f / lsum;
  const int64_t prow = ((int64_t)qrow * n_heads + head) * num_splits + s;
  uint16_t* dst = o_partial + prow * kDc;
#pragma unroll
  for (int dblk = 0; dblk < 16; ++dblk) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dblk + 8 * g + 4 * kh;
      const f32x2 v01 = {o[dblk][4 * g] * inv, o[dblk][4 * g + 1] * inv};
      const f32x2 v23 = {o[dblk][4 * g + 2] * inv, o[dblk][4 * g + 3] * inv};
      *reinterpret_cast<uint2*>(dst + d) =
          make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(v01, bf16x2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, bf16x2)));
    }
  }
  if (kh == 0) lse_partial[prow] = (m_ref + __log2f(lsum)) * kLn2;
}

template <int NW>
static hipError_t launch_nw(const CacheView& cache, int rows, int n_heads, const int32_t* seq_lens,
                            const int32_t* cu_q_lens, int batch, const uint16_t* q_abs, float scale, int split_tokens,
                            int num_splits, uint16_t* o_partial, float* lse_partial, hipStream_t stream) {
  const int groups = (n_heads + 32 * NW - 1) / (32 * NW);
  const int64_t nwg = (int64_t)groups * num_splits * rows;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_mfma_kernel<NW>, dim3((unsigned)nwg), dim3(NW * 64), 0, stream, cache, n_heads, groups,
                     seq_lens, cu_q_lens, batch, q_abs, scale * kLog2e, split_tokens, num_splits, o_partial,
                     lse_partial);
  return hipGetLastError();
}

hipError_t launch_attention(const CacheView& cache, int rows, int n_heads, const int32_t* seq_lens,
                            const int32_t* cu_q_lens, int batch, const uint16_t* q_abs, float scale, int split_tokens,
                            int num_splits, uint16_t* o_partial, float* lse_partial, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
#define MLA_LAUNCH(NW_)                                                                                         \
  return launch_nw<NW_>(cache, rows, n_heads, seq_lens, cu_q_lens, batch, q_abs, scale, split_tokens, num_splits, \
                        o_partial, lse_partial, stream)
  if (n_heads >= 128) MLA_LAUNCH(4);
  if (n_heads > 64) MLA_LAUNCH(3);
  if (n_heads > 32) MLA_LAUNCH(2);
  MLA_LAUNCH(1);
#undef MLA_LAUNCH
}

}  // namespace mla
