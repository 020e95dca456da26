// Expanded-form chunked prefill: the cached latents are up-projected to per-head keys and values,
// then standard causal attention runs with 192-wide keys [k_nope | k_R] and 128-wide values
// ("Multi-Head Latent Attention: DeepSeek V2/V3 工程视角" names up-projection and the absorbed
// equivalent as the two ways to use the latent cache; "论文复现工坊 No.4", section 2: the per-head
// split of wkv_b into k_nope and v, the score as q_nope . k_nope + q_R . k_R, scale 1/sqrt(192)).
//
// For a chunk that attends to a long cached prefix this does fewer multiply-adds than the absorbed
// form: per (query, key, head) 2 (192 + 128) instead of 2 (576 + 512), plus 2 * 256 * 512 per
// (key, head) for the up-projection, shared by every query of the chunk that sees the key.
//
// Two kernels:
//   1. upproj_kernel: [K_up | V_up](b, h, t) = [W_UK[h]; W_UV[h]] c_t for every cached token t of every
//      sequence (bf16 out, fp32 accumulation). Work-group (256 tokens, head), 8 waves; the A operand
//      is the head's 256 weight rows, the B operand the tokens' latents, both through LDS in K stages
//      of 64.
//   2. expanded_attn_kernel: work-group (256 queries of one sequence, head), 8 waves of 32 queries.
//      Keys stream in 64-key stages (K_up, k_R from the cache rows, V_up) through LDS. Scores are
//      S^T = K Q^T (queries in registers as the B operand), so every lane holds one query's scores
//      and the softmax weights become the B operand of O^T += V^T P^T without leaving registers;
//      V^T comes from LDS with transposing reads. Online softmax with a lazy reference: the running
//      max only moves (and the accumulators are rescaled) when a tile's max exceeds it by 2^8.
#include <algorithm>
#include <type_traits>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kXcds = 8;
constexpr int kSeg = 128;  // bytes of one row of an LDS sub-tile (64 bf16)

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Barrier after this wave's LDS reads are complete; builtins, so the compiler's wait insertion
// knows those reads are over.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0 (gfx9 encoding)
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  r.z = (int)bytes;
  r.w = 0x00020000;
  return r;
}

// One wave instruction of a stage copy: 64 lanes x 16 bytes from rsrc + voff + soff into LDS at
// M0 + 16 lane. Inline asm so the compiler does not drain it before unrelated LDS reads; waited for
// with wait_vmcnt before the barrier that publishes the stage. M0 holds the LDS destination; no
// compiler-generated code in these kernels uses M0.
__device__ __forceinline__ void copy_seg(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t m0) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(rsrc), "s"(m0),
               "s"(soff)
               : "memory", "m0");
#pragma clang diagnostic pop
}

__device__ __forceinline__ bf16x8 lds_b128(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

__device__ __forceinline__ i16x4 lds_tr16(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

// 16-byte chunk swizzle of a 128-byte LDS row: the rows one LDS cycle serves (8 or 16 rows of one
// chunk) land on distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ uint32_t seg_off(int row, int chunk) { return row * kSeg + 16 * (chunk ^ swz(row)); }
// Swizzle of the value sub-tiles, which only transposing reads touch: one read instruction covers rows
// r0 .. r0 + 7 (two groups of four) at four adjacent chunks, and rows r and r + 2 must then differ in
// bit 2 of the swizzle to reach different banks; the rotation of the row within its 8 does that (swz
// above left rows r, r + 2 2-way conflicted: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE 0.50 -> 0 on a
// kernel that issues exactly these reads).
__device__ __forceinline__ int swz_v(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
// Swizzle of the attention's key sub-tiles: the same rotation, flipped by bit 3 of the row. The 16 rows
// one LDS cycle serves at one chunk still fall on distinct bank groups, and rows 32 apart share a
// swizzle, so every key-operand address is a per-lane base plus a compile-time offset.
__device__ __forceinline__ int swz_k(int row) { return swz_v(row) ^ (2 * ((row >> 3) & 1)); }

// Lanes l and l ^ 32 hold the low and high 8 bytes of four 16-byte chunks: x[2q], x[2q + 1] the lane's
// half of chunk q. After the exchange the low lane holds whole chunks 0 (c[0]) and 1 (c[1]), the high
// lane whole chunks 2 and 3 (v_permlane32_swap hands the low lane the high lane's first operand and the
// high lane the low lane's second operand), so each stores 16-byte pieces.
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

// Work-groups go to the XCDs round-robin by id; logical index L runs contiguously on one XCD.
__device__ __forceinline__ int xcd_logical(int h, int G) {
  const int q = G / kXcds, r = G % kXcds, x = h % kXcds, slot = h / kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + slot;
}

// Base of (seq, logical block) in the cache; seq and blk are wave-uniform. The table is read through
// the constant address space, i.e. with a scalar load (counted by lgkmcnt): a vector load would make
// its wait also drain the stage copies in flight.
__device__ __forceinline__ const uint16_t* block_base(const CacheView& c, int seq, int blk) {
  const __attribute__((address_space(4))) int32_t* tab = (const __attribute__((address_space(4))) int32_t*)c.table;
  int64_t phys;
  if (c.table) {
    phys = (int64_t)__builtin_amdgcn_readfirstlane(tab[(int64_t)seq * c.max_blocks + blk]);
  } else {
    phys = (int64_t)seq * c.max_blocks + blk;
  }
  return c.data + phys * (int64_t)(kBlock * kRow);
}

// max and sum of a value over the lane pair (l, l ^ 32), returned to both lanes: v_permlane32_swap
// trades the two halves in registers (a shuffle through ds_bpermute would wait on the LDS queue)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x4_lo(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// Up-projection. Work-group (head h, 256-token tile mt of sequence b), eight waves:
// D[n][t] = sum_k W[n][k] c_t[k], n < 256 the head's W_UK rows then W_UV rows, t the tile's tokens,
// k over the 512 latents in stages of 64. Stage in LDS: rows 0..255 the tokens' latents, rows
// 256..511 the weight rows (64 KB; two stage buffers). Wave (wn, wm) = (w / 4, w % 4) computes weight
// rows 128 wn .. +127 (wn = 0: keys, 1: values) for tokens 64 wm .. +63 as 4 x 2 blocks of 32 x 32.
// The larger tile (against 128 tokens) cuts the bytes copied into LDS per multiply-add by a third.
constexpr int kUpTok = 256, kUpW = 256, kUpWaves = 8, kUpStages = 2;
constexpr int kUpStageBytes = (kUpTok + kUpW) * kSeg;  // 64 KB
constexpr int kUpInstr = 8;                              // copy instructions per wave per stage
constexpr int kUpPad = 128;                              // lpad granule
constexpr int kUpOutPitch = 2 * kDnope * 2 + 16;         // staged output row: keys | values, padded (528 B)
constexpr int kUpLds = kUpStages * kUpStageBytes > kUpTok * kUpOutPitch ? kUpStages * kUpStageBytes
                                                                        : kUpTok * kUpOutPitch;

__global__ void __launch_bounds__(512) upproj_kernel(CacheView cache, const int32_t* __restrict__ seq_lens,
                                                     int n_heads, int mtiles, int lpad,
                                                     const uint16_t* __restrict__ w_uk,
                                                     const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ k_up,
                                                     uint16_t* __restrict__ v_up) {
  __shared__ __attribute__((aligned(1024))) char smem[kUpLds];
  lds_char* lds = (lds_char*)smem;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  const int L = xcd_logical((int)blockIdx.x, (int)gridDim.x);
  const int h = L % n_heads, mt = (L / n_heads) % mtiles, b = L / (n_heads * mtiles);
  const int len = seq_lens[b];
  const int m0 = mt * kUpTok;
  if (m0 >= len) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, rl = lane >> 3;

  // latents: wave w copies tokens m0 + 32 w .. +31, all in cache block (m0 + 32 w) / 64; tokens past
  // the sequence end copy its last token (finite values, never weighed by the attention)
  const int last = len - 1;
  const int blk = min((m0 + 32 * wave) / kBlock, last / kBlock);
  const i32x4 rc = buffer_rsrc(block_base(cache, b, blk), kBlock * kRowBytes);
  // weights: wave w copies rows 32 (w % 4) .. +31 of W_UK[h] (w < 4) or W_UV[h] (w >= 4)
  const i32x4 rw = buffer_rsrc((wave < 4 ? w_uk : w_uv) + (int64_t)h * kDnope * kDc, kDnope * kDc * 2);
  uint32_t voff[kUpInstr];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = 32 * wave + 8 * i + rl;
    int tok = m0 + lr;
    if (tok > last) tok = last;
    const int row = (tok / kBlock == blk) ? tok % kBlock : last % kBlock;
    voff[i] = (uint32_t)(row * kRowBytes + 16 * ((lane & 7) ^ swz(lr)));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = kUpTok + 32 * wave + 8 * i + rl;
    const int row = 32 * (wave & 3) + 8 * i + rl;
    voff[4 + i] = (uint32_t)(row * kDc * 2 + 16 * ((lane & 7) ^ swz(lr)));
  }
  auto issue = [&](int st) {
    const uint32_t buf = lds0 + (uint32_t)((st % kUpStages) * kUpStageBytes);
    const uint32_t soff = (uint32_t)(st * kSeg);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      copy_seg(rc, voff[i], soff, __builtin_amdgcn_readfirstlane(buf + (32 * wave + 8 * i) * kSeg));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      copy_seg(rw, voff[4 + i], soff, __builtin_amdgcn_readfirstlane(buf + (kUpTok + 32 * wave + 8 * i) * kSeg));
  };

  const int wn = wave >> 2, wm = wave & 3, khalf = lane >> 5;
  const int wrow0 = kUpTok + 128 * wn + (lane & 31), trow0 = 64 * wm + (lane & 31);
  f32x16 acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[j][i] = f32x16{};

  constexpr int nst = kDc / 64;  // 8 stages
  issue(0);
  for (int st = 0; st < nst; ++st) {
    wait_vmcnt<0>();
    wg_barrier();  // stage st is in LDS; every wave is done with stage st - 1, whose buffer st + 1 reuses
    if (st + 1 < nst) issue(st + 1);
    const lds_char* buf = lds + (st % kUpStages) * kUpStageBytes;
    bf16x8 wa[2][4], tb[2][2];
    auto load = [&](int kk, int slot) {
#pragma unroll
      for (int j = 0; j < 4; ++j) wa[slot][j] = lds_b128(buf + seg_off(wrow0 + 32 * j, 2 * kk + khalf));
#pragma unroll
      for (int i = 0; i < 2; ++i) tb[slot][i] = lds_b128(buf + seg_off(trow0 + 32 * i, 2 * kk + khalf));
    };
    load(0, 0);
    static_for<0, 4>([&](auto kk) {
      constexpr int cur = decltype(kk)::value & 1;
      if constexpr (decltype(kk)::value + 1 < 4) load(decltype(kk)::value + 1, cur ^ 1);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[cur][j], tb[cur][i], acc[j][i], 0, 0, 0);
    });
  }

  // The tile goes out through LDS as whole rows: staged as [token][keys (256 B) | values (256 B)] with
  // a padded pitch, then every store instruction writes two tokens' 512 bytes (two 256-byte rows of
  // K_up and of V_up). D layout: lane holds token column lane % 32 and weight rows
  // 8 (e / 4) + 4 (lane / 32) + e % 4 of a block, i.e. four consecutive outputs per (block, e / 4).
  wg_barrier();  // every wave is done reading the stages
  // The lane pair (l, l ^ 32) (the same token, columns 4 khalf .. +3 of each 8) trades halves so that
  // every staging store is a whole 16-byte piece: the 8-byte stores of the halves were 2-way bank
  // conflicted at this pitch (tokens t and t + 16 of 32 lanes on the same banks).
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tl = 64 * wm + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x[8];
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        x[2 * e4] = pack_bf16x4_lo(acc[j][i][4 * e4], acc[j][i][4 * e4 + 1]);
        x[2 * e4 + 1] = pack_bf16x4_lo(acc[j][i][4 * e4 + 2], acc[j][i][4 * e4 + 3]);
      }
      u32x4 chunk[2];
      pair_chunks(x, chunk);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int col = 128 * wn + 32 * j + 8 * (2 * khalf + t);
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lds + tl * kUpOutPitch + 2 * col) = chunk[t];
      }
    }
  }
  wg_barrier();
  const int64_t kvbase = ((int64_t)(b * n_heads + h) * lpad + m0) * kDnope;
  // 256 tokens x 32 chunks of 16 bytes; thread t takes chunk t % 32 of tokens t / 32 + 16 k. Rows past
  // lpad (a last tile that overhangs it) are not stored.
  const int c = threadIdx.x & 31, part = c >> 4, cc = c & 15;
  uint16_t* dst = (part == 0 ? k_up : v_up) + kvbase + 8 * cc;
#pragma unroll 4
  for (int k = 0; k < kUpTok / 16; ++k) {
    const int tl = (threadIdx.x >> 5) + 16 * k;
    if (m0 + tl >= lpad) break;
    const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lds + tl * kUpOutPitch + 16 * c);
    *reinterpret_cast<u32x4*>(dst + (int64_t)tl * kDnope) = v;
  }
}

// ------------------------------------------------------------------------------------------------
// Attention. Work-group (256 queries of one sequence, head): eight waves, two per SIMD, wave w owns
// queries 32 w .. +31, so one wave's softmax (VALU) runs beside the other wave's MFMAs. Stage = 64
// keys in five LDS sub-tiles of 64 rows x 128 bytes: 0, 1 = K_up columns 0-63, 64-127; 2 = k_R (from
// the cache rows); 3, 4 = V_up columns 0-63, 64-127. Copy instruction i of wave w moves rows
// 8 w .. +7 of sub-tile i.
constexpr int kFaQ = 256, kFaWaves = 8, kFaKeys = 64, kFaStages = 3;
constexpr int kFaSub = kFaKeys * kSeg;        // 8 KB
constexpr int kFaStageBytes = 5 * kFaSub;     // 40 KB
constexpr int kFaInstr = 5;                   // copy instructions per wave per stage
constexpr float kRescaleExcess = 8.0f;        // log2 units: weights stay below 2^8 between rescales

__global__ void __launch_bounds__(512) expanded_attn_kernel(CacheView cache, const int32_t* __restrict__ seq_lens,
                                                            const int32_t* __restrict__ cu_q_lens, int n_heads,
                                                            int qtiles, int lpad, const uint16_t* __restrict__ q_nope,
                                                            const uint16_t* __restrict__ q_rope,
                                                            const uint16_t* __restrict__ k_up,
                                                            const uint16_t* __restrict__ v_up, float scale_log2,
                                                            uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(1024))) char smem[kFaStages * kFaStageBytes];
  lds_char* lds = (lds_char*)smem;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  const int L = xcd_logical((int)blockIdx.x, (int)gridDim.x);
  const int qt = L % qtiles, h = (L / qtiles) % n_heads, b = L / (qtiles * n_heads);
  const int q0 = cu_q_lens[b], qlen = cu_q_lens[b + 1] - q0, len = seq_lens[b];
  if (qt * kFaQ >= qlen) return;
  const int pos0 = len - qlen;  // position of the chunk's first query
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, khalf = lane >> 5;
  const int wg_last = min(qt * kFaQ + kFaQ - 1, qlen - 1);
  const int nkt = (pos0 + wg_last + 1 + kFaKeys - 1) / kFaKeys;  // key tiles the work-group needs
  const int w_first = qt * kFaQ + 32 * wave;                    // the wave's first query (chunk index)
  const bool w_live = w_first < qlen;
  const int w_last = min(w_first + 31, qlen - 1);
  const int w_nkt = w_live ? (pos0 + w_last + 1 + kFaKeys - 1) / kFaKeys : 0;

  // the lane's query: chunk index jq (clamped into the chunk), position pq
  const int jq = min(w_first + (lane & 31), qlen - 1);
  const int pq = pos0 + jq;
  // Q^T operand (B): query jq, elements 16 ks + 8 khalf .. +7 of [q_nope | q_R]
  bf16x8 qop[12];
  {
    const int64_t row = (int64_t)(q0 + jq) * n_heads + h;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      const int d = 16 * ks + 8 * khalf;
      qop[ks] = ks < 8 ? *reinterpret_cast<const bf16x8*>(q_nope + row * kDnope + d)
                       : *reinterpret_cast<const bf16x8*>(q_rope + row * kDr + (d - kDnope));
    }
  }
  // The query loads complete here, with a wait the compiler sees: otherwise it guards the loop's
  // MFMAs with waits on its own count of outstanding loads, which the stage copies would also satisfy
  // only once they complete.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0, expcnt 7, lgkmcnt 15 (gfx9 encoding)

  const int64_t kv_base = ((int64_t)(b * n_heads + h) * lpad) * kDnope;
  auto issue = [&](int kt) {
    const uint32_t buf = lds0 + (uint32_t)((kt % kFaStages) * kFaStageBytes) + (uint32_t)(8 * wave * kSeg);
    const int t0 = kt * kFaKeys;
    const i32x4 rk = buffer_rsrc(k_up + kv_base + (int64_t)t0 * kDnope, kFaKeys * kDnope * 2);
    const i32x4 rv = buffer_rsrc(v_up + kv_base + (int64_t)t0 * kDnope, kFaKeys * kDnope * 2);
    const i32x4 rr = buffer_rsrc(block_base(cache, b, kt), kBlock * kRowBytes);
    // lane l lands at row r = 8 w + l / 8, slot l % 8 of each sub-tile, so it fetches chunk
    // (l % 8) ^ swz_k(r) (keys, k_R) or (l % 8) ^ swz_v(r) (values); the offsets are recomputed here
    // rather than held across the loop (the empty asm makes the lane index opaque at this point)
    int lv = lane;
    asm volatile("" : "+v"(lv));
    const int r = 8 * wave + (lv >> 3);
    const int c16 = 16 * ((lv & 7) ^ swz_k(r));
    const uint32_t okv = (uint32_t)(r * kDnope * 2 + c16);
    const uint32_t ov = (uint32_t)(r * kDnope * 2 + 16 * ((lv & 7) ^ swz_v(r)));  // value sub-tiles
    copy_seg(rk, okv, 0, __builtin_amdgcn_readfirstlane(buf + 0 * kFaSub));
    copy_seg(rk, okv + kSeg, 0, __builtin_amdgcn_readfirstlane(buf + 1 * kFaSub));
    copy_seg(rr, (uint32_t)(r * kRowBytes + kDc * 2 + c16), 0, __builtin_amdgcn_readfirstlane(buf + 2 * kFaSub));
    copy_seg(rv, ov, 0, __builtin_amdgcn_readfirstlane(buf + 3 * kFaSub));
    copy_seg(rv, ov + kSeg, 0, __builtin_amdgcn_readfirstlane(buf + 4 * kFaSub));
  };

  // K operand (A): key row 32 kb + lane % 32, elements 16 ks + 8 khalf: sub-tile ks / 4 (ks < 8) or
  // 2 (k_R), chunk 2 (ks % 4) + khalf.
  // V^T operand (A, transposing reads): in 16-lane group g, lane r reads key row
  //   32 kb + 16 half + 8 rd + 4 (g / 2) + r / 4 at value column 32 j + 16 (g % 2) + 4 (r % 4)
  // and receives column 32 j + lane % 32 of 4 keys: the key order of the weights' B operand.
  const int g16 = lane >> 4, r16 = lane & 15;
  // per-lane parts of the operand addresses; the rest of each address is a compile-time offset.
  // Keys: row 32 kb + n (n = lane % 32) at chunk 2 m + khalf (m = ks % 4): n * 128 + 16 ((2 m +
  // khalf) ^ swz_k(n)), plus 4096 kb. Values: row 8 q + rl (q = 4 kb + 2 half + rd, rl = 4 (g16 / 2) +
  // r16 / 4 < 8) at chunk 4 (j % 2) + 2 (g16 % 2) + (r16 / 2) % 2, byte 8 (r16 % 2).
  uint32_t kl[4], vl[2];
  {
    const int n = lane & 31, rl = 4 * (g16 >> 1) + (r16 >> 2);
#pragma unroll
    for (int m = 0; m < 4; ++m) kl[m] = (uint32_t)(n * kSeg + 16 * ((2 * m + khalf) ^ swz_k(n)));
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2)
      vl[p2] = (uint32_t)(rl * kSeg + 16 * ((4 * p2 + 2 * (g16 & 1) + ((r16 >> 1) & 1)) ^ swz_v(rl)) + 8 * (r16 & 1));
#pragma unroll
    for (int m = 0; m < 4; ++m) asm volatile("" : "+v"(kl[m]));  // held, not recomputed in the loop
    asm volatile("" : "+v"(vl[0]), "+v"(vl[1]));
  }
  float m_ref = -INFINITY, lsum = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = f32x16{};

  issue(0);
  if (nkt > 1) issue(1);
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt)
      wait_vmcnt<kFaInstr>();
    else
      wait_vmcnt<0>();
    wg_barrier();  // stage kt is in LDS; every wave is done with stage kt - 1, whose buffer kt + 2 reuses
    if (kt + 2 < nkt) issue(kt + 2);
    if (kt >= w_nkt) continue;  // every key of this tile is after the wave's last query
    const lds_char* buf = lds + (kt % kFaStages) * kFaStageBytes;
    const int t0 = kt * kFaKeys;
    const bool masked = t0 + kFaKeys - 1 > pos0 + w_first;
    // two halves of 32 keys: scores, softmax, value product
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) {
        const int sub = ks < 8 ? ks >> 2 : 2;
        const bf16x8 kop = lds_b128(buf + kl[ks & 3] + (sub * kFaSub + 32 * kb * kSeg));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], sc, 0, 0, 0);
      }
      // softmax: lane holds query jq and keys t0 + 32 kb + 8 (e / 4) + 4 khalf + e % 4; the max is
      // taken on the raw scores (scale > 0), masked keys become -inf
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (masked) {
          const int t = t0 + 32 * kb + 8 * (e >> 2) + 4 * khalf + (e & 3);
          if (t > pq) sc[e] = -INFINITY;
        }
        mx = fmaxf(mx, sc[e]);
      }
      mx = pair_max(mx) * scale_log2;
      if (__any(mx > m_ref + kRescaleExcess)) {
        const float mn = fmaxf(m_ref, mx);
        const float f = exp2f(m_ref - mn);  // 0 on the first tile (m_ref = -inf)
        lsum *= f;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] *= f;
        m_ref = mn;
      }
      // p = 2^(scale_log2 s - m_ref) <= 2^8 (v_exp_f32: arguments below -126 give 0, weights below
      // fp32's normal range anyway)
      const float nm = -m_ref;
      bf16x8 pk[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * half + e], scale_log2, nm));
          lsum += p;
          pk[half][e] = (__bf16)p;
        }
      }
      // O^T[value column][query] += V^T P^T over the half's 32 keys
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sub = 3 + (j >> 1);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          i16x4 t[2];
#pragma unroll
          for (int rd = 0; rd < 2; ++rd)
            t[rd] = lds_tr16(buf + vl[j & 1] + (sub * kFaSub + (32 * kb + 16 * half + 8 * rd) * kSeg));
          const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
          o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pk[half], o[j], 0, 0, 0);
        }
      }
    }
  }
  if (!w_live) return;

  // out[j, h, d] = O / l; lanes l and l ^ 32 hold the same query (different keys and value rows)
  const float tot = pair_sum(lsum);
  const float inv = 1.f / tot;
  const int jl = w_first + (lane & 31);
  if (jl >= qlen) return;
  const int64_t row = (int64_t)(q0 + jl) * n_heads + h;
  uint16_t* orow = out + row * kDv;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int d = 32 * j + 8 * e4 + 4 * khalf;
      const uint2 v = make_uint2(pack_bf16x4_lo(o[j][4 * e4] * inv, o[j][4 * e4 + 1] * inv),
                                 pack_bf16x4_lo(o[j][4 * e4 + 2] * inv, o[j][4 * e4 + 3] * inv));
      *reinterpret_cast<uint2*>(orow + d) = v;
    }
  if (lse_out != nullptr && khalf == 0) lse_out[row] = (m_ref + log2f(tot)) * 0.6931471805599453f;
}

size_t prefill_expanded_kv_bytes(int batch, int n_heads, int max_seq_len) {
  const size_t lpad = (size_t)((max_seq_len + kUpPad - 1) / kUpPad) * kUpPad;
  return 2 * (size_t)batch * n_heads * lpad * kDnope * 2;
}

hipError_t launch_prefill_expanded(const CacheView& cache, int batch, int n_heads, const int32_t* seq_lens,
                                   const int32_t* cu_q_lens, int max_q_len, int max_seq_len, const uint16_t* q_nope,
                                   const uint16_t* q_rope, const uint16_t* w_uk, const uint16_t* w_uv, float scale,
                                   void* workspace, uint16_t* out, float* lse_out, hipStream_t stream) {
  const int mtiles = (max_seq_len + kUpTok - 1) / kUpTok;
  const int lpad = (max_seq_len + kUpPad - 1) / kUpPad * kUpPad;
  uint16_t* k_up = static_cast<uint16_t*>(workspace);
  uint16_t* v_up = k_up + (size_t)batch * n_heads * lpad * kDnope;
  const int64_t g1 = (int64_t)batch * mtiles * n_heads;
  const int qtiles = (max_q_len + kFaQ - 1) / kFaQ;
  const int64_t g2 = (int64_t)batch * n_heads * qtiles;
  if (g1 > 0x7FFFFFFF || g2 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(upproj_kernel, dim3((unsigned)g1), dim3(kUpWaves * 64), 0, stream, cache, seq_lens, n_heads, mtiles, lpad, w_uk,
                     w_uv, k_up, v_up);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(expanded_attn_kernel, dim3((unsigned)g2), dim3(kFaWaves * 64), 0, stream, cache, seq_lens, cu_q_lens, n_heads,
                     qtiles, lpad, q_nope, q_rope, k_up, v_up, scale_log2, out, lse_out);
  return hipGetLastError();
}

}  // namespace mla
