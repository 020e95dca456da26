// Tiled bf16 GEMM with fp32 split-K partials: part[s][m][n] = sum over split s's K range of
// A[m][k] * B[n][k]. Both operands are K-contiguous (activations [M, K]; a weight in the nn.Linear
// row layout [N, K]), which is how the projections around the latent cache store them.
//
// Work-group: one (N tile, M tile, K split), four waves in a 2 x 2 grid over a BM x BN tile; each wave
// holds (BM/64) x (BN/64) accumulators of v_mfma_f32_32x32x16_bf16 (a 32 x 32 fp32 block each).
// Operands stream global -> LDS with buffer_load ... lds in K stages of 64 (128 bytes per row), four
// stage buffers deep (the whole 160 KB of LDS). A wave instruction moves eight whole 128-byte row segments: lane l fetches row
// 8i + l/8 at 16-byte chunk (l % 8) ^ swz(row) and lands at LDS offset 16 l, so a row's chunks sit
// XOR-swizzled by the row index and the MFMA operand reads (32 rows at one chunk) spread over the
// banks. Rows of A past M are fetched from row M - 1 and never stored.
#include <algorithm>
#include <type_traits>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kBK = 64;          // K per stage
constexpr int kRowSeg = kBK * 2; // bytes of one row in a stage
constexpr int kXcds = 8;         // accelerator complex dies, each with its own L2
constexpr int kNumBuf = 4;       // stage buffers: three stages in flight while one is consumed

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

// Work-group barrier after this wave's LDS reads are complete (lgkmcnt 0). Written with builtins so
// that the compiler's wait insertion knows those reads are over and does not add a wait of its own
// in front of the next MFMAs (which would also drain the reads issued after the barrier).
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

// One wave instruction of a stage copy (1 KB). Issued from inline asm so that the compiler does not
// make the LDS reads of other stages wait for it; completion is awaited with wait_vmcnt before the
// barrier that publishes the stage. M0 holds the LDS destination; no compiler-generated code in
// this kernel uses M0.
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

// LDS byte offset of (row, 16-byte chunk) of a stage: the chunk is XOR-swizzled by
// swz(row) = (row ^ row / 8) % 8, which gives the rows that one LDS cycle serves (8 rows of one
// 16-byte chunk for 32 banks, 16 rows for 64) distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ uint32_t seg_off(int row, int chunk) { return row * kRowSeg + 16 * (chunk ^ swz(row)); }

}  // namespace

template <int BM, int BN>
__global__ void __launch_bounds__(256) gemm_bt_partial_kernel(int M, int N, int K, int nsplit,
                                                              const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B,
                                                              float* __restrict__ part) {
  constexpr int kStageBytes = (BM + BN) * kRowSeg;
  constexpr int kAInstr = BM / 32;  // copy instructions per wave per stage (8 rows each, 4 waves)
  constexpr int kBInstr = BN / 32;
  constexpr int kMi = BM / 64, kNj = BN / 64;  // 32 x 32 blocks per wave
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sizes");
  __shared__ __attribute__((aligned(1024))) char smem[kNumBuf * kStageBytes];
  lds_char* lds = (lds_char*)smem;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Work-groups are handed to the 8 XCDs round-robin by id. Logical tile L = ((s * mtiles) + mt) *
  // ntiles + nt is placed so that each XCD runs a contiguous range of L: the N tiles of one (M tile,
  // split) share their A rows in one L2, and an XCD touches the weight of one or two splits only.
  const int ntiles = N / BN, mtiles = (M + BM - 1) / BM;
  const int G = (int)gridDim.x, h = (int)blockIdx.x;
  const int q = G / kXcds, r = G % kXcds, xcd = h % kXcds, slot = h / kXcds;
  const int L = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
  const int nt = L % ntiles, mt = (L / ntiles) % mtiles, s = L / (ntiles * mtiles);
  const int n0 = nt * BN, m0 = mt * BM;
  const int nst_all = K / kBK;
  const int st0 = (int)((int64_t)s * nst_all / nsplit), st1 = (int)((int64_t)(s + 1) * nst_all / nsplit);
  const int nst = st1 - st0;

  // copy descriptors: wave w copies A rows [BM/4 w, BM/4 (w+1)) and B rows [BN/4 w, BN/4 (w+1))
  const i32x4 ra = buffer_rsrc(A, (uint32_t)((int64_t)M * K * 2));
  const i32x4 rb = buffer_rsrc(B, (uint32_t)((int64_t)N * K * 2));
  uint32_t va[kAInstr], vb[kBInstr];
  // lane l lands at LDS row lr (of the stage), slot l % 8, so it fetches chunk (l % 8) ^ swz(lr)
  const int rl = lane >> 3;
#pragma unroll
  for (int i = 0; i < kAInstr; ++i) {
    const int lr = (BM / 4) * wave + 8 * i + rl;
    const int r = min(m0 + lr, M - 1);
    va[i] = (uint32_t)r * (uint32_t)(K * 2) + 16 * ((lane & 7) ^ swz(lr));
  }
#pragma unroll
  for (int i = 0; i < kBInstr; ++i) {
    const int lr = BM + (BN / 4) * wave + 8 * i + rl;
    const int r = n0 + (BN / 4) * wave + 8 * i + rl;
    vb[i] = (uint32_t)r * (uint32_t)(K * 2) + 16 * ((lane & 7) ^ swz(lr));
  }
  auto issue = [&](int st) {
    const uint32_t buf = lds0 + (uint32_t)((st % kNumBuf) * kStageBytes);
    const uint32_t soff = (uint32_t)((st0 + st) * kRowSeg);
#pragma unroll
    for (int i = 0; i < kAInstr; ++i)
      copy_seg(ra, va[i], soff, __builtin_amdgcn_readfirstlane(buf + ((BM / 4) * wave + 8 * i) * kRowSeg));
#pragma unroll
    for (int i = 0; i < kBInstr; ++i)
      copy_seg(rb, vb[i], soff,
               __builtin_amdgcn_readfirstlane(buf + (BM + (BN / 4) * wave + 8 * i) * kRowSeg));
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int arow0 = (BM / 2) * wm + (lane & 31), brow0 = BM + (BN / 2) * wn + (lane & 31);
  const int khalf = lane >> 5;
  f32x16 acc[kMi][kNj];
#pragma unroll
  for (int i = 0; i < kMi; ++i)
#pragma unroll
    for (int j = 0; j < kNj; ++j) acc[i][j] = f32x16{};

  // Stage st + 1's operands are read from LDS into registers while the MFMAs of stage st run from
  // the other register set, so the reads overlap the matrix work instead of waiting in front of it.
  bf16x8 opa[2][kBK / 16][kMi], opb[2][kBK / 16][kNj];
  auto read_stage = [&](int st, auto slot) {
    constexpr int sl = decltype(slot)::value;
    const lds_char* buf = lds + (st % kNumBuf) * kStageBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
#pragma unroll
      for (int i = 0; i < kMi; ++i) opa[sl][kk][i] = lds_b128(buf + seg_off(arow0 + 32 * i, 2 * kk + khalf));
#pragma unroll
      for (int j = 0; j < kNj; ++j) opb[sl][kk][j] = lds_b128(buf + seg_off(brow0 + 32 * j, 2 * kk + khalf));
    }
  };
  // Wait until this wave's copies of stage `st` are done, then a barrier publishes the stage (and
  // tells every wave that the reads issued before it are over). Stages up to st + kNumBuf - 2 have
  // been issued by then, and their copies may stay pending.
  auto stage_ready = [&](int st) {
    const int pending = min(nst - 1, st + kNumBuf - 2) - st;
    if (pending >= 2)
      wait_vmcnt<2 * (kAInstr + kBInstr)>();
    else if (pending == 1)
      wait_vmcnt<kAInstr + kBInstr>();
    else
      wait_vmcnt<0>();
    wg_barrier();
  };

  auto mfma_stage = [&](auto slot) {
    constexpr int sl = decltype(slot)::value;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk)
#pragma unroll
      for (int i = 0; i < kMi; ++i)
#pragma unroll
        for (int j = 0; j < kNj; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[sl][kk][i], opb[sl][kk][j], acc[i][j], 0, 0, 0);
  };
  // one stage that has a successor: refill the freed buffer, publish and read stage st + 1 into the
  // other register set, multiply stage st
  auto step = [&](int st, auto slot) {
    constexpr int sl = decltype(slot)::value;
    // stage st - 1's buffer is free: every wave read it before the previous barrier
    if (st + kNumBuf - 1 < nst) issue(st + kNumBuf - 1);
    stage_ready(st + 1);
    read_stage(st + 1, std::integral_constant<int, sl ^ 1>{});
    mfma_stage(slot);
  };

  for (int st = 0; st < kNumBuf - 1 && st < nst; ++st) issue(st);
  stage_ready(0);  // nst >= 1 (the launcher gives every split at least one stage)
  read_stage(0, std::integral_constant<int, 0>{});
  int st = 0;
  for (; st + 2 < nst; st += 2) {
    step(st, std::integral_constant<int, 0>{});
    step(st + 1, std::integral_constant<int, 1>{});
  }
  if (st + 1 < nst) {
    step(st, std::integral_constant<int, 0>{});
    mfma_stage(std::integral_constant<int, 1>{});
  } else {
    mfma_stage(std::integral_constant<int, 0>{});
  }

  // D layout: lane holds rows 8 (e / 4) + 4 (lane / 32) + e % 4 and column lane % 32 of a block
  float* out = part + (int64_t)s * M * N;
#pragma unroll
  for (int i = 0; i < kMi; ++i)
#pragma unroll
    for (int j = 0; j < kNj; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + (BM / 2) * wm + 32 * i + 8 * (e >> 2) + 4 * khalf + (e & 3);
        const int n = n0 + (BN / 2) * wn + 32 * j + (lane & 31);
        if (m < M) out[(int64_t)m * N + n] = acc[i][j][e];
      }
}

// ------------------------------------------------------------------------------------------------
// Split-K GEMM for few rows (M up to a few hundred): part[s][m][n] = sum over split s of A[m][k] B[n][k].
// Work-group (column tile of 32, split s, block of 32 rows): wave w takes a quarter of the split's K
// range with v_mfma_f32_32x32x16_bf16 straight from global memory (both operands K-contiguous), two
// K steps of operands in flight; the four partial tiles are added through LDS. Many splits spread
// the weight B over many work-groups, so it streams from HBM once at full width. B may be two weights
// over the same K stacked by rows: columns n < N1 are rows of B, the rest rows n - N1 of B2.
constexpr int kKStep = 16;  // K per MFMA
constexpr int kAhead = 4;   // K steps whose operands are loaded ahead (a 64-long quarter at once)

__global__ void __launch_bounds__(256) splitk_gemm_kernel(int M, int N, int K, int split_len,
                                                          const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ B, int N1,
                                                          const uint16_t* __restrict__ B2,
                                                          float* __restrict__ part) {
  __shared__ float red[4 * 32 * 32];
  const int ct = blockIdx.x, s = blockIdx.y, tb = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int quarter = split_len / 4;
  const int k0 = s * split_len + wave * quarter;
  const int steps = quarter / kKStep;
  // A: row 32 tb + lane % 32 (clamped; rows past the end are computed and not stored), K half lane / 32
  const int row = min(32 * tb + (lane & 31), M - 1);
  const uint16_t* pa = A + (int64_t)row * K + k0 + 8 * (lane >> 5);
  // B: output column 32 ct + lane % 32 (a row of B, or of B2 past N1; N1 is a multiple of 32), the
  // same K half
  const int col = 32 * ct + (lane & 31);
  const uint16_t* pb = (32 * ct < N1 ? B + (int64_t)col * K : B2 + (int64_t)(col - N1) * K) + k0 + 8 * (lane >> 5);
  bf16x8 a[kAhead], b[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    if (i < steps) {
      a[i] = *reinterpret_cast<const bf16x8*>(pa + i * kKStep);
      b[i] = *reinterpret_cast<const bf16x8*>(pb + i * kKStep);
    }
  }
  f32x16 acc = f32x16{};
  for (int k = 0; k < steps; k += kAhead) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      if (k + i < steps) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], acc, 0, 0, 0);
        if (k + i + kAhead < steps) {
          a[i] = *reinterpret_cast<const bf16x8*>(pa + (k + i + kAhead) * kKStep);
          b[i] = *reinterpret_cast<const bf16x8*>(pb + (k + i + kAhead) * kKStep);
        }
      }
    }
  }
  // D: lane holds row 8 (j / 4) + 4 (lane / 32) + j % 4 and column lane % 32 of the tile
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int m = 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
    red[(wave * 32 + m) * 32 + (lane & 31)] = acc[j];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 32 * 32; e += 256) {
    const int m = e >> 5, n = e & 31;
    const int t = 32 * tb + m;
    if (t < M) part[((int64_t)s * M + t) * N + 32 * ct + n] = red[e] + red[1024 + e] + red[2048 + e] + red[3072 + e];
  }
}

int splitk_splits(int M, int N, int K) {
  // enough work-groups (column tiles x splits x row blocks) to spread B over the chip, each split a
  // multiple of 64 (four waves x 16) and at least 256 long
  const int tblocks = (M + 31) / 32;
  int ns = 512 / std::max(1, (N / 32) * tblocks);
  ns = std::max(1, std::min(std::min(ns, kGemmMaxSplits), K / 256));
  while ((K / 64) % ns != 0) --ns;
  return ns;
}

hipError_t launch_splitk_gemm2(int M, int N1, int N2, int K, int nsplit, const uint16_t* A, const uint16_t* B,
                               const uint16_t* B2, float* part, hipStream_t stream) {
  const int N = N1 + N2;
  if (M <= 0 || N1 % 32 != 0 || N2 % 32 != 0 || N <= 0 || K % 64 != 0 || nsplit < 1 || (K / 64) % nsplit != 0 ||
      (N2 > 0 && B2 == nullptr))
    return hipErrorInvalidValue;
  const int tblocks = (M + 31) / 32;
  if (tblocks > 65535 || nsplit > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(splitk_gemm_kernel, dim3(N / 32, nsplit, tblocks), dim3(256), 0, stream, M, N, K, K / nsplit, A, B,
                     N1, B2, part);
  return hipGetLastError();
}

hipError_t launch_splitk_gemm(int M, int N, int K, int nsplit, const uint16_t* A, const uint16_t* B, float* part,
                              hipStream_t stream) {
  return launch_splitk_gemm2(M, N, 0, K, nsplit, A, B, nullptr, part, stream);
}

int gemm_bt_splits(int M, int N, int K) {
  const int tiles = ((M + kGemmBM - 1) / kGemmBM) * (N / kGemmBN);
  int ns = std::max(1, 256 / std::max(1, tiles));
  ns = std::min(ns, std::max(1, K / kBK / 4));  // at least four stages per split
  return std::min(ns, kGemmMaxSplits);
}

hipError_t launch_gemm_bt_partial(int M, int N, int K, int nsplit, const uint16_t* A, const uint16_t* B, float* part,
                                  hipStream_t stream) {
  if (M <= 0 || N % kGemmBN != 0 || K % kBK != 0 || nsplit < 1 || nsplit > K / kBK) return hipErrorInvalidValue;
  if ((int64_t)M * K * 2 > 0xFFFFFFFFll || (int64_t)N * K * 2 > 0xFFFFFFFFll) return hipErrorInvalidValue;
  const int64_t wgs = (int64_t)((M + kGemmBM - 1) / kGemmBM) * (N / kGemmBN) * nsplit;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bt_partial_kernel<kGemmBM, kGemmBN>), dim3((unsigned)wgs), dim3(256), 0, stream, M, N, K,
                     nsplit, A, B, part);
  return hipGetLastError();
}

}  // namespace mla
