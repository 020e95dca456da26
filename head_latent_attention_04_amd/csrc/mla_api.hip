// C ABI of the MLA library: host-side validation, workspace layout and kernel launches.
// Every check happens before the first HIP call, so an invalid call enqueues nothing.
#include <math.h>
#include <algorithm>
#include <stddef.h>

#include <mutex>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int32_t kMaxSplitTokens = 0x7FFFFFC0;  // largest block multiple: one split per row
constexpr int32_t kMaxPrefillTokens = 1 << 24;    // query tokens of one mla_chunked_prefill call

// true if p is a multiple of n bytes (n a power of two); NULL counts as aligned (optional pointers)
bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

int check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->n_heads <= 0 || d->d_c <= 0 || d->d_rope <= 0 || d->d_nope <= 0 || d->d_v <= 0 || d->block_size <= 0)
    return MLA_ERR_BAD_ARG;
  if (!(d->scale > 0.f) || !isfinite(d->scale)) return MLA_ERR_BAD_ARG;
  if (!(d->rope_theta > 1.f) || !isfinite(d->rope_theta)) return MLA_ERR_BAD_ARG;
  if (d->d_c != mla::kDc || d->d_rope != mla::kDr || d->d_nope != mla::kDnope || d->d_v != mla::kDv ||
      d->block_size != mla::kBlock || d->n_heads % 16 != 0 || d->n_heads > 65535)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// The cache rows are read and written in 16-byte pieces (and copied into LDS by 16-byte buffer
// loads), the block table as int32.
int check_cache(const mla_cache* c) {
  if (!c || !c->data) return MLA_ERR_NULL;
  if (c->num_blocks <= 0 || c->max_blocks_per_seq <= 0) return MLA_ERR_BAD_ARG;
  if (!aligned(c->data, 16) || !aligned(c->block_table, 4)) return MLA_ERR_BAD_ARG;
  return MLA_OK;
}

int check_splits(const mla_dims* d, int32_t batch, int32_t split_tokens, int32_t num_splits) {
  if (batch < 0 || batch > 65535) return MLA_ERR_BAD_ARG;
  if (split_tokens <= 0 || split_tokens % d->block_size != 0) return MLA_ERR_BAD_ARG;
  if (num_splits <= 0 || num_splits > 65535) return MLA_ERR_BAD_ARG;
  if ((int64_t)split_tokens * num_splits > (int64_t)INT32_MAX) return MLA_ERR_BAD_ARG;
  return MLA_OK;
}

mla::CacheView view(const mla_cache* c) { return mla::CacheView{c->data, c->block_table, c->max_blocks_per_seq}; }

int launched(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }


// ---- the allocation-free decode's scratch --------------------------------------------------------
// One static device array per GPU the library runs on (it lives until the process ends). Host code
// never passes `scratch` itself to a kernel or a copy: in host code that name is a host-side
// stand-in. Its device address is looked up once per device (with the device current) and kept.
static __device__ __align__(256) uint8_t scratch[MLA_NO_ALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];

// Device address of the current device's scratch (hipGetSymbolAddress on the first call per device).
hipError_t device_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_status[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_status[dev] != hipSuccess) return g_scratch_status[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// Splits of each absorbed-prefill row's causal key range. One while the (row, 128-head group)
// work-groups fill the compute units; with fewer than kPrefillSplitCus of them, as many splits as
// still fit in one wave of work-groups on that many units (at most kMaxPrefillSplits): rounding up
// would start a second, mostly idle wave. A function of n_heads and total_q only, so the workspace
// size query knows it.
constexpr int64_t kPrefillSplitCus = 256;
constexpr int64_t kMaxPrefillSplits = 8;

int prefill_splits(int32_t n_heads, int32_t total_q) {
  const int64_t wgs = (int64_t)(total_q > 0 ? total_q : 0) * ((mla::q_tiles(n_heads) + 3) / 4);
  if (wgs <= 0 || wgs >= kPrefillSplitCus) return 1;
  return (int)std::min<int64_t>(kMaxPrefillSplits, kPrefillSplitCus / wgs);
}

struct PrefillWorkspace {
  size_t q_abs, o_lat, lse, total;
};

PrefillWorkspace prefill_layout(const mla_dims* d, int32_t total_q) {
  PrefillWorkspace w;
  const size_t parts = (size_t)(total_q > 0 ? total_q : 0) * (size_t)d->n_heads * prefill_splits(d->n_heads, total_q);
  w.q_abs = 0;
  w.o_lat = align256((size_t)(total_q > 0 ? total_q : 0) * mla::q_tiles(d->n_heads) * mla::kQTileElems * 2);
  w.lse = w.o_lat + align256(parts * mla::kDc * 2);
  w.total = w.lse + align256(parts * 4);
  return w;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_BAD_ARG: return "MLA_ERR_BAD_ARG: a size is out of range or inconsistent";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: no kernel for this shape";
    case MLA_ERR_LAUNCH: return "MLA_ERR_LAUNCH: the HIP runtime rejected a launch";
    case MLA_ERR_TOO_LARGE:
      return "MLA_ERR_TOO_LARGE: the call needs more than the library's static scratch holds";
    default: return "unknown MLA status";
  }
}

int mla_rope_append(const mla_dims* dims, const mla_cache* cache, int32_t num_tokens, const int32_t* token_seq,
                    const int32_t* token_pos, const uint16_t* c_kv, const uint16_t* k_rope, uint16_t* q_rope_inout,
                    hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (num_tokens < 0) return MLA_ERR_BAD_ARG;
  if (num_tokens == 0) return MLA_OK;
  if (!token_seq || !token_pos || !c_kv || !k_rope) return MLA_ERR_NULL;
  if (!aligned(token_seq, 4) || !aligned(token_pos, 4) || !aligned(c_kv, 16) || !aligned(k_rope, 4) ||
      !aligned(q_rope_inout, 16))
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_rope_append(view(cache), dims->n_heads, num_tokens, token_seq, token_pos, c_kv, k_rope,
                                          q_rope_inout, dims->rope_theta, stream));
}

int mla_decode_merge_latent(const mla_dims* dims, int32_t batch, int32_t num_splits, const uint16_t* o_partial,
                            const float* lse_partial, uint16_t* o_lat, float* lse_out, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || num_splits < 1) return MLA_ERR_BAD_ARG;
  if (batch == 0) return MLA_OK;
  if (!o_partial || !lse_partial || !o_lat) return MLA_ERR_NULL;
  if (((uintptr_t)o_partial & 15) != 0 || ((uintptr_t)o_lat & 15) != 0) return MLA_ERR_BAD_ARG;
  return launched(mla::launch_merge_latent(batch, dims->n_heads, num_splits, o_partial, lse_partial, o_lat, lse_out,
                                           stream));
}

int mla_prepare_output_weight(const mla_dims* dims, int32_t dim, const uint16_t* w_o, uint16_t* w_o_prepared,
                              hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (dim <= 0) return MLA_ERR_BAD_ARG;
  if (dim % 64 != 0) return MLA_ERR_UNSUPPORTED;
  if (!w_o || !w_o_prepared) return MLA_ERR_NULL;
  if (((uintptr_t)w_o & 15) != 0 || ((uintptr_t)w_o_prepared & 15) != 0) return MLA_ERR_BAD_ARG;
  return launched(mla::launch_prepare_rows(dim, (int64_t)dims->n_heads * dims->d_v, w_o, w_o_prepared, stream));
}

int mla_fold_output_weights(const mla_dims* dims, int32_t dim, const uint16_t* w_o, const uint16_t* w_uv,
                            uint16_t* w_ov_prepared, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (dim <= 0) return MLA_ERR_BAD_ARG;
  if (dim % 64 != 0) return MLA_ERR_UNSUPPORTED;
  if (!w_o || !w_uv || !w_ov_prepared) return MLA_ERR_NULL;
  if (((uintptr_t)w_ov_prepared & 7) != 0) return MLA_ERR_BAD_ARG;
  return launched(mla::launch_fold_output_weights(dim, dims->n_heads, w_o, w_uv, w_ov_prepared, stream));
}

size_t mla_output_projection_workspace_size(const mla_dims* dims, int32_t num_tokens, int32_t dim, int32_t folded) {
  if (check_dims(dims) != MLA_OK || num_tokens < 0 || dim <= 0 || dim % 64 != 0) return 0;
  const int64_t K = (int64_t)dims->n_heads * (folded ? dims->d_c : dims->d_v);
  return mla::output_workspace_bytes(num_tokens, dim, K);
}

int mla_output_projection(const mla_dims* dims, int32_t num_tokens, int32_t dim, int32_t folded, const uint16_t* act,
                          const uint16_t* w_prepared, void* workspace, size_t workspace_bytes, uint16_t* y,
                          hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (num_tokens < 0 || num_tokens > 65535 * 32 || dim <= 0) return MLA_ERR_BAD_ARG;
  if (dim % 64 != 0) return MLA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MLA_OK;
  if (!act || !w_prepared || !workspace || !y) return MLA_ERR_NULL;
  const int64_t K = (int64_t)dims->n_heads * (folded ? dims->d_c : dims->d_v);
  if (workspace_bytes < mla::output_workspace_bytes(num_tokens, dim, K)) return MLA_ERR_BAD_ARG;
  if (((uintptr_t)workspace & 255) != 0 || ((uintptr_t)act & 15) != 0 || ((uintptr_t)w_prepared & 15) != 0 ||
      ((uintptr_t)y & 7) != 0)
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_output_gemm(num_tokens, dim, K, act, w_prepared, workspace, y, stream));
}

int mla_absorb_query_weights(const mla_dims* dims, int32_t q_rank, const uint16_t* w_uq, const uint16_t* w_uk,
                             uint16_t* w_q, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (q_rank <= 0) return MLA_ERR_BAD_ARG;
  if (q_rank % 64 != 0 || q_rank > 2048) return MLA_ERR_UNSUPPORTED;
  if (!w_uq || !w_uk || !w_q) return MLA_ERR_NULL;
  if (((uintptr_t)w_q & 7) != 0 || ((uintptr_t)w_uq & 7) != 0) return MLA_ERR_BAD_ARG;
  return launched(mla::launch_absorb_query_weights(dims->n_heads, q_rank, w_uq, w_uk, w_q, stream));
}

size_t mla_query_absorbed_workspace_size(const mla_dims* dims, int32_t num_tokens, int32_t dim, int32_t q_rank) {
  if (check_dims(dims) != MLA_OK || num_tokens < 0 || dim <= 0 || dim % 64 != 0 || q_rank <= 0 || q_rank % 64 != 0 ||
      q_rank > 2048)
    return 0;
  return mla::query_workspace_bytes(num_tokens, dim, q_rank);
}

int mla_query_absorbed(const mla_dims* dims, int32_t num_tokens, const int32_t* token_pos, const uint16_t* x,
                       int32_t dim, const uint16_t* w_dq, const uint16_t* gamma_q, float eps, int32_t q_rank,
                       const uint16_t* w_q, void* workspace, size_t workspace_bytes, uint16_t* q_abs,
                       hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (num_tokens < 0 || num_tokens > 65535 * 32 || dim <= 0 || q_rank <= 0) return MLA_ERR_BAD_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return MLA_ERR_BAD_ARG;
  if (dim % 64 != 0 || q_rank % 64 != 0 || q_rank > 2048) return MLA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MLA_OK;
  if (!token_pos || !x || !w_dq || !gamma_q || !w_q || !workspace || !q_abs) return MLA_ERR_NULL;
  if (workspace_bytes < mla::query_workspace_bytes(num_tokens, dim, q_rank)) return MLA_ERR_BAD_ARG;
  if (((uintptr_t)workspace & 255) != 0 || ((uintptr_t)x & 15) != 0 || ((uintptr_t)w_dq & 15) != 0 ||
      ((uintptr_t)w_q & 15) != 0 || ((uintptr_t)q_abs & 7) != 0)
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_query_absorbed(dims->n_heads, num_tokens, token_pos, x, dim, w_dq, gamma_q, eps, q_rank,
                                             w_q, dims->rope_theta, workspace, q_abs, stream));
}

size_t mla_chunked_prefill_expanded_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_seq_len) {
  if (check_dims(dims) != MLA_OK || batch < 0 || max_seq_len < 0) return 0;
  return mla::prefill_expanded_kv_bytes(batch, dims->n_heads, max_seq_len);
}

int mla_chunked_prefill_expanded(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                                 const int32_t* cu_q_lens, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                                 const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk,
                                 const uint16_t* w_uv, void* workspace, size_t workspace_bytes, uint16_t* out,
                                 float* lse_out, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (batch < 0 || total_q < 0 || max_q_len < 0 || max_seq_len < 0) return MLA_ERR_BAD_ARG;
  if (batch == 0 || total_q == 0) return MLA_OK;
  if (max_q_len < 1 || max_seq_len < max_q_len) return MLA_ERR_BAD_ARG;
  if (!seq_lens || !cu_q_lens || !q_nope || !q_rope || !w_uk || !w_uv || !workspace || !out) return MLA_ERR_NULL;
  if (workspace_bytes < mla::prefill_expanded_kv_bytes(batch, dims->n_heads, max_seq_len)) return MLA_ERR_BAD_ARG;
  if (((uintptr_t)workspace & 255) != 0 || ((uintptr_t)q_nope & 15) != 0 || ((uintptr_t)q_rope & 15) != 0 ||
      ((uintptr_t)out & 7) != 0)
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_prefill_expanded(view(cache), batch, dims->n_heads, seq_lens, cu_q_lens, max_q_len,
                                               max_seq_len, q_nope, q_rope, w_uk, w_uv, dims->scale, workspace, out,
                                               lse_out, stream));
}

size_t mla_kv_down_append_workspace_size(const mla_dims* dims, int32_t num_tokens, int32_t dim) {
  if (check_dims(dims) != MLA_OK || num_tokens < 0 || dim <= 0 || dim % 64 != 0) return 0;
  return mla::kv_down_workspace_bytes(num_tokens, dim);
}

int mla_kv_down_append(const mla_dims* dims, const mla_cache* cache, int32_t num_tokens, const int32_t* token_seq,
                       const int32_t* token_pos, const uint16_t* x, int32_t dim, const uint16_t* w_dkv,
                       const uint16_t* gamma, float eps, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (num_tokens < 0 || num_tokens > 65535 * 32 || dim <= 0) return MLA_ERR_BAD_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return MLA_ERR_BAD_ARG;
  if (dim % 64 != 0) return MLA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MLA_OK;
  if (!token_seq || !token_pos || !x || !w_dkv || !gamma || !workspace) return MLA_ERR_NULL;
  if (workspace_bytes < mla::kv_down_workspace_bytes(num_tokens, dim)) return MLA_ERR_BAD_ARG;
  if (((uintptr_t)workspace & 255) != 0 || ((uintptr_t)x & 15) != 0 || ((uintptr_t)w_dkv & 15) != 0)
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_kv_down(view(cache), num_tokens, token_seq, token_pos, x, dim, w_dkv, gamma, eps,
                                      dims->rope_theta, workspace, stream));
}

size_t mla_kv_down_query_absorbed_workspace_size(const mla_dims* dims, int32_t num_tokens, int32_t dim,
                                                 int32_t q_rank) {
  if (check_dims(dims) != MLA_OK || num_tokens < 0 || num_tokens > 65535 * 32 || dim <= 0 || dim % 64 != 0 ||
      q_rank <= 0 || q_rank % 64 != 0 || q_rank > 2048)
    return 0;
  return mla::kv_down_query_workspace_bytes(num_tokens, dim, q_rank);
}

int mla_kv_down_query_absorbed(const mla_dims* dims, const mla_cache* cache, int32_t num_tokens,
                               const int32_t* token_seq, const int32_t* token_pos, const uint16_t* x, int32_t dim,
                               const uint16_t* w_dkv, const uint16_t* gamma_kv, float eps_kv, const uint16_t* w_dq,
                               const uint16_t* gamma_q, float eps_q, int32_t q_rank, const uint16_t* w_q,
                               void* workspace, size_t workspace_bytes, uint16_t* q_abs, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (num_tokens < 0 || num_tokens > 65535 * 32 || dim <= 0 || q_rank <= 0) return MLA_ERR_BAD_ARG;
  if (!(eps_kv >= 0.f) || !isfinite(eps_kv) || !(eps_q >= 0.f) || !isfinite(eps_q)) return MLA_ERR_BAD_ARG;
  if (dim % 64 != 0 || q_rank % 64 != 0 || q_rank > 2048) return MLA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MLA_OK;
  if (!token_seq || !token_pos || !x || !w_dkv || !gamma_kv || !w_dq || !gamma_q || !w_q || !workspace || !q_abs)
    return MLA_ERR_NULL;
  if (workspace_bytes < mla::kv_down_query_workspace_bytes(num_tokens, dim, q_rank)) return MLA_ERR_BAD_ARG;
  if (!aligned(workspace, 256) || !aligned(x, 16) || !aligned(w_dkv, 16) || !aligned(w_dq, 16) ||
      !aligned(w_q, 16) || !aligned(q_abs, 8))
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_kv_down_query(view(cache), dims->n_heads, num_tokens, token_seq, token_pos, x, dim,
                                            w_dkv, gamma_kv, eps_kv, w_dq, gamma_q, eps_q, q_rank, w_q,
                                            dims->rope_theta, workspace, q_abs, stream));
}

int mla_check_inputs(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                     const int32_t* cu_q_lens, int32_t total_q, int32_t* error_word, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (batch < 0 || (cu_q_lens != nullptr && total_q < 0)) return MLA_ERR_BAD_ARG;
  if (!error_word || (batch > 0 && !seq_lens)) return MLA_ERR_NULL;
  if (!aligned(error_word, 4)) return MLA_ERR_BAD_ARG;
  return launched(mla::launch_check_inputs(batch, seq_lens, cache->block_table, cache->max_blocks_per_seq,
                                           cache->num_blocks, dims->block_size, cu_q_lens, total_q, error_word,
                                           stream));
}

int mla_decode_plan(const mla_dims* dims, int32_t batch, int32_t max_seq_len, int32_t num_cus,
                    int32_t* split_tokens, int32_t* num_splits) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!split_tokens || !num_splits) return MLA_ERR_NULL;
  if (batch <= 0 || max_seq_len < 0 || num_cus <= 0) return MLA_ERR_BAD_ARG;
  const int64_t bs = dims->block_size;
  const int64_t blocks = (max_seq_len + bs - 1) / bs;
  // enough splits per sequence that batch * splits covers every compute unit once
  int64_t per_seq = (num_cus + batch - 1) / batch;
  if (per_seq < 1) per_seq = 1;
  if (blocks > 0 && per_seq > blocks) per_seq = blocks;
  int64_t blocks_per_split = blocks > 0 ? (blocks + per_seq - 1) / per_seq : 1;
  int64_t tok = blocks_per_split * bs;
  int64_t ns = blocks > 0 ? (blocks + blocks_per_split - 1) / blocks_per_split : 1;
  if (tok > INT32_MAX || ns > 65535) return MLA_ERR_BAD_ARG;
  *split_tokens = (int32_t)tok;
  *num_splits = (int32_t)ns;
  return MLA_OK;
}

// Cost model of the two chunked-prefill forms on MI355X (rates measured with the benchmark at 2 x 1024
// new tokens after 8192: the absorbed attention sustains 1.15 PFLOP/s, the expanded form's
// up-projection 0.80 and its attention 0.91; the absorbed form's absorption and combine cost about
// 0.12 us per query row; each form about 20 us of launches). The absorbed attention runs one
// work-group per query row (per 128 heads) and split (prefill_splits), and counts whole waves of
// work-groups on the compute units; the expanded form up-projects every cached token in 256-token
// tiles and attends in 256-query tiles.
int mla_chunked_prefill_plan(const mla_dims* dims, int32_t batch, const int32_t* seq_lens, const int32_t* q_lens,
                             int32_t num_cus, int32_t* use_expanded, float* absorbed_us, float* expanded_us) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!use_expanded) return MLA_ERR_NULL;
  if (batch < 0 || num_cus <= 0) return MLA_ERR_BAD_ARG;
  if (batch > 0 && (!seq_lens || !q_lens)) return MLA_ERR_NULL;
  constexpr double kAbsorbedRate = 1.15e15, kUpRate = 0.80e15, kExpandedAttnRate = 0.91e15;
  constexpr double kPerRowUs = 0.12, kLaunchUs = 20.0;
  const double H = dims->n_heads;
  auto up256 = [](double x) { return ceil(x / 256.0) * 256.0; };
  double pairs = 0, pairs_tiles = 0, up_tokens = 0, rows = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const double L = seq_lens[b], q = q_lens[b];
    if (q < 0 || L < 0 || q > L) return MLA_ERR_BAD_ARG;
    if (q == 0) continue;
    pairs += q * (L - q) + q * (q + 1) / 2;          // visible (query, key) pairs under the causal rule
    pairs_tiles += up256(q) * (L - q) + up256(q) * up256(q) / 2;
    up_tokens += up256(L);
    rows += q;
  }
  const int groups = (mla::q_tiles(dims->n_heads) + 3) / 4;
  const double wg = rows * groups * prefill_splits(dims->n_heads, (int32_t)std::min(rows, (double)kMaxPrefillTokens));
  const double wave_factor = wg > 0 ? ceil(wg / num_cus) * num_cus / wg : 1.0;
  const double t_abs = pairs * H * 2 * (mla::kRow + mla::kDc) / kAbsorbedRate * 1e6 * wave_factor + kPerRowUs * rows +
                       kLaunchUs;
  const double t_exp = up_tokens * H * 2 * 256 * mla::kDc / kUpRate * 1e6 +
                       pairs_tiles * H * 2 * (mla::kDnope + mla::kDr + mla::kDv) / kExpandedAttnRate * 1e6 + kLaunchUs;
  *use_expanded = t_exp < t_abs ? 1 : 0;
  if (absorbed_us) *absorbed_us = (float)t_abs;
  if (expanded_us) *expanded_us = (float)t_exp;
  return MLA_OK;
}

size_t mla_decode_workspace_size(const mla_dims* dims, int32_t batch) {
  if (check_dims(dims) != MLA_OK || batch < 0) return 0;
  return align256((size_t)batch * mla::q_tiles(dims->n_heads) * mla::kQTileElems * 2);
}

int mla_absorb(const mla_dims* dims, int32_t rows, const uint16_t* q_nope, const uint16_t* q_rope,
               const uint16_t* w_uk, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (rows < 0 || rows > 65535 * 128) return MLA_ERR_BAD_ARG;
  if (rows == 0) return MLA_OK;
  if (!q_nope || !q_rope || !w_uk || !workspace) return MLA_ERR_NULL;
  if (workspace_bytes < mla_decode_workspace_size(dims, rows)) return MLA_ERR_BAD_ARG;
  if (!aligned(workspace, 256) || !aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk, 16))
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_absorb(rows, dims->n_heads, q_nope, q_rope, w_uk, static_cast<uint16_t*>(workspace),
                                     false, stream));
}

int mla_rope_append_absorb(const mla_dims* dims, const mla_cache* cache, int32_t num_tokens, const int32_t* token_seq,
                           const int32_t* token_pos, const uint16_t* c_kv, const uint16_t* k_rope,
                           uint16_t* q_rope_inout, const uint16_t* q_nope, const uint16_t* w_uk, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (num_tokens < 0 || num_tokens > 65535 * 128) return MLA_ERR_BAD_ARG;
  if (num_tokens == 0) return MLA_OK;
  if (!token_seq || !token_pos || !c_kv || !k_rope || !q_rope_inout || !q_nope || !w_uk || !workspace)
    return MLA_ERR_NULL;
  if (workspace_bytes < mla_decode_workspace_size(dims, num_tokens)) return MLA_ERR_BAD_ARG;
  if (!aligned(workspace, 256) || !aligned(token_seq, 4) || !aligned(token_pos, 4) || !aligned(c_kv, 16) ||
      !aligned(k_rope, 4) || !aligned(q_rope_inout, 16) || !aligned(q_nope, 16) || !aligned(w_uk, 16))
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_rope_absorb(view(cache), dims->n_heads, num_tokens, token_seq, token_pos, c_kv, k_rope,
                                          q_rope_inout, dims->rope_theta, q_nope, w_uk,
                                          static_cast<uint16_t*>(workspace), stream));
}

int mla_decode_attend(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                      const void* workspace, size_t workspace_bytes, int32_t split_tokens, int32_t num_splits,
                      uint16_t* o_partial, float* lse_partial, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if ((st = check_splits(dims, batch, split_tokens, num_splits)) != MLA_OK) return st;
  if (batch == 0) return MLA_OK;
  if (!seq_lens || !workspace || !o_partial || !lse_partial) return MLA_ERR_NULL;
  if (workspace_bytes < mla_decode_workspace_size(dims, batch)) return MLA_ERR_BAD_ARG;
  if (!aligned(workspace, 256) || !aligned(seq_lens, 4) || !aligned(o_partial, 16) || !aligned(lse_partial, 4))
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_attention(view(cache), batch, dims->n_heads, seq_lens, nullptr, batch,
                                        static_cast<const uint16_t*>(workspace), true, dims->scale, split_tokens,
                                        num_splits, o_partial, lse_partial, stream));
}

int mla_decode(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
               const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk, int32_t split_tokens,
               int32_t num_splits, void* workspace, size_t workspace_bytes, uint16_t* o_partial, float* lse_partial,
               hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if ((st = check_splits(dims, batch, split_tokens, num_splits)) != MLA_OK) return st;
  if (batch == 0) return MLA_OK;
  if (!seq_lens || !q_nope || !q_rope || !w_uk || !workspace || !o_partial || !lse_partial) return MLA_ERR_NULL;
  if (workspace_bytes < mla_decode_workspace_size(dims, batch)) return MLA_ERR_BAD_ARG;
  if (!aligned(workspace, 256) || !aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk, 16) ||
      !aligned(seq_lens, 4) || !aligned(o_partial, 16) || !aligned(lse_partial, 4))
    return MLA_ERR_BAD_ARG;
  st = mla_absorb(dims, batch, q_nope, q_rope, w_uk, workspace, workspace_bytes, stream);
  if (st != MLA_OK) return st;
  return mla_decode_attend(dims, cache, batch, seq_lens, workspace, workspace_bytes, split_tokens, num_splits,
                           o_partial, lse_partial, stream);
}

int mla_decode_no_alloc(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                        const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk, int32_t split_tokens,
                        int32_t num_splits, uint16_t* o_partial, float* lse_partial, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if ((st = check_splits(dims, batch, split_tokens, num_splits)) != MLA_OK) return st;
  if (batch == 0) return MLA_OK;
  if (!seq_lens || !q_nope || !q_rope || !w_uk || !o_partial || !lse_partial) return MLA_ERR_NULL;
  if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk, 16) || !aligned(seq_lens, 4) ||
      !aligned(o_partial, 16) || !aligned(lse_partial, 4))
    return MLA_ERR_BAD_ARG;
  const size_t need = mla_decode_workspace_size(dims, batch);
  if (need > (size_t)MLA_NO_ALLOC_SCRATCH_BYTES) return MLA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (device_scratch(&ws) != hipSuccess) return MLA_ERR_LAUNCH;
  // the absorbed query rows of every head tile are written before the attention reads them (padding
  // heads as zeros), so nothing left in the scratch by an earlier call is read
  hipError_t e = mla::launch_absorb(batch, dims->n_heads, q_nope, q_rope, w_uk, static_cast<uint16_t*>(ws), false,
                                    stream);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  return launched(mla::launch_attention(view(cache), batch, dims->n_heads, seq_lens, nullptr, batch,
                                        static_cast<const uint16_t*>(ws), true, dims->scale, split_tokens, num_splits,
                                        o_partial, lse_partial, stream));
}

int mla_decode_absorbed(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                        const uint16_t* q_abs, int32_t split_tokens, int32_t num_splits, uint16_t* o_partial,
                        float* lse_partial, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if ((st = check_splits(dims, batch, split_tokens, num_splits)) != MLA_OK) return st;
  if (batch == 0) return MLA_OK;
  if (!seq_lens || !q_abs || !o_partial || !lse_partial) return MLA_ERR_NULL;
  if (!aligned(seq_lens, 4) || !aligned(q_abs, 16) || !aligned(o_partial, 16) || !aligned(lse_partial, 4))
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_attention(view(cache), batch, dims->n_heads, seq_lens, nullptr, batch, q_abs, false,
                                        dims->scale, split_tokens, num_splits, o_partial, lse_partial, stream));
}

int mla_decode_combine(const mla_dims* dims, int32_t batch, int32_t num_splits, const uint16_t* o_partial,
                       const float* lse_partial, const uint16_t* w_uv, uint16_t* out, float* lse_out,
                       hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || num_splits <= 0 || num_splits > 65535) return MLA_ERR_BAD_ARG;
  if (batch == 0) return MLA_OK;
  if (!o_partial || !lse_partial || !w_uv || !out) return MLA_ERR_NULL;
  if (!aligned(o_partial, 16) || !aligned(lse_partial, 4) || !aligned(w_uv, 16) || !aligned(out, 8) ||
      !aligned(lse_out, 4))
    return MLA_ERR_BAD_ARG;
  return launched(mla::launch_combine(batch, dims->n_heads, num_splits, o_partial, lse_partial, w_uv, out, lse_out,
                                      stream));
}

size_t mla_chunked_prefill_workspace_size(const mla_dims* dims, int32_t total_q) {
  if (check_dims(dims) != MLA_OK || total_q < 0) return 0;
  return prefill_layout(dims, total_q).total;
}

int mla_chunked_prefill(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                        const int32_t* cu_q_lens, int32_t total_q, int32_t max_q_len, const uint16_t* q_nope,
                        const uint16_t* q_rope, const uint16_t* w_uk, const uint16_t* w_uv, void* workspace,
                        size_t workspace_bytes, uint16_t* out, float* lse_out, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  // one attention work-group per (query token, group of 128 heads): the grid stays far below 2^31
  if (batch < 0 || total_q < 0 || max_q_len < 0 || total_q > kMaxPrefillTokens) return MLA_ERR_BAD_ARG;
  if (batch == 0 || total_q == 0) return MLA_OK;
  if (!seq_lens || !cu_q_lens || !q_nope || !q_rope || !w_uk || !w_uv || !workspace || !out) return MLA_ERR_NULL;
  PrefillWorkspace lay = prefill_layout(dims, total_q);
  if (workspace_bytes < lay.total) return MLA_ERR_BAD_ARG;
  if (!aligned(workspace, 256) || !aligned(seq_lens, 4) || !aligned(cu_q_lens, 4) || !aligned(q_nope, 16) ||
      !aligned(q_rope, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16) || !aligned(out, 8) || !aligned(lse_out, 4))
    return MLA_ERR_BAD_ARG;
  char* ws = static_cast<char*>(workspace);
  uint16_t* q_abs = reinterpret_cast<uint16_t*>(ws + lay.q_abs);
  uint16_t* o_lat = reinterpret_cast<uint16_t*>(ws + lay.o_lat);
  float* lse = reinterpret_cast<float*>(ws + lay.lse);
  // many rows: the absorbed queries in the plain layout, which the absorption writes in whole lines
  hipError_t e = mla::launch_absorb(total_q, dims->n_heads, q_nope, q_rope, w_uk, q_abs, true, stream);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  // one query token per row. With enough rows the whole causal key range of a row is one split
  // (split_tokens only bounds a split, so the largest block multiple covers any sequence). With few
  // rows the range is cut into prefill_splits pieces of the descriptor's capacity (max_blocks_per_seq
  // blocks bound every length), each a block multiple; splits past a row's length stay empty.
  (void)max_q_len;
  int32_t split_tokens = kMaxSplitTokens, num_splits = 1;
  const int splits = prefill_splits(dims->n_heads, total_q);
  const int64_t cap = (int64_t)cache->max_blocks_per_seq * dims->block_size;
  if (splits > 1 && cap <= ((int64_t)1 << 30)) {
    const int64_t bs = dims->block_size;
    split_tokens = (int32_t)(((cap + splits - 1) / splits + bs - 1) / bs * bs);
    num_splits = (int32_t)((cap + split_tokens - 1) / split_tokens);  // <= splits
  }
  e = mla::launch_attention(view(cache), total_q, dims->n_heads, seq_lens, cu_q_lens, batch, q_abs, false, dims->scale,
                            split_tokens, num_splits, o_lat, lse, stream);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  return launched(mla::launch_combine(total_q, dims->n_heads, num_splits, o_lat, lse, w_uv, out, lse_out, stream));
}

}  // extern "C"
