/*
 * mla.h - C ABI of the weight-absorbed Multi-Head Latent Attention (MLA) library for gfx950.
 *
 * The library computes MLA decode and chunked prefill over a paged, compressed latent KV
 * cache in which each token keeps one row [c_KV (d_c) | k_R (d_rope)] shared by all heads.
 * Per head, q_nope is absorbed through W_UK into the latent space, scored against the row
 * together with the decoupled-RoPE query, the softmax weights reduce c_KV, and the reduced
 * latent is up-projected through W_UV.
 *
 * Sources (page title, section):
 *   "论文复现工坊 No.4：从零复现 DeepSeek-V2/V3 多头潜在注意力 MLA" (m.xxqk.cn), sections 1, 2, 4:
 *       latent c_KV cached with a decoupled RoPE key; the module's shapes and its scale
 *       1/sqrt(qk_nope_head_dim + qk_rope_head_dim); Q_absorbed = Q W_UK^T scored against c^KV.
 *   "淺析DeepSeek多頭潛在注意力機制（MLA）" (itdecent.cn), "大模型的整體推理過程",
 *       "MLA的數學原理", "MLA與ROPE的融合": decode appends the new token then attends over
 *       all cached tokens; x_t (W_q W_k^T) c_i^T; RoPE angle theta_i = 10000^(-2i/d) and a
 *       RoPE key shared by all heads.
 *   "Multi-Head Latent Attention: DeepSeek V2/V3 工程视角" (xuquant.com), section 一:
 *       n_h = 128, d_c = 512, d_h^R = 64, 576 cached elements per token per layer.
 *   "Multi-Head Latent Attention（MLA）原理与工程实践全解析" (cnnetsun.cn), section 3.3:
 *       flattened [batch, seq, latent] cache rows and block-managed (paged) storage.
 *
 * Conventions for every entry point:
 *   - Every tensor pointer is a DEVICE pointer; bf16 values are passed as uint16_t bit patterns;
 *     all integer tables are int32. The caller owns every buffer; the library allocates nothing,
 *     keeps no state between calls and never synchronises.
 *   - Work is enqueued on `stream` and runs asynchronously. Calls are safe to capture in a graph.
 *   - Arguments are validated on the host before any HIP call. A call returns MLA_OK (0) or a
 *     negative status; on an error nothing has been enqueued (except MLA_ERR_LAUNCH, reported
 *     after a launch failed).
 *   - Contents of device buffers are a caller contract that the host cannot check: block ids
 *     must lie in [0, num_blocks), every seq_len must satisfy
 *     0 <= seq_len <= max_blocks_per_seq * block_size, positions must be < seq_len.
 *   - Supported shapes: d_c = 512, d_rope = 64, d_nope = 128, d_v = 128, block_size = 64,
 *     n_heads a positive multiple of 16. Others return MLA_ERR_UNSUPPORTED.
 *   - Alignment (checked on the host; a misaligned pointer returns MLA_ERR_BAD_ARG before any HIP
 *     call): the kernels move bf16 tensors in 16-byte pieces, so unless an entry point states
 *     otherwise every bf16 tensor pointer (cache data, c_kv, q_nope, q_rope, q_abs, w_uk, w_uv,
 *     o_partial) must be 16-byte aligned, bf16 outputs of d_v elements per row (out) 8-byte
 *     aligned, int32 and fp32 pointers 4-byte aligned, k_rope 4-byte aligned, and workspaces
 *     256-byte aligned. Optional pointers that are NULL are not checked.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OK 0
#define MLA_ERR_NULL (-1)        /* a required pointer is NULL */
#define MLA_ERR_BAD_ARG (-2)     /* a size is negative, zero where it must be positive, or inconsistent */
#define MLA_ERR_UNSUPPORTED (-3) /* a shape this library has no kernel for */
#define MLA_ERR_LAUNCH (-4)      /* the HIP runtime reported an error for a launch */
#define MLA_ERR_TOO_LARGE (-5)   /* mla_decode_no_alloc: the call needs more than the static scratch holds */

/* Bits of the error word mla_check_inputs writes (0: no rule broken). */
#define MLA_CHECK_BAD_LENGTH 1      /* a seq_lens entry < 0 or > max_blocks_per_seq * block_size */
#define MLA_CHECK_BAD_BLOCK 2       /* a block a sequence uses (logical block < ceil(len / block_size)) is
                                       outside [0, num_blocks) */
#define MLA_CHECK_BAD_OFFSETS 4     /* cu_q_lens is not 0 = cu[0] <= cu[1] <= ... <= cu[batch] = total_q */
#define MLA_CHECK_CHUNK_TOO_LONG 8  /* a chunk has more new tokens than its sequence has tokens */

/* Bytes of the static device scratch of mla_decode_no_alloc (one array per GPU, kept until exit). */
#define MLA_NO_ALLOC_SCRATCH_BYTES (16u << 20)

/* Model dimensions ("论文复现工坊 No.4", section 2: the module's constructor arguments). */
typedef struct mla_dims {
  int32_t n_heads;    /* query heads n_h; multiple of 16 */
  int32_t d_c;        /* latent width (kv_lora_rank), 512 */
  int32_t d_rope;     /* decoupled RoPE width (qk_rope_head_dim), 64 */
  int32_t d_nope;     /* per-head non-RoPE query/key width (qk_nope_head_dim), 128 */
  int32_t d_v;        /* per-head value width (v_head_dim), 128 */
  int32_t block_size; /* tokens per cache block, 64 */
  float scale;        /* softmax scale, normally 1/sqrt(d_nope + d_rope); must be finite and > 0 */
  float rope_theta;   /* RoPE base, normally 10000; must be > 1 */
} mla_dims;

/* Paged latent cache (data 16-byte aligned, block_table 4-byte aligned). Row of token t of sequence b lives at
 *   data + ((int64)phys * block_size + t % block_size) * (d_c + d_rope),
 *   phys = block_table[b * max_blocks_per_seq + t / block_size]   (paged), or
 *   phys = b * max_blocks_per_seq + t / block_size                 (block_table == NULL: contiguous).
 * A row is [c_KV (d_c) | k_R rotated at t (d_rope)], bf16, 1152 bytes at the supported shape. */
typedef struct mla_cache {
  uint16_t* data;             /* [num_blocks, block_size, d_c + d_rope] bf16 */
  int64_t num_blocks;         /* > 0 */
  const int32_t* block_table; /* [batch, max_blocks_per_seq] int32, or NULL */
  int32_t max_blocks_per_seq; /* > 0 */
} mla_cache;

/* Human-readable name of a status code (static storage, never NULL). */
const char* mla_status_string(int status);

/* ---------------------------------------------------------------------------------------------
 * mla_rope_append - rotate the decoupled RoPE key and query of new tokens and append the keys.
 * ("淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA與ROPE的融合"; "论文复现工坊 No.4", sections 1-2.)
 *
 * For each new token i (0 <= i < num_tokens) of sequence token_seq[i] at position p = token_pos[i]:
 *   row = [c_kv[i] | R_p k_rope[i]] is written to the cache slot of (token_seq[i], p);
 *   if q_rope_inout != NULL, q_rope_inout[i, h, :] = R_p q_rope_inout[i, h, :] for every head h.
 * R_p turns each interleaved pair (x_{2j}, x_{2j+1}) by p * rope_theta^(-2j/d_rope), computed in
 * fp64 and rounded to bf16 (round-to-nearest-even).
 *   c_kv         [num_tokens, d_c] bf16, k_rope [num_tokens, d_rope] bf16 (not rotated)
 *   token_seq    [num_tokens] int32 in [0, batch of the table)
 *   token_pos    [num_tokens] int32 >= 0
 *   q_rope_inout [num_tokens, n_heads, d_rope] bf16, rotated in place (may be NULL)
 * Two new tokens must not map to the same slot. num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------------------------- */
int mla_rope_append(const mla_dims* dims, const mla_cache* cache, int32_t num_tokens,
                    const int32_t* token_seq, const int32_t* token_pos, const uint16_t* c_kv,
                    const uint16_t* k_rope, uint16_t* q_rope_inout, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_kv_down_append - the KV down-projection of new tokens, fused with mla_rope_append's rotation
 * and append ("论文复现工坊 No.4", section 2: kv_combined = wkv_a(x), split into the latent part and
 * the decoupled RoPE key, the latent part through kv_norm; section 4: that RMSNorm follows the W_DKV
 * projection).
 * For each new token i: kv = x[i] . W_DKV^T (fp32 accumulation, rounded to bf16);
 *   c_KV = bf16(kv[0:d_c] / sqrt(mean(kv[0:d_c]^2) + eps) * gamma);  k_R = kv[d_c:d_c+d_rope];
 *   then the row [c_KV | R_p k_R] goes to the slot of (token_seq[i], token_pos[i]) exactly as
 *   mla_rope_append writes it (no query).
 *   x      [num_tokens, dim] bf16;  dim a positive multiple of 64 (else MLA_ERR_UNSUPPORTED)
 *   w_dkv  [d_c + d_rope, dim] bf16 (the nn.Linear row layout of wkv_a)
 *   gamma  [d_c] bf16 (kv_norm's weight);  eps >= 0 (finite)
 *   workspace >= mla_kv_down_append_workspace_size(dims, num_tokens, dim) bytes (fp32 partial sums
 *   over splits of the input dimension), 256-byte aligned
 *   x and w_dkv 16-byte aligned; num_tokens <= 2097120
 * Errors: MLA_ERR_NULL for a missing pointer, MLA_ERR_BAD_ARG for a negative count, a bad eps, a
 * small or misaligned buffer, MLA_ERR_UNSUPPORTED for dim % 64 != 0. The workspace size query
 * returns 0 for arguments the call would reject.
 * Two launches on `stream`; num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------------------------- */
size_t mla_kv_down_append_workspace_size(const mla_dims* dims, int32_t num_tokens, int32_t dim);
int mla_kv_down_append(const mla_dims* dims, const mla_cache* cache, int32_t num_tokens, const int32_t* token_seq,
                       const int32_t* token_pos, const uint16_t* x, int32_t dim, const uint16_t* w_dkv,
                       const uint16_t* gamma, float eps, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Split planning for decode (host only, no HIP call).
 * Chooses split_tokens (a multiple of block_size) and num_splits = ceil(max_seq_len / split_tokens)
 * so that batch * num_splits work-groups fill `num_cus` compute units. Returns MLA_OK or an error.
 * ------------------------------------------------------------------------------------------- */
int mla_decode_plan(const mla_dims* dims, int32_t batch, int32_t max_seq_len, int32_t num_cus,
                    int32_t* split_tokens, int32_t* num_splits);

/* Bytes of device workspace mla_decode needs for `batch` sequences (the absorbed queries). */
size_t mla_decode_workspace_size(const mla_dims* dims, int32_t batch);

/* ---------------------------------------------------------------------------------------------
 * mla_decode - absorbed decode attention, split over the key axis (one query token per sequence).
 * ("论文复现工坊 No.4", sections 2 and 4; "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA的數學原理",
 *  "大模型的整體推理過程": the query is the sequence's last token and sees all seq_len tokens.)
 *
 * For sequence b with L = seq_lens[b] cached tokens, every head h and split s (tokens
 * [s*split_tokens, min((s+1)*split_tokens, L))):
 *   q_abs[h]    = W_UK[h]^T q_nope[b, h]                   (d_c, rounded to bf16)
 *   s_t         = scale * (q_abs[h] . c_t + q_rope[b, h] . kR_t)
 *   lse_partial[b, h, s] = ln sum_t exp(s_t)                (-inf for an empty split)
 *   o_partial[b, h, s, :] = sum_t exp(s_t - lse_partial) c_t  (rounded to bf16; 0 for an empty split)
 *   seq_lens     [batch] int32, 0 <= L <= num_splits * split_tokens
 *   q_nope       [batch, n_heads, d_nope] bf16
 *   q_rope       [batch, n_heads, d_rope] bf16, already rotated at position L-1
 *   w_uk         [n_heads, d_nope, d_c] bf16 (row d of head h maps c to the key's element d)
 *   split_tokens multiple of block_size, > 0; num_splits > 0
 *   workspace    >= mla_decode_workspace_size(dims, batch) bytes, 256-byte aligned
 *   o_partial    [batch, n_heads, num_splits, d_c] bf16 (a softmax-weighted mean of c rows)
 *   lse_partial  [batch, n_heads, num_splits] fp32
 * ------------------------------------------------------------------------------------------- */
int mla_decode(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
               const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk,
               int32_t split_tokens, int32_t num_splits, void* workspace, size_t workspace_bytes,
               uint16_t* o_partial, float* lse_partial, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_decode_no_alloc - mla_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. It computes exactly what
 * mla_decode computes (same kernels, same outputs bit for bit) but takes no workspace: the absorbed
 * queries go to a static device array of MLA_NO_ALLOC_SCRATCH_BYTES (16 MiB) that the library holds
 * on each GPU it runs on until the process ends. Nothing is allocated and nothing is freed; the
 * array's device address is looked up (hipGetSymbolAddress) on the first call on each device, with
 * the call's device current (the stream must belong to the current device).
 *   Arguments as mla_decode, without workspace / workspace_bytes.
 *   Limit: mla_decode_workspace_size(dims, batch) <= MLA_NO_ALLOC_SCRATCH_BYTES, i.e. batch <= 113 at
 *   n_heads = 128 (147,456 bytes per row); beyond it MLA_ERR_TOO_LARGE, before any HIP call.
 *   All calls on one GPU share its array: calls that overlap on one GPU (different streams, or host
 *   threads racing on one stream's enqueue order) race on it and must be serialised by the caller.
 *   The array keeps the last call's contents; every call writes all the scratch it later reads.
 * ------------------------------------------------------------------------------------------- */
int mla_decode_no_alloc(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                        const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk, int32_t split_tokens,
                        int32_t num_splits, uint16_t* o_partial, float* lse_partial, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_absorb / mla_decode_attend - the two halves of mla_decode, for callers that schedule or time
 * them apart ("论文复现工坊 No.4", section 4: the absorption Q W_UK^T is a step of its own before
 * scoring against c^KV).
 *   mla_absorb(rows): q_abs[r, h] = [W_UK[h]^T q_nope[r, h] (d_c, bf16) | q_rope[r, h]] for r < rows,
 *     written to `workspace` in the library's internal operand order (opaque to the caller);
 *     q_nope [rows, n_heads, d_nope], q_rope [rows, n_heads, d_rope] bf16; w_uk as for mla_decode;
 *     workspace >= mla_decode_workspace_size(dims, rows) bytes, 256-byte aligned.
 *   mla_decode_attend(batch): mla_decode's attention and outputs, reading the queries that
 *     mla_absorb(rows = batch) left in `workspace` (same dims, same workspace).
 * mla_absorb followed by mla_decode_attend on one stream computes exactly what mla_decode does.
 * ------------------------------------------------------------------------------------------- */
int mla_absorb(const mla_dims* dims, int32_t rows, const uint16_t* q_nope, const uint16_t* q_rope,
               const uint16_t* w_uk, void* workspace, size_t workspace_bytes, hipStream_t stream);

int mla_decode_attend(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                      const void* workspace, size_t workspace_bytes, int32_t split_tokens, int32_t num_splits,
                      uint16_t* o_partial, float* lse_partial, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_rope_append_absorb - mla_rope_append of new tokens followed by mla_absorb of the same tokens,
 * in one launch (the step's front half: "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA與ROPE的融合"
 * rotates the decoupled key and query; "论文复现工坊 No.4", section 4 absorbs W_UK into the query).
 * Row i of the absorption is token i (decode: one new token per sequence, token i of sequence i):
 *   cache, token_seq, token_pos, c_kv, k_rope  as for mla_rope_append
 *   q_rope_inout [num_tokens, n_heads, d_rope] bf16, rotated in place (required here)
 *   q_nope       [num_tokens, n_heads, d_nope] bf16;  w_uk as for mla_decode
 *   workspace    >= mla_decode_workspace_size(dims, num_tokens) bytes, 256-byte aligned; afterwards it
 *                holds what mla_absorb(rows = num_tokens) on the rotated queries leaves there, bit for bit
 * The cache, q_rope_inout and workspace end up exactly as after mla_rope_append then mla_absorb.
 * ------------------------------------------------------------------------------------------- */
int mla_rope_append_absorb(const mla_dims* dims, const mla_cache* cache, int32_t num_tokens,
                           const int32_t* token_seq, const int32_t* token_pos, const uint16_t* c_kv,
                           const uint16_t* k_rope, uint16_t* q_rope_inout, const uint16_t* q_nope,
                           const uint16_t* w_uk, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_decode_absorbed - mla_decode for callers that already hold the absorbed queries, e.g. with
 * W_UK folded into the query up-projection ahead of time ("淺析DeepSeek多頭潛在注意力機制（MLA）",
 * "MLA的數學原理": x_t (W_q W_k^T) is one precomputable product).
 *   q_abs  [batch, n_heads, d_c + d_rope] bf16; row = [W_UK[h]^T q_nope (d_c) | q_R rotated at L-1]
 * Everything else (split rule, outputs, empty splits, contracts) is exactly as for mla_decode;
 * no workspace is needed.
 * ------------------------------------------------------------------------------------------- */
int mla_decode_absorbed(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                        const uint16_t* q_abs, int32_t split_tokens, int32_t num_splits, uint16_t* o_partial,
                        float* lse_partial, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_decode_combine - log-sum-exp merge of the split partials and the W_UV up-projection.
 * ("论文复现工坊 No.4", section 1: no K or V tensor is ever expanded; the value side is
 *  W_UV applied after the latent reduction.)
 *   lse[b,h]   = ln sum_s exp(lse_partial[b,h,s])        (-inf if every split is empty)
 *   o_lat      = sum_s exp(lse_partial[b,h,s] - lse[b,h]) o_partial[b,h,s,:]   (fp32 accumulation)
 *   out[b,h,:] = W_UV[h] o_lat                             (bf16; 0 if every split is empty)
 *   w_uv    [n_heads, d_v, d_c] bf16;  out [batch, n_heads, d_v] bf16
 *   lse_out [batch, n_heads] fp32, natural log (may be NULL)
 * ------------------------------------------------------------------------------------------- */
int mla_decode_combine(const mla_dims* dims, int32_t batch, int32_t num_splits, const uint16_t* o_partial,
                       const float* lse_partial, const uint16_t* w_uv, uint16_t* out, float* lse_out,
                       hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_chunked_prefill_plan - which form of the causal chunked prefill is expected to be faster on
 * MI355X (host only, no HIP call): mla_chunked_prefill (absorbed: 2 (d_c + d_rope) + 2 d_c multiply-adds
 * per visible (query, key) pair and head) or mla_chunked_prefill_expanded (every cached token
 * up-projected through W_UK and W_UV, then 2 (d_nope + d_rope) + 2 d_v per pair and head)
 * ("Multi-Head Latent Attention: DeepSeek V2/V3 工程视角" names the two ways). A cost model with rates
 * measured on MI355X; short chunks over a long prefix favour the absorbed form, long chunks the
 * expanded one (at 8192 cached tokens the two meet at about 256 new tokens per sequence).
 *   seq_lens, q_lens  HOST arrays [batch]: cached tokens (chunk included) and chunk lengths, 0 <= q <= L
 *   num_cus           compute units (256 on MI355X)
 *   use_expanded      out: 1 if the expanded form is expected faster, else 0
 *   absorbed_us, expanded_us  out (may be NULL): the model's estimates in microseconds
 * ------------------------------------------------------------------------------------------- */
int mla_chunked_prefill_plan(const mla_dims* dims, int32_t batch, const int32_t* seq_lens, const int32_t* q_lens,
                             int32_t num_cus, int32_t* use_expanded, float* absorbed_us, float* expanded_us);

/* Bytes of device workspace mla_chunked_prefill needs for `total_q` query tokens. */
size_t mla_chunked_prefill_workspace_size(const mla_dims* dims, int32_t total_q);

/* ---------------------------------------------------------------------------------------------
 * mla_chunked_prefill - causal attention of a chunk of new tokens, absorbed form.
 * ("淺析DeepSeek多頭潛在注意力機制（MLA）", "大模型的整體推理過程": masked self-attention over
 *  the prompt; the same absorbed scores and latent reduction as decode.)
 * Query j of sequence b (cu_q_lens[b] <= j < cu_q_lens[b+1]) sits at position
 *   p = seq_lens[b] - (cu_q_lens[b+1] - cu_q_lens[b]) + (j - cu_q_lens[b])
 * and attends to cached tokens 0..p (the chunk must already be appended):
 *   out[j, h, :] = W_UV[h] sum_{t<=p} softmax_t(scale (q_abs . c_t + q_rope[j,h] . kR_t)) c_t
 *   seq_lens  [batch] int32 (tokens cached, chunk included); cu_q_lens [batch+1] int32, cu_q_lens[0] = 0,
 *             cu_q_lens[batch] = total_q, each chunk length <= max_q_len and <= its seq_len
 *   q_nope    [total_q, n_heads, d_nope] bf16;  q_rope [total_q, n_heads, d_rope] bf16 rotated at p
 *   w_uk, w_uv as for decode;  out [total_q, n_heads, d_v] bf16;  lse_out [total_q, n_heads] fp32 or NULL
 *   workspace >= mla_chunked_prefill_workspace_size(dims, total_q) bytes, 256-byte aligned
 *   total_q <= 16777216; q_nope, q_rope, w_uk, w_uv 16-byte aligned, out 8-byte aligned
 * Three launches (absorption, attention, combine with W_UV). With fewer than 256 (query row,
 * 128-head group) pairs the attention splits each row's keys into up to 8 pieces of the cache
 * descriptor's capacity (max_blocks_per_seq * block_size, rounded to blocks) so the work covers more
 * compute units, and the combine merges them; the workspace size accounts for it.
 * ------------------------------------------------------------------------------------------- */
int mla_chunked_prefill(const mla_dims* dims, const mla_cache* cache, int32_t batch,
                        const int32_t* seq_lens, const int32_t* cu_q_lens, int32_t total_q,
                        int32_t max_q_len, const uint16_t* q_nope, const uint16_t* q_rope,
                        const uint16_t* w_uk, const uint16_t* w_uv, void* workspace,
                        size_t workspace_bytes, uint16_t* out, float* lse_out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * The output side ("论文复现工坊 No.4", section 2: the heads' outputs [n_heads, d_v] flattened
 * head-major and projected by wo; section 4's absorption taken on the value side: W_UV folded into
 * wo, so decode hands the merged latent straight to the output GEMM).
 *
 * mla_decode_merge_latent - the log-sum-exp merge of mla_decode_combine without W_UV:
 *   o_lat[b, h] = sum_s exp(lse_s - lse*) o_partial[b, h, s] / sum_s exp(lse_s - lse*)  (bf16, 512 wide),
 *   lse_out[b, h] = lse* (or NULL); a row whose splits are all empty gives zeros and -inf.
 *   o_partial, lse_partial as written by mla_decode_attend; o_lat [batch, n_heads, 512] bf16;
 *   o_partial and o_lat 16-byte aligned.
 * mla_prepare_output_weight - wo's weight W_O [dim, n_heads d_v] (row-major, bf16) copied into MFMA
 *   operand order: row n, element k at (((n / 32) (K / 16) + k / 16) 64 + n % 32 + 32 ((k / 8) % 2)) 8
 *   + k % 8 with K = n_heads d_v (16-byte aligned buffers).
 * mla_fold_output_weights - W_OV[:, h d_c:(h+1) d_c] = W_O[:, h d_v:(h+1) d_v] W_UV[h] (fp32 sums, one
 *   rounding), [dim, n_heads d_c] in the same operand order with K = n_heads d_c (w_ov 8-byte aligned).
 * mla_output_projection - y [num_tokens, dim] bf16 = act W^T, W the prepared weight:
 *   folded = 0: act = the attention output [num_tokens, n_heads, d_v] (mla_decode_combine's out),
 *               W = mla_prepare_output_weight's;  y = wo(out)
 *   folded = 1: act = o_lat [num_tokens, n_heads, d_c] (mla_decode_merge_latent's), W = W_OV
 *   fp32 partial sums over splits of K in the workspace (>= mla_output_projection_workspace_size
 *   bytes, 256-byte aligned), one rounding; act and W 16-byte aligned, y 8-byte aligned.
 * dim must be a positive multiple of 64 (else MLA_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------------------------- */
int mla_decode_merge_latent(const mla_dims* dims, int32_t batch, int32_t num_splits, const uint16_t* o_partial,
                            const float* lse_partial, uint16_t* o_lat, float* lse_out, hipStream_t stream);
int mla_prepare_output_weight(const mla_dims* dims, int32_t dim, const uint16_t* w_o, uint16_t* w_o_prepared,
                              hipStream_t stream);
int mla_fold_output_weights(const mla_dims* dims, int32_t dim, const uint16_t* w_o, const uint16_t* w_uv,
                            uint16_t* w_ov_prepared, hipStream_t stream);
size_t mla_output_projection_workspace_size(const mla_dims* dims, int32_t num_tokens, int32_t dim, int32_t folded);
int mla_output_projection(const mla_dims* dims, int32_t num_tokens, int32_t dim, int32_t folded, const uint16_t* act,
                          const uint16_t* w_prepared, void* workspace, size_t workspace_bytes, uint16_t* y,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * The query path with the query and key projections multiplied ahead of time
 * ("论文复现工坊 No.4", section 2: wq_a, q_norm (RMSNorm over q_lora_rank), wq_b with per-head
 * output [q_nope (d_nope) | q_R (d_rope)]; section 4: the absorbed query is scored against c_KV;
 * "淺析DeepSeek多頭潛在注意力機制（MLA）", "MLA的數學原理": the product of the query and key
 * projections formed once).
 *
 * mla_absorb_query_weights - once per weight set: the prepared query weight w_q, head h's 576 rows
 *   [W_UQK[h] = W_UK[h]^T W_UQ_nope[h] (d_c rows, fp32 sums, one rounding); W_QR[h] (d_rope rows, copied)]
 *   of q_rank elements each, stored in MFMA operand order: row n, element k of head h at
 *     (((h * 18 + n / 32) * (q_rank / 16) + k / 16) * 64 + n % 32 + 32 ((k / 8) % 2)) * 8 + k % 8
 *   (n_heads * 576 * q_rank bf16 in all, 8-byte aligned).
 *   w_uq  [n_heads (d_nope + d_rope), q_rank] bf16 (wq_b's weight; head h's rows are its q_nope rows,
 *         then its q_R rows), 8-byte aligned;  w_uk [n_heads, d_nope, d_c] bf16 as for decode.
 *   q_rank a positive multiple of 64 up to 2048 (else MLA_ERR_UNSUPPORTED).
 *
 * mla_query_absorbed - the decode kernel's query rows straight from the hidden state:
 *   c_q = bf16(RMSNorm(bf16(x W_DQ^T)) with eps and gamma_q)
 *   q_abs[t, h, 0:d_c]   = bf16(W_UQK[h] c_q[t])
 *   q_abs[t, h, d_c:576] = R_pos(t) bf16(W_QR[h] c_q[t])   (fp64 angles as mla_rope_append, one rounding)
 *   x [num_tokens, dim] bf16, dim a multiple of 64;  w_dq [q_rank, dim];  gamma_q [q_rank]
 *   w_q the prepared weight of mla_absorb_query_weights;  token_pos [num_tokens] int32;
 *   q_abs [num_tokens, n_heads, 576] bf16 (the layout mla_decode_absorbed takes);
 *   workspace >= mla_query_absorbed_workspace_size(...) bytes, 256-byte aligned;  x, w_dq, w_q
 *   16-byte aligned, q_abs 8-byte aligned.
 * Three launches on `stream`; num_tokens == 0 is a no-op. The size query returns 0 for arguments
 * the call would reject.
 * ------------------------------------------------------------------------------------------- */
int mla_absorb_query_weights(const mla_dims* dims, int32_t q_rank, const uint16_t* w_uq, const uint16_t* w_uk,
                             uint16_t* w_q, hipStream_t stream);
size_t mla_query_absorbed_workspace_size(const mla_dims* dims, int32_t num_tokens, int32_t dim, int32_t q_rank);
int mla_query_absorbed(const mla_dims* dims, int32_t num_tokens, const int32_t* token_pos, const uint16_t* x,
                       int32_t dim, const uint16_t* w_dq, const uint16_t* gamma_q, float eps, int32_t q_rank,
                       const uint16_t* w_q, void* workspace, size_t workspace_bytes, uint16_t* q_abs,
                       hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_check_inputs - a device-side check of the index data the other calls take on trust: the host
 * cannot read device-resident lengths, block ids and chunk offsets, and the append and attention
 * kernels address the cache with them ("论文复现工坊 No.4", section 2: the cache is addressed by
 * sequence and position; the paged layout adds the block table of the descriptor above).
 *   seq_lens   [batch] int32 (device): every sequence's length (as mla_decode / mla_chunked_prefill)
 *   cu_q_lens  [batch + 1] int32 (device) or NULL: the chunk offsets of a prefill; NULL for decode
 *   total_q    the prefill's total_q (ignored when cu_q_lens is NULL)
 *   error_word [1] int32 (device, 4-byte aligned): written with the OR of the MLA_CHECK_* bits of the
 *              rules the data breaks, 0 when it breaks none (batch == 0 writes 0)
 * One work-group of one launch on `stream`; it reads seq_lens, the block table and cu_q_lens only
 * (never the cache), so it is safe on bad data, allocates nothing, and can be captured in a graph.
 * Cost grows with batch * max_blocks_per_seq (a debugging aid, not part of the hot path).
 * Errors: MLA_ERR_NULL for a missing pointer (seq_lens when batch > 0, error_word), MLA_ERR_BAD_ARG
 * for batch < 0, total_q < 0 with offsets, or a misaligned error_word; dims and cache as everywhere.
 * ------------------------------------------------------------------------------------------- */
int mla_check_inputs(const mla_dims* dims, const mla_cache* cache, int32_t batch, const int32_t* seq_lens,
                     const int32_t* cu_q_lens, int32_t total_q, int32_t* error_word, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_kv_down_query_absorbed - mla_kv_down_append and mla_query_absorbed of the same new tokens in one
 * call, the two projections of the hidden state that come before the attention ("论文复现工坊 No.4",
 * section 2: wkv_a with kv_norm on the latent part, wq_a with q_norm, then wq_b; section 4: the key
 * up-projection absorbed into the query). Results: the cache rows exactly as mla_kv_down_append
 * writes them and q_abs exactly as mla_query_absorbed writes it (bit for bit wherever the two calls
 * split the input dimension the same way, as at 32 tokens of width 4096 with q_rank 512).
 *   Arguments as the two calls: cache, token_seq, token_pos, x [num_tokens, dim], w_dkv, gamma_kv
 *   and eps_kv as mla_kv_down_append's w_dkv, gamma and eps; w_dq, gamma_q, eps_q, q_rank, w_q and
 *   q_abs as mla_query_absorbed's;
 *   workspace >= mla_kv_down_query_absorbed_workspace_size(dims, num_tokens, dim, q_rank) bytes,
 *   256-byte aligned; x, w_dkv, w_dq, w_q 16-byte aligned, q_abs 8-byte aligned;
 *   num_tokens <= 2097120.
 * Errors: MLA_ERR_NULL for a missing pointer, MLA_ERR_BAD_ARG for a negative count, a bad eps, a
 * small or misaligned buffer, MLA_ERR_UNSUPPORTED for dim or q_rank not a multiple of 64 or
 * q_rank > 2048. The size query returns 0 for arguments the call would reject.
 * Below 256 tokens three launches on `stream` (one split-K GEMM over both weights, one finishing
 * launch for both paths, the query GEMM) instead of the two calls' five; from 256 tokens the two
 * calls' launches one after the other. num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------------------------- */
size_t mla_kv_down_query_absorbed_workspace_size(const mla_dims* dims, int32_t num_tokens, int32_t dim,
                                                 int32_t q_rank);
int mla_kv_down_query_absorbed(const mla_dims* dims, const mla_cache* cache, int32_t num_tokens,
                               const int32_t* token_seq, const int32_t* token_pos, const uint16_t* x, int32_t dim,
                               const uint16_t* w_dkv, const uint16_t* gamma_kv, float eps_kv, const uint16_t* w_dq,
                               const uint16_t* gamma_q, float eps_q, int32_t q_rank, const uint16_t* w_q,
                               void* workspace, size_t workspace_bytes, uint16_t* q_abs, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * mla_chunked_prefill_expanded - the same causal chunked prefill as mla_chunked_prefill, computed in
 * the expanded form ("Multi-Head Latent Attention: DeepSeek V2/V3 工程视角" names the up-projection
 * of the latent cache and its absorbed equivalent as the two ways to attend; "论文复现工坊 No.4",
 * section 2: k_nope and v are the per-head split of wkv_b applied to c_KV, the score is
 * q_nope . k_nope + q_R . k_R, scaled by 1/sqrt(d_nope + d_rope)):
 *   k_nope[t, h] = W_UK[h] c_t,  v[t, h] = W_UV[h] c_t   (every cached token, rounded to bf16)
 *   out[j, h, :] = sum_{t<=p} softmax_t(scale (q_nope[j,h] . k_nope[t,h] + q_rope[j,h] . kR_t)) v[t, h]
 * Arguments as mla_chunked_prefill, plus
 *   max_seq_len  host bound on every seq_lens[b] (sizes the up-projected keys and values), >= max_q_len
 *   workspace >= mla_chunked_prefill_expanded_workspace_size(dims, batch, max_seq_len) bytes, 256-byte
 *   aligned (2 x batch x n_heads x roundup(max_seq_len, 128) x 128 bf16); q_nope, q_rope 16-byte
 *   aligned, out 8-byte aligned.
 * Fewer multiply-adds than the absorbed form when a chunk attends to a long prefix; more memory
 * traffic (the up-projected keys and values are written and read back). Two launches on `stream`.
 * ------------------------------------------------------------------------------------------- */
size_t mla_chunked_prefill_expanded_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_seq_len);
int mla_chunked_prefill_expanded(const mla_dims* dims, const mla_cache* cache, int32_t batch,
                                 const int32_t* seq_lens, const int32_t* cu_q_lens, int32_t total_q,
                                 int32_t max_q_len, int32_t max_seq_len, const uint16_t* q_nope,
                                 const uint16_t* q_rope, const uint16_t* w_uk, const uint16_t* w_uv,
                                 void* workspace, size_t workspace_bytes, uint16_t* out, float* lse_out,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
