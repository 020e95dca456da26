/* A C99 program that runs one decode step on the GPU through include/mla.h alone: HIP runtime calls
 * for memory and a stream, the library for all of the work. No Python or torch in this process.
 *
 * argv[1] is a directory of little-endian raw arrays written by the test that runs this program:
 *   meta.bin      int32 [6]: batch B, heads H, num_blocks, max_blocks_per_seq, history tokens Th, paged
 *   seq_lens.bin  int32 [B]; table.bin int32 [B, max_blocks_per_seq] (paged only)
 *   hist_seq.bin, hist_pos.bin int32 [Th]; hist_ckv.bin bf16 [Th, 512]; hist_kr.bin bf16 [Th, 64]
 *   new_seq.bin, new_pos.bin int32 [B]; new_ckv.bin bf16 [B, 512]; new_kr.bin bf16 [B, 64]
 *   q_nope.bin bf16 [B, H, 128]; q_rope.bin bf16 [B, H, 64] (not rotated); w_uk.bin, w_uv.bin bf16 [H, 128, 512]
 * The step: every cache slot set to a bf16 NaN; the history appended (mla_rope_append); the device-side
 * input check (mla_check_inputs, which must report nothing); the new tokens appended with the queries'
 * RoPE part rotated in place; the split plan for this GPU's compute units; mla_decode; mla_decode_combine.
 * Written back to the same directory: out.bin bf16 [B, H, 128], lse.bin fp32 [B, H], cache.bin (the
 * whole cache after the appends), q_rope_rot.bin bf16 [B, H, 64], plan.bin int32 [2] (split tokens,
 * splits). Exit status 0 on success; otherwise the number of the step that failed. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla.h"

static char g_dir[4096];

static void* read_all(const char* name, size_t bytes) {
  char path[4200];
  void* p = malloc(bytes ? bytes : 1);
  FILE* f;
  snprintf(path, sizeof(path), "%s/%s", g_dir, name);
  f = fopen(path, "rb");
  if (!f || !p || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path);
    exit(2);
  }
  fclose(f);
  return p;
}

static void write_all(const char* name, const void* p, size_t bytes) {
  char path[4200];
  FILE* f;
  snprintf(path, sizeof(path), "%s/%s", g_dir, name);
  f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(3);
  }
  fclose(f);
}

/* device copy of a host array */
static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess) {
    fprintf(stderr, "hipMalloc of %zu bytes failed\n", bytes);
    exit(4);
  }
  if (bytes && hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "copy to the device failed\n");
    exit(4);
  }
  return d;
}

#define STEP(n, call)                                                               \
  do {                                                                              \
    int st_ = (call);                                                               \
    if (st_ != MLA_OK) {                                                            \
      fprintf(stderr, "step %d: %s returned %s\n", n, #call, mla_status_string(st_)); \
      return 10 + n;                                                                \
    }                                                                               \
  } while (0)

#define HIPCHECK(n, call)                                              \
  do {                                                                 \
    if ((call) != hipSuccess) {                                        \
      fprintf(stderr, "step %d: %s failed\n", n, #call);               \
      return 10 + n;                                                   \
    }                                                                  \
  } while (0)

int main(int argc, char** argv) {
  int32_t* meta;
  int32_t B, H, nblk, maxb, th, paged, max_len = 0, split_tokens = 0, num_splits = 0, num_cus = 0, err_word = -1;
  size_t row = 576, cache_elems, ws_bytes;
  int32_t *seq_lens, *table = NULL;
  void *d_seq_lens, *d_table = NULL, *d_hseq, *d_hpos, *d_hckv, *d_hkr, *d_nseq, *d_npos, *d_nckv, *d_nkr;
  void *d_qn, *d_qr, *d_wuk, *d_wuv, *d_cache, *d_ws, *d_op, *d_lp, *d_out, *d_lse, *d_err;
  uint16_t* host_u16;
  float* host_f32;
  hipStream_t stream;
  mla_dims dims = {0, 512, 64, 128, 128, 64, 0.07216878364870322f, 10000.0f};
  mla_cache cache;
  int32_t plan[2];
  int b;

  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 1;
  }
  snprintf(g_dir, sizeof(g_dir), "%s", argv[1]);
  meta = (int32_t*)read_all("meta.bin", 6 * sizeof(int32_t));
  B = meta[0], H = meta[1], nblk = meta[2], maxb = meta[3], th = meta[4], paged = meta[5];
  dims.n_heads = H;
  seq_lens = (int32_t*)read_all("seq_lens.bin", (size_t)B * 4);
  for (b = 0; b < B; ++b) max_len = seq_lens[b] > max_len ? seq_lens[b] : max_len;
  if (paged) table = (int32_t*)read_all("table.bin", (size_t)B * maxb * 4);

  HIPCHECK(1, hipStreamCreate(&stream));
  d_seq_lens = to_device(seq_lens, (size_t)B * 4);
  if (paged) d_table = to_device(table, (size_t)B * maxb * 4);
  d_hseq = to_device(read_all("hist_seq.bin", (size_t)th * 4), (size_t)th * 4);
  d_hpos = to_device(read_all("hist_pos.bin", (size_t)th * 4), (size_t)th * 4);
  d_hckv = to_device(read_all("hist_ckv.bin", (size_t)th * 512 * 2), (size_t)th * 512 * 2);
  d_hkr = to_device(read_all("hist_kr.bin", (size_t)th * 64 * 2), (size_t)th * 64 * 2);
  d_nseq = to_device(read_all("new_seq.bin", (size_t)B * 4), (size_t)B * 4);
  d_npos = to_device(read_all("new_pos.bin", (size_t)B * 4), (size_t)B * 4);
  d_nckv = to_device(read_all("new_ckv.bin", (size_t)B * 512 * 2), (size_t)B * 512 * 2);
  d_nkr = to_device(read_all("new_kr.bin", (size_t)B * 64 * 2), (size_t)B * 64 * 2);
  d_qn = to_device(read_all("q_nope.bin", (size_t)B * H * 128 * 2), (size_t)B * H * 128 * 2);
  d_qr = to_device(read_all("q_rope.bin", (size_t)B * H * 64 * 2), (size_t)B * H * 64 * 2);
  d_wuk = to_device(read_all("w_uk.bin", (size_t)H * 128 * 512 * 2), (size_t)H * 128 * 512 * 2);
  d_wuv = to_device(read_all("w_uv.bin", (size_t)H * 128 * 512 * 2), (size_t)H * 128 * 512 * 2);

  /* the cache, every slot a bf16 NaN until written */
  cache_elems = (size_t)nblk * 64 * row;
  HIPCHECK(2, hipMalloc(&d_cache, cache_elems * 2));
  HIPCHECK(2, hipMemsetD16((hipDeviceptr_t)d_cache, 0x7FC0, cache_elems));
  memset(&cache, 0, sizeof(cache));
  cache.data = (uint16_t*)d_cache;
  cache.num_blocks = nblk;
  cache.block_table = (const int32_t*)d_table;
  cache.max_blocks_per_seq = maxb;

  /* 3: the history */
  if (th > 0)
    STEP(3, mla_rope_append(&dims, &cache, th, (const int32_t*)d_hseq, (const int32_t*)d_hpos,
                            (const uint16_t*)d_hckv, (const uint16_t*)d_hkr, NULL, stream));
  /* 4: the device-side check of lengths and block ids */
  d_err = to_device(&err_word, 4);
  STEP(4, mla_check_inputs(&dims, &cache, B, (const int32_t*)d_seq_lens, NULL, 0, (int32_t*)d_err, stream));
  /* 5: the step's new tokens, the queries' RoPE part turned in place */
  STEP(5, mla_rope_append(&dims, &cache, B, (const int32_t*)d_nseq, (const int32_t*)d_npos, (const uint16_t*)d_nckv,
                          (const uint16_t*)d_nkr, (uint16_t*)d_qr, stream));
  /* 6: the plan for this GPU */
  HIPCHECK(6, hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, 0));
  STEP(6, mla_decode_plan(&dims, B, max_len, num_cus, &split_tokens, &num_splits));
  /* 7: attention (absorption inside) and 8: the combine with W_UV */
  ws_bytes = mla_decode_workspace_size(&dims, B);
  HIPCHECK(7, hipMalloc(&d_ws, ws_bytes));
  HIPCHECK(7, hipMalloc(&d_op, (size_t)B * H * num_splits * 512 * 2));
  HIPCHECK(7, hipMalloc(&d_lp, (size_t)B * H * num_splits * 4));
  HIPCHECK(7, hipMalloc(&d_out, (size_t)B * H * 128 * 2));
  HIPCHECK(7, hipMalloc(&d_lse, (size_t)B * H * 4));
  STEP(7, mla_decode(&dims, &cache, B, (const int32_t*)d_seq_lens, (const uint16_t*)d_qn, (const uint16_t*)d_qr,
                     (const uint16_t*)d_wuk, split_tokens, num_splits, d_ws, ws_bytes, (uint16_t*)d_op, (float*)d_lp,
                     stream));
  STEP(8, mla_decode_combine(&dims, B, num_splits, (const uint16_t*)d_op, (const float*)d_lp, (const uint16_t*)d_wuv,
                             (uint16_t*)d_out, (float*)d_lse, stream));
  HIPCHECK(9, hipStreamSynchronize(stream));

  HIPCHECK(10, hipMemcpy(&err_word, d_err, 4, hipMemcpyDeviceToHost));
  if (err_word != 0) {
    fprintf(stderr, "mla_check_inputs reported %d\n", (int)err_word);
    return 30;
  }
  host_u16 = (uint16_t*)malloc(cache_elems * 2);
  host_f32 = (float*)malloc((size_t)B * H * 4);
  HIPCHECK(10, hipMemcpy(host_u16, d_out, (size_t)B * H * 128 * 2, hipMemcpyDeviceToHost));
  write_all("out.bin", host_u16, (size_t)B * H * 128 * 2);
  HIPCHECK(10, hipMemcpy(host_f32, d_lse, (size_t)B * H * 4, hipMemcpyDeviceToHost));
  write_all("lse.bin", host_f32, (size_t)B * H * 4);
  HIPCHECK(10, hipMemcpy(host_u16, d_qr, (size_t)B * H * 64 * 2, hipMemcpyDeviceToHost));
  write_all("q_rope_rot.bin", host_u16, (size_t)B * H * 64 * 2);
  HIPCHECK(10, hipMemcpy(host_u16, d_cache, cache_elems * 2, hipMemcpyDeviceToHost));
  write_all("cache.bin", host_u16, cache_elems * 2);
  plan[0] = split_tokens;
  plan[1] = num_splits;
  write_all("plan.bin", plan, sizeof(plan));
  printf("decode step done: B=%d H=%d, plan %d x %d on %d compute units\n", (int)B, (int)H, (int)split_tokens,
         (int)num_splits, (int)num_cus);
  return 0;
}
