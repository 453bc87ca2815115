/*
 * One decode step driven through the C ABI of libwmtp from plain C: device memory from
 * hipMalloc, no Python and no torch in the call path.
 *
 *   decode_step <inputs.bin> <outputs.bin>
 *
 * The inputs (written by tests/test_c_abi_gpu.py from seeded synthetic data) hold one
 * sequence: a paged K|V pool of n0 context tokens with its block table, the verify
 * queries and new tokens of one target layer, and a draft query and new token.  The
 * program runs, in stream order:
 *   1. the verify layer: wmtp_verify_attn_append (t_q new tokens) + wmtp_combine;
 *   2. the windowed draft step: the ring filled from the context by wmtp_ring_append,
 *      then wmtp_draft_attn_append (WMTP_SINK_WINDOW) + wmtp_combine;
 *   3. the native draft step into final outputs: wmtp_draft_attn_noalloc (WMTP_FULL)
 *      over the pool, with its own token appended;
 * and checks three argument errors (a NULL shape, a misaligned query, a workspace one
 * byte short), which must return their codes and enqueue nothing.  The outputs file
 * holds the three (out, lse) pairs in fp32 and the three error codes.  Exit status 0
 * on success; any unexpected return code is printed and gives exit status 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "wmtp.h"

#define CHECK_HIP(x)                                                             \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(1);                                                                   \
    }                                                                            \
  } while (0)

#define CHECK_WMTP(x)                                                            \
  do {                                                                           \
    int s_ = (x);                                                                \
    if (s_ != WMTP_OK) {                                                         \
      fprintf(stderr, "%s:%d %s: %d (%s)\n", __FILE__, __LINE__, #x, s_, wmtp_status_str(s_)); \
      exit(1);                                                                   \
    }                                                                            \
  } while (0)

/* Header of the inputs file: int32 fields, then the scale (fp32), then the arrays. */
typedef struct {
  int32_t magic;          /* 0x57'4d'54'50 */
  int32_t num_q_heads, num_kv_heads, head_dim;
  int32_t t_q;            /* verify query tokens */
  int32_t n0;             /* context tokens cached before the step */
  int32_t num_blocks;     /* physical blocks of the pool */
  int32_t max_blocks;     /* block-table row length */
  int32_t sink, window, headroom;
  float scale;
} header;

static void* read_exact(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "short read (%zu bytes)\n", bytes);
    exit(1);
  }
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void write_back(FILE* f, const void* dev, size_t bytes) {
  void* h = malloc(bytes);
  if (!h) exit(1);
  CHECK_HIP(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
  if (fwrite(h, 1, bytes, f) != bytes) {
    fprintf(stderr, "short write\n");
    exit(1);
  }
  free(h);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <inputs.bin> <outputs.bin>\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  header hd;
  if (fread(&hd, sizeof hd, 1, in) != 1 || hd.magic != 0x574d5450) {
    fprintf(stderr, "bad inputs header\n");
    return 1;
  }
  const int Hq = hd.num_q_heads, Hk = hd.num_kv_heads, D = hd.head_dim, tq = hd.t_q, n0 = hd.n0;
  const int slots = hd.sink + hd.window + hd.headroom;
  const size_t row = (size_t)D * 2; /* bf16 bytes of one head's row */
  const size_t pool_bytes = (size_t)hd.num_blocks * Hk * 2 * 16 * row;

  void* pool_h = read_exact(in, pool_bytes);
  void* bt_h = read_exact(in, (size_t)hd.max_blocks * 4);
  void* qv_h = read_exact(in, (size_t)tq * Hq * row);
  void* kv_new_h = read_exact(in, (size_t)tq * Hk * row);
  void* vv_new_h = read_exact(in, (size_t)tq * Hk * row);
  void* qd_h = read_exact(in, (size_t)Hq * row);
  void* kd_new_h = read_exact(in, (size_t)Hk * row);
  void* vd_new_h = read_exact(in, (size_t)Hk * row);
  void* kctx_h = read_exact(in, (size_t)n0 * Hk * row);
  void* vctx_h = read_exact(in, (size_t)n0 * Hk * row);
  fclose(in);

  hipStream_t st;
  CHECK_HIP(hipStreamCreate(&st));
  uint8_t* pool = (uint8_t*)to_device(pool_h, pool_bytes);
  int32_t* bt = (int32_t*)to_device(bt_h, (size_t)hd.max_blocks * 4);
  void* qv = to_device(qv_h, (size_t)tq * Hq * row);
  void* kv_new = to_device(kv_new_h, (size_t)tq * Hk * row);
  void* vv_new = to_device(vv_new_h, (size_t)tq * Hk * row);
  void* qd = to_device(qd_h, (size_t)Hq * row);
  void* kd_new = to_device(kd_new_h, (size_t)Hk * row);
  void* vd_new = to_device(vd_new_h, (size_t)Hk * row);
  void* kctx = to_device(kctx_h, (size_t)n0 * Hk * row);
  void* vctx = to_device(vctx_h, (size_t)n0 * Hk * row);

  wmtp_shape shape = {Hq, Hk, D, hd.scale, WMTP_BF16};
  /* one pool, K and V of a (block, head) side by side: v starts 16 rows after k */
  wmtp_paged paged = {pool, pool + 16 * row, bt, WMTP_BLOCK_SIZE, hd.max_blocks, hd.num_blocks, 32};

  /* ---- 1. verify layer: append t_q tokens at n0 .. n0 + t_q - 1, attend, combine */
  const int32_t len_v = n0 + tq;
  const int64_t ws_v_bytes = wmtp_verify_workspace_bytes(&shape, tq, &len_v, 1, 0);
  if (ws_v_bytes < 0) {
    fprintf(stderr, "wmtp_verify_workspace_bytes: %lld\n", (long long)ws_v_bytes);
    return 1;
  }
  void* ws_v = NULL;
  CHECK_HIP(hipMalloc(&ws_v, (size_t)ws_v_bytes + 256));
  wmtp_partials parts;
  CHECK_WMTP(wmtp_verify_attn_append(&shape, qv, tq, &paged, kv_new, vv_new, &len_v, 1, 0, ws_v,
                                     (size_t)ws_v_bytes, &parts, st));
  float *out_v = NULL, *lse_v = NULL;
  CHECK_HIP(hipMalloc((void**)&out_v, (size_t)tq * Hq * D * 4));
  CHECK_HIP(hipMalloc((void**)&lse_v, (size_t)tq * Hq * 4));
  CHECK_WMTP(wmtp_combine(&parts, out_v, lse_v, WMTP_F32, st));

  /* ---- 2. windowed draft step: ring from the context, then append + attend at n0 + 1 */
  const size_t ring_bytes = (size_t)Hk * slots * row;
  void *rk = NULL, *rv = NULL;
  int32_t* tags = NULL;
  CHECK_HIP(hipMalloc(&rk, ring_bytes));
  CHECK_HIP(hipMalloc(&rv, ring_bytes));
  CHECK_HIP(hipMalloc((void**)&tags, (size_t)slots * 4));
  CHECK_HIP(hipMemsetAsync(tags, 0xff, (size_t)slots * 4, st)); /* every slot empty (-1) */
  wmtp_ring ring = {rk, rv, tags, hd.sink, hd.window, hd.headroom, NULL, NULL};
  const int32_t pos0 = 0;
  CHECK_WMTP(wmtp_ring_append(&shape, &ring, kctx, vctx, &pos0, 1, n0, st));
  const int32_t len_d = n0 + 1;
  const int64_t ws_d_bytes =
      wmtp_draft_workspace_bytes(WMTP_SINK_WINDOW, &shape, &len_d, 1, 0, hd.sink, hd.window, hd.headroom);
  if (ws_d_bytes < 0) {
    fprintf(stderr, "wmtp_draft_workspace_bytes: %lld\n", (long long)ws_d_bytes);
    return 1;
  }
  void* ws_d = NULL;
  CHECK_HIP(hipMalloc(&ws_d, (size_t)ws_d_bytes + 256));
  CHECK_WMTP(wmtp_draft_attn_append(WMTP_SINK_WINDOW, &shape, qd, NULL, &ring, kd_new, vd_new, &len_d, 1, 0,
                                    ws_d, (size_t)ws_d_bytes, &parts, st));
  float *out_w = NULL, *lse_w = NULL;
  CHECK_HIP(hipMalloc((void**)&out_w, (size_t)Hq * D * 4));
  CHECK_HIP(hipMalloc((void**)&lse_w, (size_t)Hq * 4));
  CHECK_WMTP(wmtp_combine(&parts, out_w, lse_w, WMTP_F32, st));

  /* ---- 3. native draft step into final outputs, no workspace: the pool now holds the
   * context and the verify tokens; the draft token goes to position n0 + t_q */
  const int32_t len_n = n0 + tq + 1;
  float *out_n = NULL, *lse_n = NULL;
  CHECK_HIP(hipMalloc((void**)&out_n, (size_t)Hq * D * 4));
  CHECK_HIP(hipMalloc((void**)&lse_n, (size_t)Hq * 4));
  CHECK_WMTP(wmtp_draft_attn_noalloc(WMTP_FULL, &shape, qd, &paged, NULL, kd_new, vd_new, &len_n, 1, 0, out_n,
                                     lse_n, WMTP_F32, st));

  /* ---- argument errors: their codes, and nothing enqueued */
  int32_t errs[3];
  errs[0] = wmtp_verify_attn(NULL, qv, tq, &paged, &len_v, 1, 0, ws_v, (size_t)ws_v_bytes, &parts, st);
  errs[1] = wmtp_verify_attn(&shape, (const uint8_t*)qv + 2, tq, &paged, &len_v, 1, 0, ws_v, (size_t)ws_v_bytes,
                             &parts, st);
  errs[2] = wmtp_verify_attn(&shape, qv, tq, &paged, &len_v, 1, 0, ws_v, (size_t)ws_v_bytes - 1, &parts, st);
  CHECK_HIP(hipStreamSynchronize(st));

  FILE* out = fopen(argv[2], "wb");
  if (!out) {
    perror(argv[2]);
    return 1;
  }
  write_back(out, out_v, (size_t)tq * Hq * D * 4);
  write_back(out, lse_v, (size_t)tq * Hq * 4);
  write_back(out, out_w, (size_t)Hq * D * 4);
  write_back(out, lse_w, (size_t)Hq * 4);
  write_back(out, out_n, (size_t)Hq * D * 4);
  write_back(out, lse_n, (size_t)Hq * 4);
  if (fwrite(errs, sizeof errs, 1, out) != 1) return 1;
  fclose(out);

  void* bufs[] = {pool, bt, qv, kv_new, vv_new, qd, kd_new, vd_new, kctx, vctx, ws_v, out_v, lse_v,
                  rk, rv, tags, ws_d, out_w, lse_w, out_n, lse_n};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) CHECK_HIP(hipFree(bufs[i]));
  CHECK_HIP(hipStreamDestroy(st));
  void* host[] = {pool_h, bt_h, qv_h, kv_new_h, vv_new_h, qd_h, kd_new_h, vd_new_h, kctx_h, vctx_h};
  for (size_t i = 0; i < sizeof host / sizeof host[0]; ++i) free(host[i]);
  printf("decode_step: ok\n");
  return 0;
}
