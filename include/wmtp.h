/*
 * wmtp.h - Windowed-MTP decode attention for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the problem statement of "Windowed-MTP: Removing the
 * Full-Context Draft-KV Tax at Million-Token Context" (arxivlens.com summary,
 * Abstract): a Multi-Token-Prediction draft head runs gamma draft forwards per
 * decode step, each attending either over the whole KV cache (native MTP) or
 * over attention-sink tokens plus a window of recent tokens kept in a compact
 * ring buffer (Windowed-MTP); the target verifies gamma+1 tokens with
 * full-context attention.  The case study "Does speculative decode still pay
 * at 128K context?" (howtospark.com, Method) fixes one verify cycle as three
 * draft forwards plus one batched verify.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Ownership: the caller allocates and owns every buffer.  The library never
 *    allocates, frees or keeps a pointer after a call returns.
 *  - Pointers: arguments documented "device" are HIP device pointers; "host"
 *    arguments are read on the host before the call returns.
 *  - Streams: `stream` is a hipStream_t passed as void*; NULL is the default
 *    stream.  Every call that launches work is asynchronous, performs no host
 *    synchronisation and copies nothing host-to-device, so a sequence of calls
 *    can be captured in a HIP graph.
 *  - Errors: every int-returning call returns WMTP_OK (0) or a negative
 *    WMTP_E* code.  Argument checks run before any HIP call; on an error no
 *    work is enqueued.  No call aborts, prints, or throws across the boundary.
 *    WMTP_ELAUNCH reports a failed kernel launch (hipGetLastError).
 *  - Thread safety: the library has no mutable global state, except the fixed
 *    scratch of wmtp_draft_attn_noalloc (see there).
 *
 * Numbers
 * -------
 *  - dtype WMTP_F32: IEEE binary32.  dtype WMTP_BF16: bfloat16 (upper half of
 *    a binary32).  q, k and v share one dtype; accumulation is always fp32.
 *  - head_dim D is 64, 128 or 256; G = num_q_heads / num_kv_heads is 1, 2, 4
 *    or 8; query head h uses KV head h / G.
 *  - scale multiplies q.k (the usual value is 1/sqrt(D)).
 *  - lse outputs are natural logs of sum_t exp(scale * q.k_t).
 *
 * Memory layouts (row-major, innermost last)
 * ------------------------------------------
 *  paged pool   k, v: [num_blocks][num_kv_heads][block_size][D], block_size 16
 *  block table  [batch][max_blocks_per_seq] int32 physical block ids
 *  ring         k, v: [batch][num_kv_heads][sink + window + headroom][D]
 *               slot_pos: [batch][sink + window + headroom] int32 (absolute position, -1 empty)
 *               slot(p) = p for p < sink, else sink + (p - sink) % (window + headroom)
 *  draft q      [batch][num_q_heads][D]
 *  verify q     [batch][t_q][num_q_heads][D]
 *  new k, v     [batch][t_new][num_kv_heads][D]
 *  partials     o: [total_splits][rows_per_seq][D] fp32, lse: [total_splits][rows_per_seq] fp32
 *  combine out  [batch][rows_per_seq][D] (fp32 or bf16), lse [batch][rows_per_seq] fp32
 *               rows_per_seq = num_q_heads for the draft, t_q * num_q_heads for
 *               verify (row = i * num_q_heads + h for query token i, head h).
 */
#ifndef WMTP_H
#define WMTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
#define WMTP_OK             0
#define WMTP_EINVAL        -1   /* null pointer, bad size, bad enum, inconsistent shapes      */
#define WMTP_EUNSUPPORTED  -2   /* head_dim, group size, dtype or row count not built         */
#define WMTP_EALIGN        -3   /* a k/v/q/output base pointer is not 16-byte aligned          */
#define WMTP_EWORKSPACE    -4   /* workspace too small for the planned splits                  */
#define WMTP_ELAUNCH       -5   /* a kernel launch failed                                      */

/* ---------------------------------------------------------------- enums */
#define WMTP_F32   0
#define WMTP_BF16  1

#define WMTP_FULL         0     /* native MTP draft: every cached entry                       */
#define WMTP_SINK_WINDOW  1     /* Windowed-MTP draft: sink + window entries from the ring     */
/* Optional flag OR-ed into the draft mode (bf16 only): the PV product takes the
 * softmax weights rounded to bf16 (bf16 x bf16 products, fp32 sums) instead of
 * fp32 weights.  The normaliser is summed from the same rounded weights.  With
 * this flag both modes run on the matrix-core kernel of wmtp_verify_attn with
 * one query token (the same arithmetic), over the paged pool or over the
 * ring's visible entries.  Without it the PV product uses the fp32 weights, on
 * a kernel of vector dot products. */
#define WMTP_DRAFT_FAST_PV 0x10

#define WMTP_MAX_BATCH   64     /* sequences per call                                         */
#define WMTP_BLOCK_SIZE  16     /* tokens per paged block                                     */
/* Longest sequence (cache length, and first position + new tokens of an append) a
 * call accepts: 2^30 tokens keeps every position, split end and block index of the
 * kernels inside 32-bit arithmetic.  Longer lengths give WMTP_EINVAL. */
#define WMTP_MAX_SEQ_LEN (1 << 30)
#define WMTP_MAX_VERIFY_ROWS 96 /* t_q * G per KV head in one verify call (3 tiles of 32 rows) */

/* ---------------------------------------------------------------- descriptors */
typedef struct wmtp_shape {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  float   scale;          /* multiplies q.k                                    */
  int32_t dtype;          /* WMTP_F32 or WMTP_BF16, for q, k and v             */
} wmtp_shape;

/* Paged KV cache of one layer.  Token t of sequence b, KV head h, lives in
 * physical block blk = block_table[b][t / 16] at token row
 *     (blk * H_kv + h) * run_rows + t % 16
 * of k and of v (a row is D elements).  run_rows = 16 (or 0) gives separate K
 * and V pools [num_blocks][H_kv][16][D].  run_rows = 32 with v = k + 16 rows
 * gives one pool [num_blocks][H_kv][2][16][D] in which K and V of a (block,
 * head) form one contiguous 32-row run; the kernels then read one run of
 * 32 * D elements per block and head instead of two of half the size, which
 * streams faster from HBM.  Other run_rows >= 16 are accepted as strides. */
typedef struct wmtp_paged {
  void*          k;                   /* device, rows as above                    */
  void*          v;                   /* device, rows as above                    */
  const int32_t* block_table;         /* device, [batch][max_blocks_per_seq]      */
  int32_t        block_size;          /* must be WMTP_BLOCK_SIZE                  */
  int32_t        max_blocks_per_seq;  /* row stride of block_table                */
  int64_t        num_blocks;          /* physical blocks in k and v               */
  int32_t        run_rows;            /* 0 or 16: separate pools; >= 16: stride   */
} wmtp_paged;

/* The compact ring of the windowed draft (Windowed-MTP summary, Abstract).
 * Sinks keep slots 0..S-1; position p >= S lives in slot S + (p - S) mod (W+R);
 * slot_pos records the position a slot holds.  A draft query at length n
 * reads every slot whose position is in {0..S-1} or {n-W..n-1} and < n.  The
 * R headroom slots absorb drafted tokens that verification rejects: with
 * R >= gamma - 1 (gamma drafted tokens per cycle, at least one accepted), a
 * rejected token never overwrites an entry a later window still needs, so
 * rolling back costs nothing but, optionally, wmtp_ring_rollback. */
typedef struct wmtp_ring {
  void*    k;          /* device, [batch][H_kv][S+W+R][D]                  */
  void*    v;          /* device, same layout as k                         */
  int32_t* slot_pos;   /* device, [batch][S+W+R]: position held, -1 = none */
  int32_t  sink;       /* S >= 0                                           */
  int32_t  window;     /* W >= 1                                           */
  int32_t  headroom;   /* R >= 0 extra slots in the cycle                  */
  /* Optional per-sequence policy for the draft query (host, [batch], or
   * NULL = S / W for every sequence): sequence b attends to positions
   * {0..seq_sink[b]-1} and {n-seq_window[b]..n-1}, with
   * 0 <= seq_sink[b] <= S and 1 <= seq_window[b] <= W + R.  The layout stays
   * (S, W, R), so the values may change from one call to the next (adaptive
   * windows, dynamic sinks).  Rolling back gamma drafted tokens needs
   * seq_window[b] + gamma - 1 <= W + R. */
  const int32_t* seq_sink;
  const int32_t* seq_window;
} wmtp_ring;

/* Split-K partial results, written by wmtp_draft_attn / wmtp_verify_attn into
 * the caller's workspace and read by wmtp_combine.  Sequence b owns splits
 * split_base[b] .. split_base[b+1]-1; every split holds all rows of b.  The
 * struct is plain data (host memory) and may be copied. */
typedef struct wmtp_partials {
  float*  o;                                /* device, [total_splits][rows_per_seq][D] */
  float*  lse;                              /* device, [total_splits][rows_per_seq]    */
  int32_t batch;
  int32_t rows_per_seq;
  int32_t head_dim;
  int32_t total_splits;
  int32_t split_base[WMTP_MAX_BATCH + 1];   /* host copy of the per-sequence offsets   */
} wmtp_partials;

/* ---------------------------------------------------------------- planning (host only) */

/* Bytes of workspace wmtp_draft_attn needs.  Arguments as for wmtp_draft_attn
 * (sink/window/headroom, the ring's S/W/R, are read only in WMTP_SINK_WINDOW
 * mode, where the size covers min(n, S + W + R) entries per sequence: enough
 * for any per-sequence sinks and windows).  Returns >= 0 bytes or a negative
 * WMTP_E* code.  Makes no HIP call. */
int64_t wmtp_draft_workspace_bytes(int32_t mode, const wmtp_shape* shape, const int32_t* seq_lens_host,
                                   int32_t batch, int32_t chunk_tokens, int32_t sink, int32_t window,
                                   int32_t headroom);

/* Bytes of workspace wmtp_verify_attn needs.  Makes no HIP call. */
int64_t wmtp_verify_workspace_bytes(const wmtp_shape* shape, int32_t t_q, const int32_t* seq_lens_host,
                                    int32_t batch, int32_t split_tokens);

/* ---------------------------------------------------------------- the hot path */

/* One draft-attention step for `batch` sequences (Windowed-MTP summary,
 * Abstract; readpriors.com post, What happened).
 *
 *  mode (low 4 bits) == WMTP_FULL: sequence b attends to positions 0..n_b-1 read from
 *                            the paged pool `kv` (`ring` may be NULL).
 *  mode (low 4 bits) == WMTP_SINK_WINDOW: sequence b attends to positions {0..S-1} and
 *                            {n_b-W..n_b-1}, read from `ring` (`kv` may be NULL).
 *                            Each visible position p is read from slot(p) when
 *                            slot_pos holds p there (otherwise it is skipped);
 *                            S and W may be per sequence (wmtp_ring.seq_sink /
 *                            seq_window), and the cost follows min(n, S_b + W_b).
 *  n_b = seq_lens_host[b] (host) is the length after this step's own entry was
 *  appended, so the query attends to itself.  q: device [batch][H_q][D].
 *  chunk_tokens: entries per split (a multiple of 32).  0 = library default:
 *  the smallest multiple of 64 (at most 65536) for which the work items
 *  (sequence, KV head, split) fit one round of 256 x max(1, 512 / row bytes)
 *  items in WMTP_FULL mode (one per MI355X compute unit at head_dim 256 in
 *  bf16; narrower rows run fewer waves per item, so more items) or 512 items
 *  in WMTP_SINK_WINDOW mode, or of the smallest multiple of that holding one
 *  item per sequence and KV head.  The count depends on the shape and mode
 *  only, not on WMTP_DRAFT_FAST_PV.
 *  The call writes split partials into `workspace` (device, >= the size from
 *  wmtp_draft_workspace_bytes, 256-byte aligned) and describes them in
 *  *parts (host).  Finish with wmtp_combine. */
int wmtp_draft_attn(int32_t mode, const wmtp_shape* shape, const void* q, const wmtp_paged* kv,
                    const wmtp_ring* ring, const int32_t* seq_lens_host, int32_t batch,
                    int32_t chunk_tokens, void* workspace, size_t workspace_bytes,
                    wmtp_partials* parts, void* stream);

/* Full-context verify attention of t_q query tokens for one target layer
 * (Windowed-MTP summary, Abstract: verification stays full-context).
 *  q: device [batch][t_q][H_q][D].  n_b = seq_lens_host[b] includes the t_q
 *  query tokens' own entries; query token i attends causally to positions
 *  0..n_b-t_q+i.  Requires dtype bf16 and t_q * G <= WMTP_MAX_VERIFY_ROWS
 *  (otherwise WMTP_EUNSUPPORTED).
 *  split_tokens: entries per split (a multiple of 32; 0 = the WMTP_FULL draft
 *  default for the shape: 256 x 256 / head_dim work items).
 *  Workspace and *parts as for wmtp_draft_attn. */
int wmtp_verify_attn(const wmtp_shape* shape, const void* q, int32_t t_q, const wmtp_paged* kv,
                     const int32_t* seq_lens_host, int32_t batch, int32_t split_tokens,
                     void* workspace, size_t workspace_bytes, wmtp_partials* parts, void* stream);

/* A draft step's append and attention in one launch (Windowed-MTP summary,
 * Abstract, and readpriors.com post, What happened: each draft step adds one
 * entry and then attends).  Equal, in the cache it leaves and in *parts, to
 * wmtp_paged_append (WMTP_FULL, into `kv`) or wmtp_ring_append
 * (WMTP_SINK_WINDOW, into `ring`, with its slot tag) of one token at position
 * n_b - 1, followed by wmtp_draft_attn with the same arguments.
 *  k_new, v_new: device [batch][1][H_kv][D], 16-byte aligned, caller-owned;
 *  the work item whose keys include position n_b - 1 writes it before reading.
 *  Every n_b must be >= 1.  Other arguments, workspace and errors as for
 *  wmtp_draft_attn; NULL k_new or v_new gives WMTP_EINVAL.  Nothing is written
 *  when the call returns an error. */
int wmtp_draft_attn_append(int32_t mode, const wmtp_shape* shape, const void* q, const wmtp_paged* kv,
                           const wmtp_ring* ring, const void* k_new, const void* v_new,
                           const int32_t* seq_lens_host, int32_t batch, int32_t chunk_tokens, void* workspace,
                           size_t workspace_bytes, wmtp_partials* parts, void* stream);

/* A target layer's append of the t_q query tokens' own K/V and its verify in
 * one launch (Windowed-MTP summary, Abstract; howtospark case study, Method:
 * the verify pass covers the drafted tokens).  Equal to wmtp_paged_append of
 * t_q tokens at positions n_b - t_q .. n_b - 1 into `kv`, followed by
 * wmtp_verify_attn with the same arguments.
 *  k_new, v_new: device [batch][t_q][H_kv][D], 16-byte aligned, caller-owned;
 *  each work item writes the new positions inside its own key range before
 *  reading.  Other arguments, workspace and errors as for wmtp_verify_attn;
 *  NULL k_new or v_new gives WMTP_EINVAL.  Nothing is written when the call
 *  returns an error. */
int wmtp_verify_attn_append(const wmtp_shape* shape, const void* q, int32_t t_q, const wmtp_paged* kv,
                            const void* k_new, const void* v_new, const int32_t* seq_lens_host, int32_t batch,
                            int32_t split_tokens, void* workspace, size_t workspace_bytes, wmtp_partials* parts,
                            void* stream);

/* Log-sum-exp merge of split partials (flash-decoding combine):
 *  L = log sum_i exp(lse_i),  out = sum_i exp(lse_i - L) * o_i  per row.
 *  Splits with lse = -inf carry no keys and are skipped; a row with no live
 *  split gets out = 0 and lse = -inf.
 *  out: device [batch][rows_per_seq][D], dtype out_dtype (WMTP_F32 or
 *  WMTP_BF16, round-to-nearest-even).  lse_out: device [batch][rows_per_seq]
 *  fp32, or NULL. */
int wmtp_combine(const wmtp_partials* parts, void* out, float* lse_out, int32_t out_dtype, void* stream);

/* For callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  One draft step into final outputs:
 * wmtp_draft_attn (k_new and v_new NULL) or wmtp_draft_attn_append (both set), then
 * wmtp_combine into out / lse_out, with the same arguments, kernels and results,
 * except that the split partials go to a fixed device array of
 * WMTP_NOALLOC_SCRATCH_BYTES inside the library instead of a caller workspace.
 *  out: device [batch][H_q][D] of out_dtype (WMTP_F32 or WMTP_BF16), 16-byte
 *  aligned; lse_out: device [batch][H_q] fp32 or NULL.
 *  Allocates nothing: no hipMalloc, hipFree or allocating library call.  Each GPU
 *  that runs the call holds its own copy of the array until the process ends; its
 *  device address is resolved on the first call on that GPU (make that first call
 *  outside any graph capture).  A plan whose partials need more than
 *  WMTP_NOALLOC_SCRATCH_BYTES (wmtp_draft_workspace_bytes gives the size) returns
 *  WMTP_EWORKSPACE; with the default split sizes, batch x H_kv <= 256 and
 *  contexts up to 4M tokens need at most 4.3 MB.
 *  All calls on one GPU share the array, which keeps the last call's partials
 *  (every split writes all of its rows, so nothing needs clearing): calls that
 *  overlap on one GPU (other streams, other host threads) race; calls in order
 *  on one stream do not. */
#define WMTP_NOALLOC_SCRATCH_BYTES (16 << 20)
int wmtp_draft_attn_noalloc(int32_t mode, const wmtp_shape* shape, const void* q, const wmtp_paged* kv,
                            const wmtp_ring* ring, const void* k_new, const void* v_new,
                            const int32_t* seq_lens_host, int32_t batch, int32_t chunk_tokens, void* out,
                            float* lse_out, int32_t out_dtype, void* stream);

/* Append t_new tokens per sequence to the compact ring (Windowed-MTP summary,
 * Abstract: the ring holds the draft's window).  Token i of sequence b has
 * absolute position p = pos_host[b] + i (pos_host: host, >= 0) and is written
 * to slot(p), with slot_pos[b][slot(p)] = p, only if p < S or
 * p > pos_host[b] + t_new - 1 - (W + R) (it survives the append); so an append
 * longer than the cycle writes each slot once and equals appending the tokens
 * one by one.  t_new = n with pos 0 initialises the ring from a prefill.
 * k_new, v_new: device [batch][t_new][H_kv][D]. */
int wmtp_ring_append(const wmtp_shape* shape, const wmtp_ring* ring, const void* k_new, const void* v_new,
                     const int32_t* pos_host, int32_t batch, int32_t t_new, void* stream);

/* After verification accepted the first tokens of a draft cycle: forget every
 * ring entry at a position >= seq_lens_host[b] (slot_pos becomes -1) for each
 * sequence b.  Optional when appends stay in order (the draft query's
 * position check already hides them, and the next append at a position
 * overwrites it); it leaves the ring holding only accepted positions.
 * Touches slot_pos only; seq_lens_host: host [batch], each >= 0. */
int wmtp_ring_rollback(const wmtp_ring* ring, const int32_t* seq_lens_host, int32_t batch, void* stream);

/* Write t_new tokens per sequence into the paged pool at positions
 * pos_host[b] + i through the block table (the native draft's pool and each
 * target layer's cache).  The block-table row must already cover the
 * positions.  k_new, v_new: device [batch][t_new][H_kv][D]. */
int wmtp_paged_append(const wmtp_shape* shape, const wmtp_paged* kv, const void* k_new, const void* v_new,
                      const int32_t* pos_host, int32_t batch, int32_t t_new, void* stream);

/* ---------------------------------------------------------------- index resolution (test hooks) */

/* Element offsets of (sequence b, position positions[i], KV head h, d = 0) in
 * the paged pool, computed on the GPU by the same device code the kernels
 * use.  positions: device int32 [n]; offsets_out: device int64 [n].  A
 * position that is negative or past the block-table row gets -1. */
int wmtp_debug_resolve_paged(const wmtp_paged* kv, int32_t num_kv_heads, int32_t head_dim, int32_t b,
                             int32_t h, const int32_t* positions, int32_t n, int64_t* offsets_out,
                             void* stream);

/* Ring slot of every listed position: slots_out[i] = slot(positions[i]) for a
 * ring of S = sink, W = window, R = headroom.
 * positions: device int32 [n] (>= 0); slots_out: device int32 [n]. */
int wmtp_debug_resolve_ring(int32_t sink, int32_t window, int32_t headroom, const int32_t* positions, int32_t n,
                            int32_t* slots_out, void* stream);

/* For a query at length n, the position each ring slot must hold for the
 * sink+window visible set (-1 if the slot holds none).
 * out: device int32 [sink+window+headroom]. */
int wmtp_debug_window_positions(int32_t sink, int32_t window, int32_t headroom, int32_t n, int32_t* out,
                                void* stream);

/* ---------------------------------------------------------------- memory accounting (host only) */

/* KV memory of one sequence at `context` tokens with a native or a windowed
 * draft, and the sequences an HBM budget admits (Windowed-MTP summary,
 * Abstract: the ring frees the draft pool the window no longer reads, 7.7-11.1% of
 * total KV at 1M, room for one more concurrent 1M request).  Every
 * full-attention layer (the `target_layers`, and the native draft) keeps a
 * paged pool of ceil(context / 16) blocks of K and V; one int32 block table per
 * sequence serves them all; the windowed draft keeps only its ring of
 * S + W + R slots of K and V plus an int32 tag each. */
typedef struct wmtp_memory_plan {
  int64_t layer_bytes;          /* K+V of one paged full-attention layer        */
  int64_t block_table_bytes;    /* the sequence's block table                   */
  int64_t ring_bytes;           /* K+V+tags of the draft's ring                 */
  int64_t native_seq_bytes;     /* target layers + draft pool + table           */
  int64_t windowed_seq_bytes;   /* target layers + ring + table                 */
  double  reclaimed_fraction;   /* 1 - windowed / native                        */
  int64_t native_sequences;     /* floor(budget / native_seq_bytes)             */
  int64_t windowed_sequences;   /* floor(budget / windowed_seq_bytes)           */
} wmtp_memory_plan;

/* Fill *out (host).  context >= 1 (the reclaimed share is a fraction of a
 * sequence's KV, undefined for a sequence that holds none), target_layers >= 0,
 * budget_bytes >= 0, sink/window/headroom as in wmtp_ring.  Makes no HIP call;
 * WMTP_EINVAL on invalid arguments or int64 overflow. */
int wmtp_plan_memory(const wmtp_shape* shape, int32_t target_layers, int64_t context, int32_t sink,
                     int32_t window, int32_t headroom, int64_t budget_bytes, wmtp_memory_plan* out);

/* ---------------------------------------------------------------- measurement */

/* Streaming-read probe: `workgroups` workgroups of 256 threads each read one
 * contiguous part of src[0, bytes) with 16-byte loads and write one word per
 * thread to sink (device, workgroups * 256 uint32).  It measures the practical
 * HBM read ceiling that the attention kernels' bandwidth is compared with.
 * bytes must be a positive multiple of 16; src 16-byte aligned. */
int wmtp_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

/* Paged streaming-read probe: reads the runs runs[0..nruns) (device int32, run
 * ids clamped to [0, pool_bytes / run_bytes)) of both k and v (device, each
 * pool_bytes), run_bytes per run (a power of two, 4 KiB .. 1 MiB), in that order,
 * split over `workgroups` workgroups of 256 threads; one word per thread goes
 * to sink (device, workgroups * 256 uint32).  With the runs of a paged cache in
 * table order it is the attention kernels' access pattern without their
 * arithmetic: the practical ceiling for reading that cache. */
int wmtp_stream_read_paged(const void* k, const void* v, int64_t pool_bytes, const int32_t* runs, int32_t nruns,
                           int32_t run_bytes, uint32_t* sink, int32_t workgroups, void* stream);

/* ---------------------------------------------------------------- misc */
const char* wmtp_status_str(int status);
const char* wmtp_version(void);

#ifdef __cplusplus
}
#endif
#endif /* WMTP_H */
