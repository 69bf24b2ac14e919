/*
 * ds.h -- C ABI of the Double Sparsity decode-attention library (libds.so),
 * HIP kernels for gfx950 (MI355X).
 *
 * Pages cited by title and section:
 *   [DS]    "Double Sparsity" article, joto.ai blog archive 2025060420469:
 *           "offline calibration" (heavy channels are fixed offline per
 *           layer and head; their K values are copied into a contiguous label
 *           cache at prefill and only the new token's values are added at each
 *           decode step; labels may be kept in 4 bits) and "online forward
 *           computation" (step 1 gathers the query at the heavy channels,
 *           step 2 scores every cached token approximately from the labels,
 *           step 3 picks the top-k tokens and runs exact attention on their
 *           full K/V rows); "use in SGLang" (heavy-channel count, heavy-token
 *           count, dense fallback below a threshold).
 *   [LeanK] LeanK article, aitangshan.cn news 1293675, section 2.2 (a static,
 *           hardware-aligned subset of K channels is kept per head) and
 *           section 3.2 (attention over the pruned K).
 *   [GQA]   grouped-query attention article, trdm.cn news 80600, section 4
 *           (query heads form groups that share one K/V head).
 *
 * Conventions for every call:
 *   - Pointers are device memory owned by the caller unless marked "host".
 *     The library allocates nothing, keeps no state between calls (except
 *     the per-GPU scratch array of ds_decode_attn_noalloc) and never
 *     synchronises the stream.
 *   - fp16 is IEEE binary16.  All arrays are row-major, last index fastest.
 *   - Work is enqueued asynchronously on `stream`.  Arguments are validated on
 *     the host before anything is enqueued; on any error the call returns a
 *     negative ds_status and enqueues nothing.  A failed kernel launch returns
 *     DS_ERR_HIP.  Values that live in device memory (index tables, sequence
 *     lengths, positions) are not read by the host: out-of-range sequence
 *     lengths are clamped on the device to [0, max_seq_len], out-of-range
 *     positions are skipped; out-of-range channel or token indices in the
 *     tables are undefined behaviour.
 *   - Calls that share buffers must be ordered by the caller (same stream).
 */
#ifndef DS_H_
#define DS_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DS_ABI_VERSION 4

typedef enum {
  DS_OK = 0,
  DS_ERR_ARG = -1,       /* missing pointer, bad enum value, bad range */
  DS_ERR_SHAPE = -2,     /* inconsistent or unsupported dimensions */
  DS_ERR_DTYPE = -3,     /* label dtype / channel count combination not supported */
  DS_ERR_ALIGN = -4,     /* pointer or stride breaks the 16-byte alignment rule */
  DS_ERR_WORKSPACE = -5, /* workspace missing or smaller than required */
  DS_ERR_HIP = -6        /* the HIP runtime rejected a launch */
} ds_status;

/* Label cache element type ([DS] offline calibration: 4-bit labels). */
typedef enum { DS_LABEL_F16 = 0, DS_LABEL_INT4 = 1 } ds_label_dtype;

/* Per-KV-head layout of a LeanK cache whose heads keep different numbers of
 * K columns ([LeanK] section 2.2: each head keeps a hardware-aligned count;
 * section 4.4: heads whose K channels are all pruned drop their V cache as
 * well).  Device array [n_kv_heads] (ds_kv_desc.heads).
 *   k_cols  kept K columns of the head: a multiple of 8 up to d_k, or 0 for a
 *           fully pruned head, which stores neither K nor V, selects no token
 *           and outputs zeros;
 *   k_off   element offset of the head's K block from its batch row's (or
 *           page's) K base; the block's token stride is k_cols (rows packed);
 *   v_off   element offset of the head's V block from its batch row's (or
 *           page's) V base; token stride v_stride[2].
 * Offsets are multiples of 8 elements.  Entries are not read on the host;
 * bad ones are undefined behaviour. */
typedef struct {
  int64_t k_cols, k_off, v_off;
} ds_head_layout;

/* K/V cache description (host struct).
 * Contiguous rows (page_size == 0):
 *   K: fp16 [batch][n_kv_heads][capacity][d_k], element strides k_stride =
 *      {batch, kv head, token}; channel stride 1.
 *   V: fp16 [batch][n_kv_heads][capacity][d_v], strides v_stride likewise.
 * Paged token pool (page_size > 0; the serving form of [DS] "use in
 * SGLang", where the K/V cache is a pool of token slots shared by all
 * sequences):
 *   K: fp16 [n_pages][n_kv_heads][page_size][d_k], k_stride = {page, kv
 *      head, token}; V likewise.  Token t of batch row b lives in page
 *      page_table[b][t / page_size] at slot t % page_size.
 *   page_size is a power of two in [16, 65536]; page_table is a device int32
 *   array [batch][max_pages] whose entries for the tokens in use lie in
 *   [0, n_pages) (entries are not read on the host; out-of-range ones are
 *   undefined behaviour); capacity == max_pages * page_size; n_pages *
 *   page_size < 2^31.  The label cache stays one contiguous stream per
 *   (batch row, KV head) (ds_label_desc): its contiguity is what the
 *   approximate scores read.
 * Per-head layout (heads != NULL, either form): K and V of KV head g sit at
 * heads[g].k_off / v_off from the batch row's (page's) base, K rows of
 * heads[g].k_cols columns; k_stride[1], k_stride[2] and v_stride[1] are not
 * used; d_k is the widest kept count (the row width of the keep table).
 * Query head h belongs to KV head h / G with G = n_q_heads / n_kv_heads
 * ([GQA] section 4: consecutive query heads form a group).
 * d_q is the query width (the model's head dim); d_k is the stored K width,
 * equal to d_q unless K is LeanK-compacted to a kept subset of its columns.
 * Limits: d_q <= 256; d_k and d_v multiples of 8 with d_k <= 128 and
 * d_v == 128; G <= 8; capacity <= 2^24.
 * Alignment: K, V 16-byte aligned; every stride a multiple of 8 elements. */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads;
  int32_t d_q, d_k, d_v;
  int32_t capacity;
  int32_t page_size;  /* 0: contiguous rows; else tokens per page of the pool */
  int64_t k_stride[3];
  int64_t v_stride[3];
  const int32_t* page_table; /* paged: [batch][max_pages]; contiguous: NULL */
  int32_t max_pages;  /* paged: page-table entries per batch row; else 0 */
  int32_t n_pages;    /* paged: pages in the pool; else 0 */
  const ds_head_layout* heads; /* device [n_kv_heads] per-head layout, or NULL */
} ds_kv_desc;

/* Label cache description (host struct) ([DS] offline calibration).
 *   r      heavy channels per KV head, 1 <= r <= min(d_k, 128); even for INT4.
 *   slots  token slots per (batch, KV head) row: slots >= capacity and
 *          slots % 16 == 0 (keeps every row 16-byte aligned).
 *   F16:   codes = fp16 [batch][n_kv_heads][slots][r]; scales = NULL.
 *          Entry j of token t is K[b][g][t][chan[g][j]], bit for bit.
 *   INT4:  codes = uint8 [batch][n_kv_heads][slots][r/2];
 *          scales = fp16 [batch][n_kv_heads][slots].
 *          Per token: amax = max_j |x_j| over its r heavy values (fp32),
 *          scale = fp16_rn(amax / 7) (IEEE fp32 division), code_j =
 *          clamp(round_half_even(x_j / scale), -7, 7) (IEEE fp32 division;
 *          scale 0 gives code 0); byte i holds code 2i in its low nibble and
 *          code 2i+1 in its high nibble, two's complement.
 *   codes and scales are 16-byte aligned. */
typedef struct {
  int32_t r;
  int32_t dtype; /* ds_label_dtype */
  int32_t slots;
  int32_t reserved0; /* must be 0 */
  void* codes;
  void* scales;
} ds_label_desc;

/* Label-cache build at prefill ([DS] offline calibration: every prefill
 * token's heavy-channel values go from the K cache into the label cache).
 * Writes label slots t in [t_begin, t_end) of every (batch, KV head) row.
 *   K     fp16 K cache as described by kv (read only; contiguous rows or a
 *         paged pool, whose page table gives each token's K row).
 *   chan  int32 [n_kv_heads][r]: heavy channels, indices into the stored K
 *         columns (0 <= chan < d_k); any order, duplicates allowed.
 * Only batch, n_kv_heads, d_k, capacity, k_stride and the paging fields of
 * kv are read.
 * Errors: DS_ERR_ARG (null pointer, 0 <= t_begin <= t_end <= capacity
 * violated, paging fields given with page_size 0 or a missing page table),
 * DS_ERR_SHAPE (also a bad page size or page count), DS_ERR_DTYPE,
 * DS_ERR_ALIGN, DS_ERR_HIP. */
ds_status ds_label_build(const ds_kv_desc* kv, const void* K, const int32_t* chan,
                         const ds_label_desc* lab, int32_t t_begin, int32_t t_end,
                         hipStream_t stream);

/* Label-cache append at a decode step ([DS] offline calibration: only the new
 * token's heavy-channel values are added).  For each batch row b, writes label
 * slot pos[b] of every KV head from K[b][g][pos[b]].
 *   pos   int32 [batch] device array: the slot whose K row was just written;
 *         rows with pos[b] < 0 or pos[b] >= capacity are left untouched.
 * The result is bit-identical to ds_label_build over the same slots.
 * Errors: as ds_label_build. */
ds_status ds_label_append(const ds_kv_desc* kv, const void* K, const int32_t* chan,
                          const ds_label_desc* lab, const int32_t* pos, hipStream_t stream);

/* Stages of ds_decode_attn, for optional timing events. */
enum {
  DS_STAGE_APPEND = 0,  /* label append of the current token (flag DS_DECODE_APPEND) */
  DS_STAGE_SCORE = 1,   /* steps 1-2: query gather + approximate scores */
  DS_STAGE_SELECT = 2,  /* step 3a: top-k select */
  DS_STAGE_ATTN = 3,    /* step 3b: exact attention over the selected rows */
  DS_STAGE_COMBINE = 4, /* merge of split partial results */
  DS_STAGE_COUNT = 5
};

/* Flags for ds_decode_opts.flags. */
#define DS_DECODE_APPEND 1u         /* first append label slot seq_lens[b]-1 (as ds_label_append) */
#define DS_DECODE_VALIDATE_ONLY 2u  /* validate the arguments and return; enqueue nothing */
#define DS_DECODE_UNFUSED 4u        /* do not run the step as a single kernel */
#define DS_DECODE_STREAM 8u         /* select over every score streamed from memory (no
                                       local top-M pre-selection) */

/* Optional decode settings (host struct; pass NULL for defaults). */
typedef struct {
  int32_t n_split;   /* 0: automatic; otherwise the number of partitions of each
                        row's selected tokens in the attention pass (clamped to
                        the range the workspace was sized for) */
  uint32_t flags;    /* DS_DECODE_* */
  hipEvent_t* stage_events; /* NULL, or DS_STAGE_COUNT + 1 event slots (NULL
                               slots are skipped).  When exactly two adjacent
                               slots i and i + 1 are given, stage i's kernel
                               launch records them at the kernel's own start
                               and end (a stage that launches nothing records
                               them back to back); on the one-kernel path that
                               launch is the attention stage's.  Otherwise
                               event i is recorded on `stream` before stage i
                               and the last one after the final stage (stages
                               that launch nothing give empty intervals). */
} ds_decode_opts;

/* Kernel paths of ds_decode_attn. */
enum {
  DS_PATH_DENSE = 0,  /* k <= 0: attention over every token, no label read */
  DS_PATH_FUSED = 1,  /* one kernel per step: one workgroup per (batch, KV head)
                         row appends, scores, selects and attends (rows of up
                         to 6144 tokens for single-head groups, 16384 for
                         groups of 2 to 8 query heads; k <= 2048) */
  DS_PATH_LOCAL = 2,  /* chunked scores with a local top-M per chunk, an exact
                         merge per row, split attention, merge of splits */
  DS_PATH_STREAM = 3  /* every score streamed to the workspace, a radix select
                         per row, split attention, merge of splits */
};

/* What a ds_decode_attn call with these arguments runs (host struct, filled
 * by ds_decode_attn_plan). */
typedef struct {
  int32_t path;             /* DS_PATH_* */
  int32_t n_split;          /* partitions of each row's tokens in the attention pass */
  int32_t tokens_per_split; /* at most this many tokens per partition */
  int32_t kernels;          /* kernel launches per call */
  int32_t chunk;            /* tokens per scoring workgroup (local and stream
                               paths; 0 otherwise) */
  int32_t reserved0;
  size_t workspace_bytes;   /* as ds_decode_attn_workspace_size */
} ds_decode_plan;

/* Workspace bytes that ds_decode_attn needs for these arguments (0 if they
 * are invalid).  Depends only on the shapes, k and max_seq_len. */
size_t ds_decode_attn_workspace_size(const ds_kv_desc* kv, const ds_label_desc* lab, int32_t k,
                                     int32_t max_seq_len);

/* One Double Sparsity decode step over all (batch, KV head) rows
 * ([DS] online forward computation, steps 1-3):
 *   1. qg[j] = sum over the group's query heads h of q[b][h][keep[g][chan[g][j]]]
 *      (the group shares one token set, so its approximate score is read as
 *      the sum of its heads' scores);
 *   2. s[t] = sum_j qg[j] * label[b][g][t][j] (INT4: scale[t] * sum_j qg[j] *
 *      code[t][j]) for t < S = seq_lens[b];
 *   3. T = the min(k, S) tokens with the largest s, ties to the lower index;
 *      each query head h of the group then gets exact softmax attention
 *      o_h = sum_{t in T} softmax_t(sm_scale * q_h . K_t) V_t, with q_h read at
 *      keep[g][c] for stored K column c ([LeanK] section 2.2).
 * With k <= 0 every row attends all S tokens and no label is read (chan and
 * lab may be NULL, unless DS_DECODE_APPEND is set: a dense step still appends
 * the current token's label, so later sparse steps find the cache current);
 * with k >= S that row attends all its tokens (the dense fallback of [DS]
 * "use in SGLang").  A row with S = 0 gets a zero output.
 *   q           fp16 [batch][n_q_heads][d_q].
 *   K, V        the caches (kv); the current token must already be written.
 *               They may be device memory or pinned host memory that HIP maps
 *               into the device's address space at its host address
 *               (hipHostMalloc): the kernels then read only the selected rows
 *               (and the appended token's K row) over the host link ([DS]
 *               "experiment details": the offloading variant).
 *   seq_lens    int32 [batch] device array: tokens per row, current included.
 *   max_seq_len host upper bound of seq_lens (sizes the grid), <= capacity.
 *   keep        int32 [n_kv_heads][d_k] device array: query channel of each
 *               stored K column (LeanK); NULL means column c is channel c
 *               (then d_k must equal d_q).
 *   chan, lab   heavy channels and label cache as for ds_label_build.
 *   sm_scale    softmax scale (e.g. 1/sqrt(head dim)).
 *   out         fp16 [batch][n_q_heads][d_v]; fp32 accumulation.
 *   topk_idx    NULL, or int32 [batch][n_kv_heads][k] receiving each row's
 *               selected tokens in ascending order, padded with -1.
 *   workspace   device scratch of at least ds_decode_attn_workspace_size()
 *               bytes, 256-byte aligned; contents need no initialisation.
 * Errors: DS_ERR_ARG, DS_ERR_SHAPE, DS_ERR_DTYPE, DS_ERR_ALIGN,
 * DS_ERR_WORKSPACE, DS_ERR_HIP. */
ds_status ds_decode_attn(const ds_kv_desc* kv, const void* q, const void* K, const void* V,
                         const int32_t* seq_lens, int32_t max_seq_len, const int32_t* keep,
                         const int32_t* chan, const ds_label_desc* lab, int32_t k, float sm_scale,
                         void* out, int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                         const ds_decode_opts* opts, hipStream_t stream);

/* Scratch bytes of ds_decode_attn_noalloc (per GPU). */
#define DS_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* ds_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It takes the same arguments, launches
 * the same kernels and gives the same results as ds_decode_attn; the scratch
 * that ds_decode_attn takes from the caller's workspace comes instead from a
 * device array of DS_NOALLOC_SCRATCH_BYTES that the library holds on each GPU
 * from the first use of the library there until the process ends.  The call
 * allocates nothing.  Its first call on a device (the device current at the
 * call, which must be the device of `stream`) looks up that array's address.
 * Every call on a GPU shares the one array: calls that overlap on one GPU
 * (other streams, other threads) race on it and give undefined results; the
 * caller orders them.  The scratch needs no clearing between calls (each call
 * writes what it reads).
 * Errors: those of ds_decode_attn; DS_ERR_WORKSPACE when these shapes need
 * more than DS_NOALLOC_SCRATCH_BYTES (as ds_decode_attn_workspace_size
 * reports); DS_ERR_HIP when the array's address cannot be found. */
ds_status ds_decode_attn_noalloc(const ds_kv_desc* kv, const void* q, const void* K,
                                 const void* V, const int32_t* seq_lens, int32_t max_seq_len,
                                 const int32_t* keep, const int32_t* chan,
                                 const ds_label_desc* lab, int32_t k, float sm_scale, void* out,
                                 int32_t* topk_idx, const ds_decode_opts* opts,
                                 hipStream_t stream);

/* Host-only query: fills *plan for a ds_decode_attn call with these shapes,
 * k, max_seq_len and options (no device pointer is read and nothing is
 * enqueued).  Errors: DS_ERR_ARG (plan NULL, max_seq_len or n_split out of
 * range) and the shape and dtype errors of ds_decode_attn. */
ds_status ds_decode_attn_plan(const ds_kv_desc* kv, const ds_label_desc* lab, int32_t k,
                              int32_t max_seq_len, const ds_decode_opts* opts,
                              ds_decode_plan* plan);

/* Batch policy of [DS] "use in SGLang" (the sparse-decode threshold): a
 * batch decodes with Double Sparsity only when k > 0, its longest sequence
 * has at least `threshold` tokens and its shortest at least k; otherwise the
 * whole batch decodes densely (ds_decode_attn with k <= 0, which may still
 * append labels).  Host-only; returns 1 (sparse) or 0 (dense). */
int32_t ds_sparse_decode_enabled(int32_t max_seq_len, int32_t min_seq_len, int32_t k,
                                 int32_t threshold);

/* Agreement of two heavy-channel tables, [DS] "offline calibration" (the
 * article compares the outlier channels fixed offline with those an online
 * pass finds, by the share they have in common).  chan_a, chan_b: host
 * int32 [n_kv_heads][r], read only; overlap: host float [n_kv_heads],
 * written: for head g, the number of distinct channels of chan_a[g] that
 * chan_b[g] also holds, divided by r.  Host-only: no device memory, nothing
 * enqueued, nothing allocated.  Errors: DS_ERR_ARG (a pointer NULL, n_kv_heads
 * or r below 1, a channel id outside [0, 4096)). */
ds_status ds_channel_overlap(const int32_t* chan_a, const int32_t* chan_b, int32_t n_kv_heads,
                             int32_t r, float* overlap);

/* Heavy-channel calibration criteria ([DS] offline calibration: channels
 * found from outliers of K, of the query, or of their product). */
typedef enum { DS_CALIB_K = 0, DS_CALIB_Q = 1, DS_CALIB_QK = 2 } ds_calib_criterion;

/* Workspace bytes that ds_calibrate_channels needs for kv's batch, KV heads
 * and d_k (and n_q_heads when n_win > 0), n_tok sample tokens and n_win
 * window queries (0 if the arguments are invalid). */
size_t ds_calibrate_workspace_size(const ds_kv_desc* kv, int32_t n_tok, int32_t n_win);

/* Heavy-channel calibration ([DS] offline calibration: the channels that
 * move the attention scores most are chosen once from a few samples;
 * [LeanK] section 1.1: a channel's importance is the L2 norm of the product
 * of the observation window's query column and the key column).  For KV
 * head g and stored K column c, with query channel qc = keep[g][c] (or c):
 *   kn_b = sum_{t < n_tok} K[b][g][t][c]^2       (sample b = batch row b)
 *   qn_b = sum_{w < n_win} sum_{h of group g} qwin[b][w][h][qc]^2
 *   DS_CALIB_K:  score = sum_b kn_b
 *   DS_CALIB_Q:  score = sum_b qn_b
 *   DS_CALIB_QK: score = sqrt(sum_b qn_b kn_b), the Frobenius norm of the
 *                per-sample rank-one products Q_b[c] K_b[c]^T taken together.
 * chan[g] receives the r columns with the largest score (ties to the lower
 * column) in ascending order: a table ds_label_build accepts.  Sums are fp32
 * in a fixed order, so a call repeats bit for bit.
 *   K       fp16 K cache (kv: batch, n_kv_heads, d_k, capacity, k_stride are
 *           read); tokens t < n_tok <= capacity count.
 *   qwin    fp16 [batch][n_win][n_q_heads][d_q] window queries, contiguous
 *           (kv's n_q_heads and d_q are read when n_win > 0); n_win may be 0
 *           (then qn = 0).
 *   keep    int32 [n_kv_heads][d_k] device array with entries in [0, d_q),
 *           or NULL (then d_k <= d_q); entries are not checked on the device.
 *   chan    int32 [n_kv_heads][r] device output, 1 <= r <= d_k.
 *   norms   NULL, or fp32 [n_kv_heads][3][d_k] device output: sum_b kn_b,
 *           sum_b qn_b and the score (a NaN score is reported as -1 and
 *           ranks last).
 *   workspace  device scratch of ds_calibrate_workspace_size() bytes.
 * K must be plain contiguous rows (page_size 0, no per-head layout).
 * Errors: DS_ERR_ARG (null pointer, n_tok, n_win, r or criterion out of
 * range, a paged kv), DS_ERR_SHAPE, DS_ERR_ALIGN (K not 16-byte aligned,
 * stride not a multiple of 8), DS_ERR_WORKSPACE, DS_ERR_HIP. */
ds_status ds_calibrate_channels(const ds_kv_desc* kv, const void* K, int32_t n_tok,
                                const void* qwin, int32_t n_win, const int32_t* keep,
                                int32_t criterion, int32_t r, int32_t* chan, float* norms,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code, any int32 value ("unknown status" for one
 * that is not a ds_status; never NULL). */
const char* ds_status_str(int32_t status);

/* DS_ABI_VERSION of the loaded library. */
int32_t ds_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DS_H_ */
