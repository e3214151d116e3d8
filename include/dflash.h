/*
 * dflash.h - C ABI of the DFlash KV-injection attention library (gfx950).
 *
 * The layer (sources cited by page title and section):
 *   "DFlash KV Injection Walkthrough", Step 2: the k concatenated target-layer
 *     hidden states of each position go through fc (no bias) and an RMSNorm,
 *     giving the context C shared by every draft layer.
 *   Same page, Step 4.1-4.5, and "DFlash源码导读二 Qwen3DFlashAttention注意力实现全解析"
 *     sections 1-5: Q from the block rows H only; K = k_proj([C; H]),
 *     V = v_proj([C; H]) with one weight for both streams; per-head RMSNorm on
 *     Q and K; RoPE over one window of positions with the queries on its last
 *     B positions; non-causal GQA attention with scale d_h^-0.5 over the draft
 *     KV cache; o_proj.
 *   Same article, section 4: the round's rows are written into the draft cache,
 *     which is later cut back to the accepted prefix.
 *   "KV Cache + Speculative Decoding 面试 Cheat Sheet", sections 5.2-5.3, 6.2:
 *     fixed-size pages, per-request page tables, a free list.
 *
 * Conventions for every entry point:
 *   - Returns DFLASH_OK (0) or a negative dflash_status; never throws.
 *   - Device pointers are caller-owned device memory; host pointers are read
 *     during the call only.  The library allocates no device memory and never
 *     frees caller memory.  Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously on it; no call synchronises the device.
 *   - All arguments are validated on the host before anything is enqueued, so
 *     a call that returns an error has changed no state.
 *   - Storage dtype is DFLASH_F32 or DFLASH_BF16 for every tensor of a call
 *     (a BF16 layer may keep its cache in DFLASH_FP8_E4M3); accumulation is
 *     always fp32.  Matrices are row-major, innermost dimension contiguous.
 *   - A cache handle is used from one stream at a time.  Calls that overlap on
 *     one workspace race.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_ERR_ARG = -1,       /* null / misaligned pointer, bad handle, bad cu array, bad fp8 scale */
  DFLASH_ERR_SHAPE = -2,     /* unsupported or inconsistent sizes */
  DFLASH_ERR_DTYPE = -3,     /* unsupported dtype, or a cache dtype the layer cannot use */
  DFLASH_ERR_RANGE = -4,     /* crop outside [0, current length]; window beyond a ring's rows */
  DFLASH_ERR_CAPACITY = -5,  /* sequence capacity, page table or page pool exhausted */
  DFLASH_ERR_HIP = -6,       /* a HIP runtime call or kernel launch failed */
  DFLASH_ERR_WORKSPACE = -7  /* workspace smaller than the *_ws_bytes figure */
} dflash_status;

/* DFLASH_FP8_E4M3 is a cache dtype only: one byte per K/V element, see the
 * cache descriptor. */
typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1, DFLASH_FP8_E4M3 = 2 } dflash_dtype;

/* Limits of the library. */
#define DFLASH_MAX_SEQS 64        /* requests per cache handle */
#define DFLASH_MAX_GROUP_ROWS 64  /* (n_h / n_kv) * B query rows per K/V head */
#define DFLASH_KEY_ALIGN 64       /* contiguous capacity and page size are multiples of this */

/* ------------------------------------------------------------------------
 * One KV-injection attention layer.  All weight pointers are device memory in
 * the layer dtype.
 *   w_qkv   [(n_h + 2*n_kv) * d_h, d]: rows W_Q (n_h*d_h) | W_K | W_V, each
 *           stored output x input; row h*d_h + i is output i of head h.
 *   w_o     [d, n_h * d_h], output x input (input column h*d_h + i = head h).
 *   gamma_q, gamma_k [d_h]: per-head RMSNorm gains shared by all heads.
 * Shapes: n_h % n_kv == 0, d_h in {64, 128}, (n_h/n_kv)*B <= 64, d % 8 == 0.
 * window 0 = full attention; window > 0 = sliding layer where query position
 * p sees key position j iff p - j < window (no upper bound).
 * residual 1 adds the block rows H to the output, so that in a stack of layers
 * sharing one context C the output of layer l is the block input of layer l+1
 * (H_{l+1} = H_l + o_proj_l; the decoder internals between layers are not part
 * of this library).
 * ---------------------------------------------------------------------- */
typedef struct dflash_layer_desc {
  int32_t d, n_h, n_kv, d_h;
  float eps;            /* RMSNorm epsilon (Q/K norms) */
  double rope_theta;    /* RoPE base; w_i = theta^(-2i/d_h) */
  int32_t window;
  int32_t dtype;        /* dflash_dtype */
  int32_t residual;     /* 0: out = o_proj(attn); 1: out = H + o_proj(attn), the
                           chaining of a layer stack (the next layer's block rows) */
  const void *w_qkv;
  const void *w_o;
  const void *gamma_q;
  const void *gamma_k;
} dflash_layer_desc;

/* ------------------------------------------------------------------------
 * Draft KV cache.  Pools and the page table are caller-owned device buffers;
 * the handle owns host metadata only (lengths, page lists, free list).
 *
 * contiguous (page_size == 0): capacity = rows per sequence (multiple of 64)
 *     K pool [n_seqs][n_kv][capacity][d_h]
 *     V pool [n_seqs][n_kv][capacity / 64][d_h][64]
 * paged (page_size > 0, multiple of 64): capacity = pages in the pool
 *     K pool [capacity][n_kv][page_size][d_h]
 *     V pool [capacity][n_kv][page_size / 64][d_h][64]
 * V is stored transposed in tiles of 64 slots: head dim i of slot j sits in
 * tile j / 64, row i, column j % 64, so the 64 keys of an attention block are
 * one contiguous run whatever the capacity or page size.
 *     block_table [n_seqs][max_pages_per_seq] int32, device; entry (s, j) is the
 *     physical page of logical page j of sequence s, valid for
 *     j < ceil(len_s / page_size) (other entries are left as they were).
 * Row `pos` of sequence s sits in logical page pos / page_size, slot
 * pos % page_size.  K rows hold post-norm post-RoPE keys; V rows raw values.
 * Allocation takes the lowest-numbered free page, sequences in index order,
 * each sequence's logical pages in order.  Crop returns every page at or
 * beyond ceil(new_len / page_size) to the free list.
 *
 * ring (contiguous only, for sliding-window layers): the cache keeps the last
 * `capacity` positions of each sequence, row pos in slot pos % capacity, so
 * lengths may exceed the capacity and memory stays O(window) however long
 * the context grows (the bounded cache of a sliding layer, "DFlash源码导读二
 * Qwen3DFlashAttention注意力实现全解析", the MLX comparison: a rotating cache
 * trimmed like the full one is cropped).  Let hw_s be the highest position
 * ever written to sequence s, plus one; positions below hw_s - capacity are
 * gone.  Each append call may bring at most `capacity` rows per sequence.  A
 * layer call on a ring needs window > 0, capacity >= window + B - 1,
 * n_s + B <= capacity, and every key the window reaches still held
 * (max(0, L_s + n_s - window + 1) >= hw_s - capacity; else DFLASH_ERR_RANGE).
 * Crop is unchanged: it sets the length, and later appends overwrite slots.
 *
 * fp8 (dtype DFLASH_FP8_E4M3, for BF16 layers; "KV Cache + Speculative
 * Decoding 面试 Cheat Sheet" 2.1 and 4.5: one byte per cached element instead
 * of two): every pool element is an OCP FP8 E4M3 byte (sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; no infinities, S.1111.111 is NaN, the largest
 * value 448).  A key element x is stored as the E4M3 value nearest x / k_scale
 * (ties to the even mantissa, magnitudes from 448 up saturated) and read as
 * that value times k_scale; values use v_scale.  The pools take 1 byte per
 * element in the same layouts; dflash_cache_append moves such bytes as they
 * are.  Both scales must be finite and > 0 (else DFLASH_ERR_ARG); other
 * dtypes ignore them.
 * ---------------------------------------------------------------------- */
typedef struct dflash_cache_desc {
  int32_t n_seqs, n_kv, d_h;
  int32_t dtype;               /* DFLASH_F32, DFLASH_BF16 or DFLASH_FP8_E4M3 */
  int32_t page_size;
  int32_t max_pages_per_seq;   /* paged only */
  int32_t ring;                /* 0 or 1 (contiguous only): keep the last `capacity` positions */
  int64_t capacity;
  void *k_pool;
  void *v_pool;
  int32_t *block_table;        /* paged only, device */
  float k_scale, v_scale;      /* DFLASH_FP8_E4M3 only */
} dflash_cache_desc;

typedef struct dflash_cache dflash_cache;

/* Create a handle with every sequence empty.  The pools are not touched. */
int dflash_cache_init(dflash_cache **out, const dflash_cache_desc *desc);
int dflash_cache_destroy(dflash_cache *c);
/* Host copies of the metadata (no device access, no synchronisation). */
int dflash_cache_lengths(const dflash_cache *c, int32_t *host_len /* [n_seqs] */);
/* [n_seqs][max_pages_per_seq], -1 where no page is mapped; contiguous caches
 * report entry (s, 0) = s. */
int dflash_cache_block_table(const dflash_cache *c, int32_t *host_table);
int64_t dflash_cache_free_pages(const dflash_cache *c);

/* ------------------------------------------------------------------------
 * Context projection ("DFlash KV Injection Walkthrough", Step 2):
 *   C[t] = RMSNorm(X_raw[t] . W_fc^T) * gamma_h,  RMSNorm over d.
 *   x_raw   [T, kd] device (each row = k layer vectors in layer order)
 *   w_fc    [d, kd] device (output x input; no bias)
 *   gamma_h [d] device
 *   c_out   [T, d] device, written in `dtype`
 *   ws      device workspace of at least dflash_ctx_project_ws_bytes(...),
 *           a figure that holds for every call with at most T rows
 * T == 0 is a no-op.  kd % 8 == 0, d % 8 == 0, d <= 16384.
 * ---------------------------------------------------------------------- */
size_t dflash_ctx_project_ws_bytes(int64_t T, int64_t kd, int64_t d, int32_t dtype);
int dflash_ctx_project(const void *x_raw, int64_t T, int64_t kd, const void *w_fc,
                       const void *gamma_h, int64_t d, float eps, int32_t dtype,
                       void *c_out, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Raw append ("DFlash源码导读二 ..." section 4, the cache update): rows
 * [cu_rows[s], cu_rows[s+1]) of k_rows / v_rows [n_rows, n_kv, d_h] (device,
 * cache dtype) land at positions len_s .. len_s + n_s - 1 of sequence s, then
 * len_s += n_s.  cu_rows is a host array [n_seqs + 1], non-decreasing from 0.
 * Bytes are copied unchanged.  Capacity, page-table or pool overflow (for a
 * ring: more than `capacity` rows for one sequence) -> DFLASH_ERR_CAPACITY
 * with nothing written.
 * ---------------------------------------------------------------------- */
int dflash_cache_append(dflash_cache *c, const int32_t *cu_rows, const void *k_rows,
                        const void *v_rows, void *stream);

/* ------------------------------------------------------------------------
 * Crop to the accepted prefix ("DFlash KV Injection Walkthrough", Step 7;
 * "DFlash源码导读二 ..." section 4): len_s = new_len[s] (host [n_seqs]).
 * Requires 0 <= new_len[s] <= len_s for every s, else DFLASH_ERR_RANGE and
 * no change.  Retained rows are untouched.  Host metadata only: nothing is
 * enqueued on `stream`.
 * ---------------------------------------------------------------------- */
int dflash_cache_crop(dflash_cache *c, const int32_t *new_len, void *stream);

/* ------------------------------------------------------------------------
 * One KV-injection attention layer for every sequence of the cache
 * ("DFlash KV Injection Walkthrough", Step 4; "DFlash源码导读二 ..." 1-5).
 *   C      [T, d] device: new context rows, sequence r owns rows
 *          [cu_ctx[r], cu_ctx[r+1]) (cu_ctx: host [n_seqs + 1]); n_r >= 0.
 *   H      [n_seqs * B, d] device: block rows, sequence r owns rows r*B .. r*B+B-1.
 *   out    [n_seqs * B, d] device: o_proj output of the block rows (plus H when
 *          the layer has residual set; out may then be the same buffer as H).
 * For each sequence r with cache length L_r: the n_r + B new K/V rows get RoPE
 * positions L_r .. L_r+n_r+B-1 (context rows first), the queries the last B of
 * them; all n_r + B rows are appended (len_r = L_r + n_r + B), then the
 * queries attend over all len_r keys.  The caller crops afterwards (to
 * L_r + n_r to keep the accepted context).  Needs ws of at least
 * dflash_kv_inject_attn_ws_bytes(L, cache, T, B) bytes; the figure depends on
 * T, B and the handle's sizes, not on the current lengths, and holds for
 * every call with at most T context rows.  The cache dtype equals the layer
 * dtype, or is DFLASH_FP8_E4M3 under a BF16 layer (else DFLASH_ERR_DTYPE):
 * the new K/V rows are then stored as fp8 and attention reads every key and
 * value as its fp8 value times the cache's scale.
 * ---------------------------------------------------------------------- */
size_t dflash_kv_inject_attn_ws_bytes(const dflash_layer_desc *L, const dflash_cache *c,
                                      int64_t T, int32_t B);
int dflash_kv_inject_attn(const dflash_layer_desc *L, dflash_cache *c, const void *C,
                          const int32_t *cu_ctx, const void *H, int32_t B, void *out,
                          void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Device-driven rounds ("DFlash KV Injection Walkthrough", Steps 6 and 7: the
 * acceptance of a round fixes how many context rows the next one injects and
 * where the cache is cut back; here both stay in device memory, so a whole
 * sequence of rounds runs without the host reading anything and can be
 * captured in one HIP graph).
 *
 * dflash_cache_device_begin puts a contiguous or paged cache (not a ring:
 * DFLASH_ERR_SHAPE) in device mode: its lengths are written to d_len
 * (device int32 [n_seqs], caller-owned, 4-byte aligned) and from then on
 * d_len holds them; the host keeps upper bounds of them, counting every
 * round with its largest number of new rows.  In device mode the host-mode
 * calls on the cache (dflash_cache_append, dflash_cache_crop and both
 * dflash_kv_inject_attn forms) return DFLASH_ERR_ARG, and
 * dflash_cache_lengths / dflash_cache_block_table report the bounds and the
 * pages reserved for them.
 *
 * dflash_kv_inject_attn_dev is dflash_kv_inject_attn for a round whose new
 * context row counts are d_rows (device int32 [n_seqs], each in 0..n_max,
 * e.g. the next_rows of dflash_accept): C holds n_seqs * n_max rows, sequence
 * r's at rows r * n_max .. r * n_max + d_rows[r] - 1 (the rest are read by the
 * projection and otherwise ignored); the n + B new rows of each sequence take
 * positions d_len[r] .. as in the host form, and d_len[r] grows by
 * d_rows[r] + B.  Capacity, page reservation and the attention split are
 * planned for the bounds: a call that would not fit if every sequence had
 * n_max new rows returns DFLASH_ERR_CAPACITY with nothing enqueued.  The
 * kernels clamp each d_rows value to 0..n_max (it is on the device, so the
 * host cannot check it): a count out of range acts as the nearest bound.
 * Workspace: dflash_kv_inject_attn_dev_ws_bytes(L, c, n_max, B).
 *
 * dflash_cache_crop_tail_dev cuts `drop` rows off every sequence on the
 * device (d_len[r] = max(0, d_len[r] - drop); drop = B after a layer call is
 * the cut back to the block start, the accepted prefix) and the bounds with
 * them.
 *
 * dflash_cache_device_reset writes host_len (host [n_seqs]) into d_len on
 * the device, each at most the current bound (else DFLASH_ERR_RANGE, nothing
 * enqueued); the bounds stay.  Captured at the start of a graph of rounds, it
 * makes every replay start from the same lengths.
 *
 * dflash_cache_device_end synchronises `stream`, reads d_len back, makes the
 * host metadata exact (pages past the true lengths return to the free list)
 * and leaves device mode; a length outside 0..bound reports
 * DFLASH_ERR_RANGE and leaves the cache in device mode.
 * ---------------------------------------------------------------------- */
int dflash_cache_device_begin(dflash_cache *c, int32_t *d_len, void *stream);
size_t dflash_kv_inject_attn_dev_ws_bytes(const dflash_layer_desc *L, const dflash_cache *c, int32_t n_max,
                                          int32_t B);
int dflash_kv_inject_attn_dev(const dflash_layer_desc *L, dflash_cache *c, const void *C, int32_t n_max,
                              const int32_t *d_rows, const void *H, int32_t B, void *out, void *ws, size_t ws_bytes,
                              void *stream);
int dflash_cache_crop_tail_dev(dflash_cache *c, int32_t drop, void *stream);
int dflash_cache_device_reset(dflash_cache *c, const int32_t *host_len, void *stream);
int dflash_cache_device_end(dflash_cache *c, void *stream);

/* ------------------------------------------------------------------------
 * The same layer call without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, results and errors are those
 * of dflash_kv_inject_attn; the workspace is a scratch buffer the library
 * holds on each GPU it runs on, DFLASH_NOALLOC_SCRATCH_BYTES bytes from the
 * first such call on that GPU until the process ends.  The call allocates
 * nothing and creates no events (stage timing does not record it).  A call
 * whose own needs (the q/k/v partial products of its rows, the attention
 * partials of its planned split, the o_proj partials) exceed the buffer
 * returns DFLASH_ERR_WORKSPACE with nothing enqueued; at the Qwen3-8B shapes a
 * batch-1 decode round on caches of up to 64K keys needs about 15-30 MB.
 * Every call on one GPU uses that GPU's one buffer: calls that overlap on a
 * GPU (other streams or threads, or a graph replayed while another call runs)
 * race.  Nothing in the buffer is expected to hold a value across calls.
 * ---------------------------------------------------------------------- */
#define DFLASH_NOALLOC_SCRATCH_BYTES (64u << 20)
int dflash_kv_inject_attn_noalloc(const dflash_layer_desc *L, dflash_cache *c, const void *C,
                                  const int32_t *cu_ctx, const void *H, int32_t B, void *out, void *stream);

/* ------------------------------------------------------------------------
 * Draft head ("DFlash KV Injection Walkthrough", Step 5): after the last draft
 * layer, every request's block rows go through a final RMSNorm over d (gain
 * gamma_f, the formula of hidden_norm), the last B-1 of them (row 0 holds the
 * already-known token, whose prediction is dropped) through lm_head, and
 * greedy sampling keeps the argmax over the vocabulary.
 *   h         [R*B, d] device: the stack's output rows of the blocks
 *   gamma_f   [d] device
 *   w_lm      [vocab, d] device (output x input, no bias)
 *   token_ids [R*(B-1)] int32 device: entry r*(B-1)+j = the draft token of
 *             block position j+1 of request r, the first maximal logit
 *   max_logit [R*(B-1)] float device, or NULL: that logit
 *   ws        device workspace of at least dflash_draft_head_ws_bytes(R, B, d,
 *             vocab, dtype) bytes
 * Logits accumulate in fp32 from operands in the storage dtype (the normed
 * rows are stored in it).  B == 1 (nothing to predict) is a no-op.
 * d % 8 == 0, d <= 16384, vocab % 4 == 0, vocab < 2^30.
 * ---------------------------------------------------------------------- */
size_t dflash_draft_head_ws_bytes(int64_t R, int32_t B, int64_t d, int64_t vocab, int32_t dtype);
int dflash_draft_head(const void *h, int64_t R, int32_t B, int64_t d, const void *gamma_f, float eps,
                      const void *w_lm, int64_t vocab, int32_t dtype, int32_t *token_ids, float *max_logit,
                      void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Acceptance of a speculative round ("DFlash KV Injection Walkthrough", Step 6
 * and Step 7), computed on the device so that the round's results stay there:
 *   draft_ids   [R*(B-1)] int32 device: entry r*(B-1)+j = the draft token of
 *               block position j+1 of request r (the token_ids layout of
 *               dflash_draft_head)
 *   posterior   [R*B] int32 device: entry r*B+j = the target's prediction of
 *               the token after block position j of request r
 *   acc         [R] int32 device: the number of leading draft tokens equal to
 *               the target's prediction from the position before (the
 *               cumulative product of the matches, summed; 0..B-1)
 *   next_rows   [R] int32 device, or NULL: acc + 1, the context rows the next
 *               round injects (the accepted positions and the corrected one)
 *   next_anchor [R] int32 device, or NULL: the target's token at the first
 *               position not accepted (posterior[r*B + acc]), which opens the
 *               next round's block
 * R == 0 is a no-op; B >= 1 (B == 1: nothing was drafted, acc = 0); R < 2^31.
 * Pointers 4-byte aligned (else DFLASH_ERR_ARG).  Asynchronous on `stream`.
 * ---------------------------------------------------------------------- */
int dflash_accept(const int32_t *draft_ids, const int32_t *posterior, int64_t R, int32_t B, int32_t *acc,
                  int32_t *next_rows, int32_t *next_anchor, void *stream);

const char *dflash_strerror(int status);

/* ------------------------------------------------------------------------
 * Stage timing (a measurement aid, off by default).  While enabled, the
 * kernels of every stage a call enqueues carry a pair of HIP events
 * (hipExtLaunchKernel start/stop events): the first kernel's start and the
 * last kernel's end as the GPU executes them, so a stage's time excludes the
 * dispatch gaps before it.  dflash_timing_read waits for the recorded events
 * (it synchronises with them, never with the whole device), folds them into
 * per-stage totals and reports the launches and summed milliseconds of one
 * stage since the last reset.  Process-wide; thread-safe.  Stages that launch
 * nothing (e.g. T == 0) are not recorded.
 * ---------------------------------------------------------------------- */
typedef enum {
  DFLASH_STAGE_CTX_GEMM = 0,     /* fc: X_raw . W_fc^T, split-K partials */
  DFLASH_STAGE_CTX_REDUCE = 1,   /* reserved: the fc split-K sum is fused into CTX_NORM */
  DFLASH_STAGE_CTX_NORM = 2,     /* fc split-K sum fused with hidden_norm */
  DFLASH_STAGE_QKV_GEMM = 3,     /* q_proj of H, k_proj/v_proj of [C; H] */
  DFLASH_STAGE_QKV_EPILOGUE = 4, /* QK-norm, RoPE, Q to workspace, K/V to cache */
  DFLASH_STAGE_ATTN = 5,         /* split-context block attention */
  DFLASH_STAGE_ATTN_COMBINE = 6, /* merge of the split partials */
  DFLASH_STAGE_O_GEMM = 7,       /* o_proj split-K partials */
  DFLASH_STAGE_O_REDUCE = 8,     /* o_proj reduction and store */
  DFLASH_STAGE_CACHE_APPEND = 9, /* dflash_cache_append copy */
  DFLASH_STAGE_PAGE_TABLE = 10,  /* device page-table and device-length updates */
  DFLASH_STAGE_HEAD_NORM = 11,   /* draft head: final RMSNorm of the block tails */
  DFLASH_STAGE_HEAD_GEMM = 12,   /* draft head: lm_head product */
  DFLASH_STAGE_HEAD_ARGMAX = 13, /* draft head: argmax over the vocabulary */
  DFLASH_STAGE_ACCEPT = 14,      /* acceptance of a round */
  DFLASH_STAGE_STREAM_READ = 15, /* dflash_stream_read (measurement) */
  DFLASH_STAGE_MFMA_PEAK = 16,   /* dflash_mfma_peak (measurement) */
  DFLASH_STAGE_COUNT = 17
} dflash_stage;

int dflash_timing_enable(int on);
int dflash_timing_read(int32_t stage, int64_t *launches, double *total_ms);
int dflash_timing_reset(void);

/* ------------------------------------------------------------------------
 * A plain streaming read (a measurement aid): reads the first bytes / 16
 * 16-byte words at src (device memory, 16-byte aligned) and writes nothing
 * (sink, a device word or NULL, is only written in a case no input meets in
 * practice).  Timed as DFLASH_STAGE_STREAM_READ, it gives the HBM read rate
 * one launch of that size reaches, beside which the layer's bandwidth-bound
 * kernels are judged.  bytes < 0 -> DFLASH_ERR_SHAPE; misaligned src ->
 * DFLASH_ERR_ARG.
 * ---------------------------------------------------------------------- */
int dflash_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

/* ------------------------------------------------------------------------
 * A matrix-core rate probe (a measurement aid): `workgroups` workgroups of
 * four waves, each wave 8 * iters bf16 16x16x32 MFMAs on register operands
 * (16384 flops each), nothing read and nothing written (sink, a device float
 * or NULL, is only written in a case no run meets).  Timed as
 * DFLASH_STAGE_MFMA_PEAK, it gives the bf16 MFMA rate this GPU sustains at its
 * clocks under load, beside which the projections' TFLOP/s are judged.
 * iters in 1..2^24 and workgroups in 1..2^20 (else DFLASH_ERR_SHAPE).
 * ---------------------------------------------------------------------- */
int dflash_mfma_peak(int32_t iters, int64_t workgroups, float *sink, void *stream);

/* ------------------------------------------------------------------------
 * GEMM plan inspection (a diagnostic, host only: nothing is enqueued).  The
 * projections of every entry point above (fc, q/k/v, o_proj, lm_head) are
 * products of M activation rows with a [N][K] weight; this reports the
 * kernel and the decomposition the library picks for one such product:
 *   out[0] kernel: DFLASH_GEMM_* below
 *   out[1] K-splits (fp32 partial products written for the consumer; 1 for
 *          the kernels that write the result directly)
 *   out[2] K-chunk per split
 *   out[3] output-column tiles (per 16-row problem set)
 *   out[4] columns per tile (256/128/64 for the tile kernel, else 0)
 *   out[5] rows per weight-streaming problem (products of more rows are done
 *          as several problems; 0 for the tile kernel)
 * dtype as for the layer calls.  Returns DFLASH_ERR_ARG for a null out,
 * DFLASH_ERR_SHAPE unless M, N, K >= 1, DFLASH_ERR_DTYPE for other dtypes.
 * ---------------------------------------------------------------------- */
typedef enum {
  DFLASH_GEMM_LDS = 0,       /* activation slice in up to 64 KB of LDS, fp32 or other K */
  DFLASH_GEMM_WIDE = 1,      /* <= 32 rows, K >= 8192: activation from L2 */
  DFLASH_GEMM_STREAM = 2,    /* <= 64 rows, K < 8192: per-wave weight rings */
  DFLASH_GEMM_FULLK = 3,     /* <= 16 rows: whole K per workgroup, no partials */
  DFLASH_GEMM_RESIDENT = 4,  /* <= 16 rows, >= 65536 columns: rows kept in LDS */
  DFLASH_GEMM_SLAB = 5,      /* 65..128 rows (33..64 at K >= 8192): slice staged in up to 160 KB of LDS */
  DFLASH_GEMM_TILE = 6       /* many rows: 256 x 256/128/64 MFMA tiles */
} dflash_gemm_kernel;
int dflash_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t *out /* [6] */);

/* ------------------------------------------------------------------------
 * Attention split inspection (a diagnostic, host only).  A layer call splits
 * the keys each query block attends to into work items of `chunk` keys per
 * (sequence, K/V head); this reports that split for given key counts:
 *   keys      [R] host: keys of sequence r, counted from its first visible
 *             key rounded down to a multiple of 64 (each >= 1)
 *   chunk_cap the largest chunk the cache allows (paged: 62 pages; ring:
 *             62 capacities; otherwise any value >= 2^30)
 *   cache_dtype the cache's dtype, a dflash_dtype value: fp8 caches fit more items
 *             per round
 *   out[0] chunk (keys per item, a multiple of 64, >= 128)
 *   out[1] items (sum over sequences of max(1, ceil(keys/chunk)) * n_kv)
 *   out[2] ring depth planned for the 64-key-block kernels (3: one workgroup
 *          per CU, 2: several)
 * Returns DFLASH_ERR_ARG for null pointers, DFLASH_ERR_DTYPE for an unknown
 * dtype, DFLASH_ERR_SHAPE unless 1 <= R <= DFLASH_MAX_SEQS, n_kv >= 1, every
 * key count >= 1 and chunk_cap >= 64.
 * ---------------------------------------------------------------------- */
int dflash_attn_plan(const int64_t *keys, int32_t R, int32_t n_kv, int64_t chunk_cap, int32_t cache_dtype,
                     int64_t *out /* [3] */);

/* ------------------------------------------------------------------------
 * Attention split override (a diagnostic for tests of split invariance: the
 * split is exact up to rounding order, so a layer's output must not depend on
 * it).  chunk > 0 makes every later layer call and dflash_attn_plan split
 * each (sequence, K/V head) into items of `chunk` keys (capped as the cache
 * requires); 0 restores the planner.  Process-wide, not synchronised with
 * calls in flight on other threads.  chunk must be 0 or a multiple of 64 in
 * [64, 2^30] (else DFLASH_ERR_SHAPE).  A layer call whose forced split needs
 * more work items than its workspace holds returns DFLASH_ERR_SHAPE with
 * nothing enqueued.
 * ---------------------------------------------------------------------- */
int dflash_attn_force_chunk(int64_t chunk);

/* ------------------------------------------------------------------------
 * In-launch merge watchdog.  When a layer call of one sequence (bf16, d_h 128,
 * 49..64 query rows per K/V head, n_kv a multiple of 8, at most one attention
 * work item per compute unit and 32 per K/V head) merges its attention split inside the
 * attention launch, the items of a K/V head wait for each other there.  Each
 * wait is bounded: a workgroup that gives up writes its rows as NaN and is
 * counted here.  *count receives the number of such workgroups on the
 * current device since the library was loaded (0 in every correct run; a
 * non-zero count means some attention work item could not become resident,
 * e.g. because other work held the compute units).  Synchronous with the
 * device.  Returns DFLASH_ERR_ARG for a null pointer, DFLASH_ERR_HIP if the
 * read fails.
 * ---------------------------------------------------------------------- */
int dflash_attn_sync_timeouts(uint32_t *count);

/* ------------------------------------------------------------------------
 * In-launch merge item order (a diagnostic for tests of the merge's
 * write-back path).  Where a layer call merges its attention split inside
 * the attention launch (see dflash_attn_sync_timeouts), on = 1 deals each
 * K/V head's work items to consecutive workgroups, so that a head's items
 * run on several XCDs and merge through the path that writes every XCD's L2
 * back first (slower; results equal up to rounding order); 0 restores the
 * order that keeps a head on one XCD.  Process-wide, not synchronised with
 * calls in flight on other threads.  Returns DFLASH_ERR_ARG unless on is 0
 * or 1.
 * ---------------------------------------------------------------------- */
int dflash_attn_force_merge_spread(int32_t on);

/* ------------------------------------------------------------------------
 * In-launch merge wait bound (a diagnostic for tests of the time-out path).
 * Each wait of a work item for the other items of its K/V head gives up
 * after `polls` polls of the device memory it waits on (0: at once, without
 * polling); a work item that gives up writes its rows as NaN and is counted
 * by dflash_attn_sync_timeouts.  The default, restored by passing 262144, is
 * about 0.3 s per wait.  Applies to later layer calls; process-wide, not
 * synchronised with calls in flight on other threads.  Returns
 * DFLASH_ERR_ARG unless 0 <= polls <= 262144.
 * ---------------------------------------------------------------------- */
int dflash_attn_set_spin_limit(int32_t polls);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
