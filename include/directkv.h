/*
 * directkv.h — C ABI of the host-resident KV-cache attention layer for MI355X (gfx950).
 *
 * One transformer layer step: the K/V projection of the new tokens, their append to a
 * KV cache that lives in pinned host memory, and causal grouped-query attention that
 * reads that cache in place over the host link (no staging copy in device memory).
 *
 * Sources (the pages this library follows):
 *  [N]  "Paper Notes: DirectKV" — System Architecture (Kernel Generator, Kernel Adaptor,
 *       Attention Fusion Engine, KV Cache Manager), Key Ideas (1) CPU-memory-aware
 *       tiling, (2) projection + attention fusion, (3) warp-level pipelining, and
 *       Fundamental Underlying Technologies / Kernel Fusion (K = X·Wk, V = X·Wv,
 *       softmax(Q·Kᵀ/√d)·V).
 *  [G]  "DirectKV Guide: Zero-Copy KV Offloading on GH200 & GB200" — section 1,
 *       eliminating the GPU staging buffer (host pages mapped into the GPU address space
 *       and dereferenced by kernels); FAQ (the method is lossless).
 *
 * Conventions shared by every call:
 *  - Element types: dkv_dtype. Activations, weights, cache and output share one dtype.
 *  - Weights are stored as bias-free linear-layer weights, [out_features, in_features]
 *    row-major: Wq is [Hq*d, D], Wk and Wv are [Hkv*d, D]; the layer computes X·Wᵀ, so
 *    head h of Q is columns [h*d, (h+1)*d) of X·Wqᵀ.
 *  - X is [B, T, D] row-major; the output is [B, T, Hq*d] row-major.
 *  - Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 *  - Causality: new token t of sequence b sits at absolute position past_len[b] + t and
 *    attends to cache rows 0 .. past_len[b] + t, its own row included.
 *  - Scores are scaled by 1/sqrt(d); no positional encoding, no bias, no output
 *    projection.
 *  - Device pointers (x, w*, out, ws) are caller-owned device memory, 16-byte aligned.
 *    past_len is a host array of B int32 values, read during the call and never
 *    written; the caller advances it by T after a successful call.
 *  - stream: a hipStream_t (0 = the null stream). Calls are asynchronous on it; the
 *    cache rows a call writes are visible to the host after the stream synchronises.
 *    Calls touching one cache must be ordered on one stream.
 *  - Return value: 0 on success, or a negative dkv_status. On error nothing has been
 *    enqueued, no cache row has been touched, and dkv_last_error() describes why.
 */
#ifndef DIRECTKV_H
#define DIRECTKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Environment variables read at each call (tuning and testing only; results are unchanged
 * except where stated):
 *   DIRECTKV_PREFILL_CHUNK=<keys>  keys per prefill super-chunk (rounded down to a multiple of
 *                                  64), instead of the L2-sized default; rounding order of the
 *                                  attention changes, not the result within tolerance;
 *   DIRECTKV_PREFILL_CHUNKED=0     prefills with several super-chunks and query tiles take one
 *                                  launch per super-chunk instead of the two-launch form (a
 *                                  chunk launch of every super-chunk's items, then a finish
 *                                  launch), and attn_workspace_bytes leaves out the two-launch
 *                                  form's running states (at most 2 GiB); rounding order
 *                                  changes, not the result within tolerance;
 *   DIRECTKV_PREFILL_INSERT=<n>    two-launch form: items of a super-chunk dispatched before
 *                                  the next one's fetchers (dispatch order only: bitwise the
 *                                  same output);
 *   DIRECTKV_PREFILL_OWN=<percent> two-launch form: share of the own-key work in the chunk
 *                                  launch; rounding order changes, not the result within
 *                                  tolerance;
 *   DIRECTKV_PREFILL_FETCHERS=<n>  past-key items per pair dispatched first in a launch
 *                                  (dispatch order only: bitwise the same output);
 *   DIRECTKV_DECODE_QPASS=0|1      decode q projected inside the attention kernel (0) or by the
 *                                  pre-pass (1); bitwise the same queries;
 *   DIRECTKV_DECODE_COMBINE=1      keep the combine launch when every sequence has one split;
 *                                  bitwise the same output.
 */

typedef enum { DKV_F32 = 0, DKV_F16 = 1, DKV_BF16 = 2 } dkv_dtype;

typedef enum {
  DKV_OK = 0,
  DKV_ERR_INVALID_ARG = -1, /* null pointer, size <= 0, misalignment, Hq % Hkv != 0, D unsupported */
  DKV_ERR_CAPACITY = -2,    /* past_len[b] < 0 or past_len[b] + T > capacity */
  DKV_ERR_UNSUPPORTED = -3, /* no kernel instance for this dtype / head_dim / group size, or a
                               call with batch * n_kv_heads * T * head_dim >= 2^31 new K elements */
  DKV_ERR_HOST_ALLOC = -4,  /* pinned host allocation failed */
  DKV_ERR_HIP = -5,         /* a HIP runtime call failed */
  DKV_ERR_WORKSPACE = -6    /* ws is null or smaller than attn_workspace_bytes() */
} dkv_status;

/*
 * A KV cache in pinned, mapped host memory ([N] System Architecture, KV Cache Manager;
 * [G] section 1). k and v are host pointers that kernels dereference directly (unified
 * addressing). Layout of each: [batch][n_kv_heads][capacity][head_dim] row-major, so
 * the rows of one (sequence, kv head) are contiguous and one token row is
 * head_dim * element-size bytes. The host may read and write rows between calls.
 */
typedef struct dkv_cache {
  void* k;
  void* v;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  int32_t dtype; /* a dkv_dtype */
  int32_t reserved;
} dkv_cache;

/*
 * Allocate the K and V buffers of a cache with hipHostMalloc (mapped, coherent): pinned
 * host memory the GPU reads and writes in place. Allocates no device memory. Contents
 * are undefined; the caller fills past rows through c->k / c->v. Supported head_dim:
 * 64, 128. capacity must be a positive multiple of 64.
 * Errors: INVALID_ARG (null out, sizes <= 0, capacity % 64), UNSUPPORTED (head_dim,
 * dtype), HOST_ALLOC (the allocation failed; *out is zeroed).
 */
int kv_alloc_host(dkv_cache* out, int32_t batch, int32_t n_kv_heads, int32_t head_dim,
                  int32_t capacity, int32_t dtype);

/* Free both buffers and zero the descriptor. Idempotent; a zeroed descriptor is OK. */
int kv_free_host(dkv_cache* c);

/*
 * Project and append T new tokens per sequence ([N] Kernel Fusion, step 1; KV Cache
 * Manager): rows [past_len[b], past_len[b] + T) of every kv head g receive
 * round(X[b]·Wkᵀ) and round(X[b]·Wvᵀ) restricted to columns [g*d, (g+1)*d), rounded to
 * nearest even in the cache dtype after fp32 accumulation. No other row is written.
 * x: [batch, T, D]; wk, wv: [Hkv*d, D]. batch must equal c->batch. T = 0 is a no-op.
 */
int kv_append(const dkv_cache* c, const void* x, const void* wk, const void* wv,
              const int32_t* past_len, int32_t batch, int32_t T, int32_t D, void* stream);

/*
 * Device workspace the attention calls need, in bytes (phase 0 = prefill with T new
 * tokens, phase 1 = decode with T = 1; phases 2 and 3 = the same for the staging baseline,
 * DKV_PREFILL_STAGED / DKV_DECODE_STAGED, which adds a device copy of the whole cache). It
 * holds the projected queries, this step's new K/V rows, per-split softmax partials and
 * per-row running softmax state. The caller allocates it (e.g. as a device tensor) and
 * passes it with its size. Returns 0 for an invalid argument.
 */
size_t attn_workspace_bytes(int32_t phase, const dkv_cache* c, int32_t batch, int32_t T,
                            int32_t n_q_heads, const int32_t* past_len);

/*
 * One prefill step of T new tokens per sequence ([N] Attention Fusion Engine, prefill
 * strategy): Q = X·Wqᵀ into the workspace, the new K/V rows appended to the host cache as
 * kv_append does, then causal grouped-query attention of the T queries over cache rows
 * 0 .. past_len[b] + t. Each past host KV row crosses the host link once; the new rows
 * are written to the host once and are not read back from it. out: [batch, T, Hq*d] in
 * the cache dtype.
 */
int attn_prefill(const dkv_cache* c, const void* x, const void* wq, const void* wk,
                 const void* wv, const int32_t* past_len, int32_t batch, int32_t T,
                 int32_t D, int32_t n_q_heads, void* out, void* ws, size_t ws_bytes,
                 void* stream);

/*
 * Ablation baselines for the comparisons the pages report ([N] Experiments & Results:
 * CPU-aware tiling vs naive zero-copy, Fig. 12; fused vs separate kernels, Fig. 13; and the
 * swap-based offloading that stages KV in GPU memory, [N] Prior work / GPU memory, Fig. 11b).
 * Same arguments, results and errors as attn_prefill; `variant` selects how the host cache is
 * read:
 *   DKV_PREFILL_FUSED    the attn_prefill path (host KV fetched once per step, new rows kept
 *                        in device memory);
 *   DKV_PREFILL_NAIVE    query-stationary tiling pointed at host memory: every query tile
 *                        streams the whole cache over the link in one launch;
 *   DKV_PREFILL_SEPARATE projection writes new K/V to the host only, and attention reads
 *                        them back over the link;
 *   DKV_PREFILL_STAGED   the past rows are first copied (DMA) into a device staging copy of
 *                        the cache held in the workspace (attn_workspace_bytes phase 2), the
 *                        fused kernels run on that copy, and the new rows are copied back;
 *   DKV_PREFILL_PERSIST  the fused path as one persistent launch per group of 8 (sequence,
 *                        kv head) pairs ([N] Key Idea (3), warp-level pipelining: a producer
 *                        streams the next key super-chunk over the link while the current one
 *                        is computed). Currently DISABLED: every call returns UNSUPPORTED, since
 *                        its launch did not complete on the GPU and the cause is not found. The
 *                        fused path's two-launch form (see DIRECTKV_PREFILL_CHUNKED) overlaps
 *                        the next super-chunk's transfer with the current one's compute instead,
 *                        with no workgroup waiting for another.
 * Errors: as attn_prefill, plus INVALID_ARG for an unknown variant.
 */
enum {
  DKV_PREFILL_FUSED = 0,
  DKV_PREFILL_NAIVE = 1,
  DKV_PREFILL_SEPARATE = 2,
  DKV_PREFILL_STAGED = 3,
  DKV_PREFILL_PERSIST = 4
};
int attn_prefill_variant(const dkv_cache* c, const void* x, const void* wq, const void* wk,
                         const void* wv, const int32_t* past_len, int32_t batch, int32_t T,
                         int32_t D, int32_t n_q_heads, void* out, void* ws, size_t ws_bytes,
                         void* stream, int32_t variant);

/*
 * One decode step (T = 1) for every sequence ([N] Attention Fusion Engine, decode
 * strategy): the new token's k and v are projected inside the attention kernel and stored
 * to host row past_len[b], and the query attends to rows 0 .. past_len[b] (ragged lengths
 * allowed). Split-KV: each split streams its share of the host rows once and writes one
 * partial; a combine merges them. out: [batch, 1, Hq*d]. q is projected once per step by a
 * small pre-pass into the workspace when the splits would otherwise re-read more than
 * 256 MiB of Wq between them, else inside the attention kernel; both give bitwise the same q
 * (the environment variable DIRECTKV_DECODE_QPASS=0 or 1 forces one of them).
 */
int attn_decode(const dkv_cache* c, const void* x, const void* wq, const void* wk,
                const void* wv, const int32_t* past_len, int32_t batch, int32_t D,
                int32_t n_q_heads, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * attn_prefill and attn_decode with a rotary position embedding, for the multi-layer decode loop
 * around the layer (the pages' layer itself has no positional encoding): q and the new k are
 * rotated at their absolute positions p = past_len[b] + t before attention and before k is rounded
 * and appended. Pair (i, i + d/2) of each head, i < d/2, turns by p * rope_theta^(-2i/d):
 * y_i = x_i cos - x_{i+d/2} sin, y_{i+d/2} = x_{i+d/2} cos + x_i sin (the rotate-half form of
 * the Llama-family decoder; Llama 3 uses rope_theta = 500000). Angles are formed in fp64. Cached
 * keys are the rotated ones, so calls on one cache must all use RoPE with the same base. Arguments,
 * workspace (attn_workspace_bytes phase 0 / 1) and errors as attn_prefill / attn_decode, plus
 * INVALID_ARG unless 1 < rope_theta <= 1e30.
 */
int attn_prefill_rope(const dkv_cache* c, const void* x, const void* wq, const void* wk,
                      const void* wv, const int32_t* past_len, int32_t batch, int32_t T,
                      int32_t D, int32_t n_q_heads, void* out, void* ws, size_t ws_bytes,
                      double rope_theta, void* stream);
int attn_decode_rope(const dkv_cache* c, const void* x, const void* wq, const void* wk,
                     const void* wv, const int32_t* past_len, int32_t batch, int32_t D,
                     int32_t n_q_heads, void* out, void* ws, size_t ws_bytes, double rope_theta,
                     void* stream);

/*
 * attn_decode for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same kernels and result as attn_decode
 * (bitwise), with no workspace argument. Its scratch (split partials and projected queries,
 * attn_workspace_bytes(1, ...) bytes) lives in a library-owned device array of 8 MiB, one per GPU,
 * held until the process ends; the call allocates nothing and calls no allocating routine.
 * Calls that need more scratch than 8 MiB return WORKSPACE (nothing enqueued). Every call on one
 * GPU uses that GPU's one array: calls that may overlap on a GPU (different streams, or different
 * host threads without ordering) race on it and must be serialised by the caller. Errors: as
 * attn_decode, plus WORKSPACE for a call beyond the scratch size.
 */
int attn_decode_noalloc(const dkv_cache* c, const void* x, const void* wq, const void* wk,
                        const void* wv, const int32_t* past_len, int32_t batch, int32_t D,
                        int32_t n_q_heads, void* out, void* stream);

/*
 * attn_decode with the staging baseline selectable: DKV_DECODE_ZEROCOPY is attn_decode;
 * DKV_DECODE_STAGED first copies rows [0, past_len[b]) of every head into a device copy of
 * the cache in the workspace (attn_workspace_bytes phase 3), runs the decode kernels on it,
 * and copies the new rows back to the host cache. Same results as attn_decode.
 */
enum { DKV_DECODE_ZEROCOPY = 0, DKV_DECODE_STAGED = 1 };
int attn_decode_variant(const dkv_cache* c, const void* x, const void* wq, const void* wk,
                        const void* wv, const int32_t* past_len, int32_t batch, int32_t D,
                        int32_t n_q_heads, void* out, void* ws, size_t ws_bytes, void* stream,
                        int32_t variant);

/*
 * ---- Paged host cache ([N] KV Cache Manager; the page manager of the pages' reference
 * simulator: 16-token pages of pinned host memory, a table from a sequence's logical pages to
 * physical pages, no device staging buffer).
 *
 * A pool of n_pages pages in pinned, mapped host memory. k and v are each
 * [n_pages][n_kv_heads][DKV_PAGE_TOKENS][head_dim] row-major: one page holds 16 consecutive
 * tokens of every kv head, and the 16 rows of one (page, head) are contiguous. Which pages a
 * sequence uses is the caller's business: a block table, a host array of int32
 * [batch][max_pages] row-major, names for logical page p of sequence b (tokens
 * [16p, 16p + 16)) its physical page block_table[b * max_pages + p]. Several sequences may
 * map the same page for reading (a shared prefix); a page a call writes must be mapped once.
 *
 * The paged calls compute exactly what the contiguous ones do on the gathered cache. They
 * read the block table during the call (it may be changed after they return), check every
 * entry they use on the host (page ids in [0, n_pages); pages written by the call mapped only
 * once among the used entries; past_len[b] + T <= 16 * max_pages, else CAPACITY), and copy it
 * to the front of the workspace, which therefore also covers batch * max_pages int32 values.
 */
#define DKV_PAGE_TOKENS 16

typedef struct dkv_paged_cache {
  void* k;
  void* v;
  int32_t n_pages;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* a dkv_dtype */
  int32_t reserved;
  int32_t pad;
} dkv_paged_cache;

/* Allocate the K and V page pools with hipHostMalloc (mapped, coherent); no device memory.
 * Contents are undefined. Errors: INVALID_ARG, UNSUPPORTED (head_dim, dtype), HOST_ALLOC. */
int kv_paged_alloc_host(dkv_paged_cache* out, int32_t n_pages, int32_t n_kv_heads, int32_t head_dim,
                        int32_t dtype);

/* Free both pools and zero the descriptor. Idempotent. */
int kv_paged_free_host(dkv_paged_cache* c);

/* Device workspace of a paged call, in bytes: phase 0 prefill (T tokens), 1 decode, 2
 * append. Covers the block table copy plus what the contiguous call needs. 0 on bad input. */
size_t attn_paged_workspace_bytes(int32_t phase, const dkv_paged_cache* c, int32_t batch, int32_t T,
                                  int32_t n_q_heads, int32_t max_pages);

/* kv_append on a paged cache: token L_b + t of head g goes to row (L_b + t) % 16 of page
 * block_table[b][(L_b + t) / 16]. No other row is written. */
int kv_paged_append(const dkv_paged_cache* c, const int32_t* block_table, int32_t max_pages, const void* x,
                    const void* wk, const void* wv, const int32_t* past_len, int32_t batch, int32_t T,
                    int32_t D, void* ws, size_t ws_bytes, void* stream);

/* attn_prefill on a paged cache (the fused path). */
int attn_prefill_paged(const dkv_paged_cache* c, const int32_t* block_table, int32_t max_pages,
                       const void* x, const void* wq, const void* wk, const void* wv,
                       const int32_t* past_len, int32_t batch, int32_t T, int32_t D, int32_t n_q_heads,
                       void* out, void* ws, size_t ws_bytes, void* stream);

/* attn_decode on a paged cache. */
int attn_decode_paged(const dkv_paged_cache* c, const int32_t* block_table, int32_t max_pages,
                      const void* x, const void* wq, const void* wk, const void* wv,
                      const int32_t* past_len, int32_t batch, int32_t D, int32_t n_q_heads, void* out,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * ---- Decode-loop helpers: the per-layer work around the attention layer in a multi-layer
 * decode step (a pre-norm decoder block: RMSNorm, the layer, an output projection with a
 * residual add, RMSNorm, a SwiGLU MLP with a residual add). The pages describe the attention
 * layer only; these exist so that a stack of layers can run end to end on synthetic weights.
 * All pointers are caller-owned device memory in the given dtype, rows are row-major.
 */

/* y[r, :] = x[r, :] / sqrt(mean_i x[r, i]^2 + eps) * weight, for r < rows; fp32 arithmetic,
 * rounded once to dtype. x, y: [rows, D]; weight: [D]. y may be x itself. */
int dkv_rmsnorm(const void* x, const void* weight, void* y, int32_t rows, int32_t D, float eps,
                int32_t dtype, void* stream);

/* y = x·wᵀ (+ residual): x [rows, K], w [N, K] (a linear layer's [out, in] weight), residual
 * and y [rows, N]; fp32 accumulation, rounded once. residual may be null, or y itself (an
 * in-place residual add); y may not overlap x. K * element size must be a multiple of 16 and
 * the pointers 16-byte aligned. */
int dkv_linear(const void* x, const void* w, const void* residual, void* y, int32_t rows, int32_t N,
               int32_t K, int32_t dtype, void* stream);

/* y[r, j] = silu(gate_up[r, j]) * gate_up[r, F + j] with silu(z) = z / (1 + e^-z):
 * gate_up [rows, 2F] (gate projection, then up projection), y [rows, F]. */
int dkv_swiglu(const void* gate_up, void* y, int32_t rows, int32_t F, int32_t dtype, void* stream);

/*
 * Streaming read (mode 0) or write (mode 1) of `bytes` bytes of pinned host memory at
 * `host_ptr` by a kernel, the same access path the attention kernels use; measures the
 * host-link rate the layer is bounded by. bytes must be a multiple of 16 * n_wg;
 * host_ptr must come from hipHostMalloc. Mode 1 overwrites the buffer.
 */
int dkv_hostlink_stream(void* host_ptr, size_t bytes, int32_t mode, int32_t n_wg, void* stream);

/*
 * Kernel timing for measurement ([N] Experiments & Results report per-kernel latency): with
 * dkv_timing(1) every later layer call also records HIP events on its own stream around each of
 * its kernel phases; dkv_timing(0) stops (both calls drop what was recorded). dkv_timing_read
 * waits for the recorded events and returns, per phase, the summed elapsed milliseconds and the
 * number of kernel launches they cover, in ms[i] and launches[i] for i < n:
 *   0 projection GEMM (prefill, append), 1 prefill attention (all launches of each call),
 *   2 decode query projection, 3 decode attention, 4 decode combine.
 * Timing adds two events per phase per call; it does not change results. Errors: INVALID_ARG
 * (null output, n <= 0), HIP (an event failed).
 */
int dkv_timing(int32_t enable);
int dkv_timing_read(float* ms, int32_t* launches, int32_t n);

/* Thread-local text describing the last non-zero status returned on this thread. */
const char* dkv_last_error(void);

/* Library version (major*10000 + minor*100 + patch). */
int32_t dkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIRECTKV_H */
