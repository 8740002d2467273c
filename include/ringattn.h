/*
 * ringattn.h -- C ABI of libringattn, the Ring Attention hot path on one
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (short names):
 *   [P1] "Ring Attention如何让大模型突破百万token上下文：从环形通信到计算重叠的技术突围"
 *        (answer.freetools.me blog post)
 *   [P2] "Ring Attention with Blockwise Transformers for Near Infinite Context"
 *        (reading notes on arXiv 2310.01889, papers.chlience.com)
 *   [P3] aiqz.cc Ring Attention explainer
 *
 * The method: the sequence is cut into N blocks, one per host; host i keeps
 * its query block Q_i fixed and attends it to every key/value block K_j, V_j
 * as the blocks travel around a ring (host i receives from i-1 and sends to
 * i+1), folding each block into an online-softmax state (row max m,
 * denominator l, numerator O) ([P1] Ring Attention的核心洞察, Online Softmax;
 * [P2] 5.2; [P3] 分块注意力, 环状拓扑).  On one GPU the N hosts are virtual:
 * their blocks live in one HBM and the neighbour send/receive is an
 * asynchronous device-to-device copy on a second stream, run by the DMA
 * engines (no compute units; an ordinary device copy where the runtime
 * refuses that kind).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers named *_dev / device buffers are device (HBM) addresses; the
 *    caller allocates and frees them.  The library never allocates device
 *    memory and never synchronises the device; it creates and destroys its
 *    own HIP events inside ra_ring_fwd / ra_ring_bwd.
 *  - Streams are hipStream_t values passed as void* (NULL = the null stream).
 *    Every call is asynchronous on its stream(s); results are ready once the
 *    stream reaches the enqueued work.
 *  - Block tensors are row-major [B][H][c][d] with d innermost ("BHCD").
 *    Element type is bf16 (RA_BF16) or fp32 (RA_F32) for Q, K, V, dO and the
 *    finalized output; the online-softmax state is always fp32:
 *    m, l: [B][Hq][c]; O (numerator): [B][Hq][c][d].
 *  - m and LSE are in natural-log units: m = running max of scaled scores,
 *    l = sum of e^(s - m) over the keys folded so far, O = sum of
 *    e^(s - m) v.  LSE = m + ln l.
 *  - Grouped heads: query head g reads key/value head g / (Hq / Hkv).
 *  - Errors: arguments are checked synchronously before any HIP call; a bad
 *    argument returns RA_ERR_INVALID_ARG (or RA_ERR_UNSUPPORTED for a shape
 *    outside the supported set) and leaves every buffer untouched; the detail
 *    is in ra_last_error() (thread-local).  A failed HIP launch/copy returns
 *    RA_ERR_HIP.  Device faults surface at the caller's next synchronisation.
 *    No exception crosses the ABI.  Calls are reentrant.
 *  - Supported shapes: head_dim 64 or 128; block_len >= 1 (any value; the
 *    last tile is masked); heads_q % heads_kv == 0; 16-byte aligned device
 *    pointers; batch, heads and block_len small enough that every element
 *    index fits in int64.
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RA_OK = 0,
    RA_ERR_INVALID_ARG = 1,
    RA_ERR_UNSUPPORTED = 2,
    RA_ERR_HIP = 3,
    RA_ERR_WORKSPACE = 4
} ra_status;

typedef enum { RA_BF16 = 0, RA_F32 = 1 } ra_dtype;

/* Causal: key token t_k is visible to query token t_q iff t_k <= t_q
 * ([P3] 工程实现, the causal block formula with j <= i). */
typedef enum { RA_MASK_NONE = 0, RA_MASK_CAUSAL = 1 } ra_mask_mode;

/* Token layout ([P1] 因果掩码的负载均衡挑战): contiguous = host h holds
 * tokens h*c .. h*c + c - 1; striped = host h holds tokens h, h+N, h+2N, ...
 * zigzag ([P1] 工程实践指南, item 因果掩码, names it beside Striped as the
 * causal load-balancing variant without defining it; the reading used here):
 * the sequence is cut into 2N chunks of c/2 tokens, host h holds chunk h in
 * rows 0..c/2-1 and chunk 2N-1-h in rows c/2..c-1, so every host sees the
 * same number of causal (query, key) pairs.  Zigzag needs an even block_len
 * (the scheduler and token index) and, under the causal mask in the ring
 * drivers, bf16 blocks with block_len % 256 == 0 (RA_ERR_UNSUPPORTED
 * otherwise).  The block calls take one (q_offset, kv_offset, stride) triple
 * and so serve zigzag blocks one quadrant at a time. */
typedef enum { RA_LAYOUT_CONTIGUOUS = 0, RA_LAYOUT_STRIPED = 1, RA_LAYOUT_ZIGZAG = 2 } ra_layout;

/* What a (query block, key block) pair needs under the mask.
 * SKIP: no visible pair ([P3] 工程实现: blocks j > i are skipped);
 * FULL: every pair visible; TRI_INCL: local rows r' <= r visible (the
 * diagonal block); TRI_STRICT: r' < r visible (striped, j > i). */
typedef enum {
    RA_BLK_SKIP = 0,
    RA_BLK_FULL = 1,
    RA_BLK_TRI_INCL = 2,
    RA_BLK_TRI_STRICT = 3,
    RA_BLK_BAND = 4, /* any other diagonal band (general offsets) */
    RA_BLK_QUADRANTS = 5 /* zigzag causal: the four (c/2 x c/2) quadrants of the
                            block pair each have their own class */
} ra_block_class;

typedef struct {
    int32_t batch;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t head_dim;  /* d: 64 or 128 */
    int32_t block_len; /* c: rows per host block */
    int32_t dtype;     /* ra_dtype */
    float scale;       /* score scale; 0 => 1/sqrt(head_dim) ([P2] 5.1) */
} ra_dims;

/* One ring step for one host, as produced by ra_schedule. */
typedef struct {
    int32_t step;      /* s = 0 .. N-1 */
    int32_t src;       /* host whose K/V block is held at this step */
    int32_t cls;       /* ra_block_class */
    int32_t pad_;
    int64_t q_offset;  /* token index of local query row 0 */
    int64_t kv_offset; /* token index of local key row 0 */
    int64_t stride;    /* token distance between consecutive local rows */
} ra_step;

/* Ring driver flags. */
#define RA_FLAG_ELIDE_SKIPPED_COPIES 1u /* single-host runs: do not copy blocks the host skips */
#define RA_FLAG_SERIALIZE 2u            /* run copies on the compute stream (no overlap) */

typedef struct {
    ra_dims dims;
    int32_t n_hosts;    /* N: blocks in the ring, sequence length S = N*c */
    int32_t host_begin; /* simulated hosts [host_begin, host_end) */
    int32_t host_end;
    int32_t layout;     /* ra_layout */
    int32_t mask;       /* ra_mask_mode */
    uint32_t flags;     /* RA_FLAG_* */
    uint32_t debug_copy_delay_us; /* >0: busy-wait this long on the comm stream before each copy */
    /* Optional (NULL = none): 2*n_hosts caller-created hipEvent_t handles.
     * Events 2s and 2s+1 are recorded on the compute stream immediately
     * before and after step s's block kernel launch(es), for timing.  Steps
     * that launch nothing record both events back to back. */
    void *const *step_events;
} ra_ring_cfg;

/* Counters of what a ring call enqueued (filled at enqueue time). */
typedef struct {
    int32_t compute_steps;    /* ring steps that launched block kernels */
    int32_t transfers;        /* K/V block transfers (per host) */
    int32_t skipped_blocks;   /* (host, step) pairs classified SKIP */
    int32_t kernel_launches;
    int64_t copy_bytes;       /* bytes moved by the side-stream copies */
    int64_t resident_bytes_per_host; /* ring buffers one virtual host holds, see ra_ring_workspace_size */
    int32_t copy_kind;        /* ra_copy_kind of the side-stream copies enqueued */
    int32_t pad_;
} ra_ring_stats;

/* How the ring transfers ran: on the DMA engines (no compute units, as a
 * neighbour's send arrives), or as an ordinary device copy because the
 * runtime refused the DMA-engine kind for at least one copy of the call. */
typedef enum { RA_COPY_NONE = 0, RA_COPY_DMA_ENGINES = 1, RA_COPY_FALLBACK = 2 } ra_copy_kind;

/* ---------------------------------------------------------------------
 * Scheduler (host code, no device work)
 * ------------------------------------------------------------------- */

/* Token index of local row r on host h ([P1] 因果掩码的负载均衡挑战).
 * Returns -1 on a bad argument. */
int64_t ra_token_index(int32_t layout, int32_t n_hosts, int64_t block_len, int32_t host,
                       int64_t r);

/* Ring schedule of host `host` ([P1] Ring Attention的核心洞察 steps 3-5;
 * [P3] 环状拓扑): at step s the host holds block src = (host - s) mod N; its
 * class under the mask and the (q_offset, kv_offset, stride) triple that
 * turns local rows into token indices.  A key row r' is visible to query row
 * r iff kv_offset + r'*stride <= q_offset + r*stride (causal) -- for
 * contiguous: FULL for src < host, TRI_INCL for src == host, SKIP for
 * src > host; for striped: TRI_INCL for src <= host, TRI_STRICT otherwise.
 * Zigzag (block_len even): q_offset, kv_offset are the first tokens of the
 * two blocks' first chunks (host*c/2, src*c/2), stride 1, and the class is
 * QUADRANTS under the causal mask (FULL otherwise): the block pair splits
 * into four c/2 x c/2 quadrants between chunk a of the query block and chunk
 * b of the key block, each contiguous with its own offsets.
 * out: host array of n_hosts entries, written in step order. */
ra_status ra_schedule(int32_t n_hosts, int32_t host, int32_t block_len, int32_t layout,
                      int32_t mask, ra_step *out);

/* Class of a (q_offset, kv_offset, stride) pair for blocks of length c
 * (host helper used by the kernels' launch logic; exposed for testing). */
int32_t ra_block_class_of(int32_t mask, int64_t q_offset, int64_t kv_offset, int64_t stride,
                          int32_t block_len);

/* ---------------------------------------------------------------------
 * Block-level device calls
 * ------------------------------------------------------------------- */

/* m = -inf, l = 0, O = 0 for B*Hq*c rows (the initial state of the page
 * demo in [P3] Python 演示).  Pointers: device, fp32. */
ra_status ra_state_init(const ra_dims *dims, float *m, float *l, float *O, void *stream);

/* Fold one key/value block into the online-softmax state of one query block
 * ([P3] 分块注意力 update rule; [P1] Online Softmax):
 *   S = scale * Q_i K_j^T, masked pairs = -inf,
 *   m' = max(m, rowmax S), l' = l e^(m - m') + rowsum e^(S - m'),
 *   O' = O e^(m - m') + e^(S - m') V_j.
 * Rows with no visible key keep their state.  mask_mode RA_MASK_CAUSAL uses
 * (q_offset, kv_offset, stride) as in ra_schedule; RA_MASK_NONE ignores them.
 * Q_i: [B][Hq][c][d], K_j, V_j: [B][Hkv][c][d] in dims->dtype (device).
 * m, l, O: in/out fp32 state (device).  bf16 contractions run on MFMA with
 * fp32 accumulation; P is rounded to bf16 (nearest even) before P V.
 * stride must be >= 1. */
ra_status ra_block_fwd(const ra_dims *dims, const void *Q_i, const void *K_j, const void *V_j,
                       int32_t mask_mode, int64_t q_offset, int64_t kv_offset, int64_t stride,
                       float *m, float *l, float *O, void *stream);

/* Merge two partial results over disjoint key sets ([P1] Online Softmax,
 * LogSumExp form): M = max(lse_a, lse_b), lse = M + ln(e^(lse_a-M) + e^(lse_b-M)),
 * O = e^(lse_a-lse) O_a + e^(lse_b-lse) O_b.  A part with lse = -inf has
 * weight 0; two empty parts give O = 0, lse = -inf.
 * All fp32 device arrays: O_* [B][Hq][c][d], lse_* [B][Hq][c].
 * O_out/lse_out may alias O_a/lse_a or O_b/lse_b exactly (in place). */
ra_status ra_merge_lse(const ra_dims *dims, const float *O_a, const float *lse_a,
                       const float *O_b, const float *lse_b, float *O_out, float *lse_out,
                       void *stream);

/* Finalize ([P2] 5.2: the output is numerator / denominator, and the
 * forward keeps what the backward needs): O_out = O / l in dims->dtype
 * (bf16 rounded to nearest even), lse = m + ln l.  Rows with l = 0 give
 * O_out = 0 and lse = -inf. */
ra_status ra_finalize(const ra_dims *dims, const float *m, const float *l, const float *O,
                      void *O_out, float *lse, void *stream);

/* Backward preprocess: D = rowsum(dO * O) for every query row, with O the
 * finalized output.  O, dO: [B][Hq][c][d] in dims->dtype; D: fp32 [B][Hq][c]. */
ra_status ra_bwd_preprocess(const ra_dims *dims, const void *O, const void *dO, float *D,
                            void *stream);

/* One block of the backward: recompute P = e^(scale Q_i K_j^T - lse_i) on the
 * visible pairs and accumulate (+=) into fp32 buffers
 *   dV_j += P^T dO_i,  dS = P * (dO_i V_j^T - D_i),
 *   dQ_i += scale dS K_j,  dK_j += scale dS^T Q_i
 * (closed-form gradient; [P2] 5.2 only states that the backward sweeps the
 * ring again accumulating dQ, dK, dV from the saved output and statistics).
 * Grouped heads sum dK, dV over the query heads of a group.
 * dQ_i: [B][Hq][c][d] fp32; dK_j, dV_j: [B][Hkv][c][d] fp32 (device).
 * Deterministic: no floating-point atomics. */
ra_status ra_block_bwd(const ra_dims *dims, const void *Q_i, const void *K_j, const void *V_j,
                       const void *dO_i, const float *lse_i, const float *D_i,
                       int32_t mask_mode, int64_t q_offset, int64_t kv_offset, int64_t stride,
                       float *dQ_i, float *dK_j, float *dV_j, void *stream);

/* Token-layout permutation (the data preparation step that assigns tokens to
 * hosts).  to_host_major != 0: full [B][H][S][d] -> host-major
 * [N][B][H][c][d]; 0: the inverse.  heads is the head count of this tensor
 * (Hq or Hkv); elements are dims->dtype.  S = n_hosts * block_len. */
ra_status ra_layout_permute(const ra_dims *dims, int32_t heads, int32_t n_hosts,
                            int32_t layout, int32_t to_host_major, const void *src, void *dst,
                            void *stream);

/* Debug: out[r*cols + r'] = 1 if the kernels' visibility predicate admits
 * key row r' for query row r under (q_offset, kv_offset, stride), else 0.
 * out_dev: device uint8 array of rows*cols. */
ra_status ra_mask_tile(int64_t q_offset, int64_t kv_offset, int64_t stride, int32_t rows,
                       int32_t cols, uint8_t *out_dev, void *stream);

/* ---------------------------------------------------------------------
 * Ring drivers
 * ------------------------------------------------------------------- */

/* Workspace bytes ra_ring_fwd (is_bwd = 0) or ra_ring_bwd (is_bwd = 1)
 * needs for cfg.  Per simulated host the ring holds the receive double
 * buffer for K and V (2 x 2 blocks) plus the fp32 state (m, l, O for the
 * forward; D, dK/dV rotating accumulators for the backward). */
ra_status ra_ring_workspace_size(const ra_ring_cfg *cfg, int32_t is_bwd, size_t *bytes);

/* Ring forward for hosts [host_begin, host_end).
 *   Q:  [host_end-host_begin][B][Hq][c][d]  (the simulated hosts' query blocks)
 *   K, V: [N][B][Hkv][c][d]                 (every host's block: the pool
 *         standing in for the other hosts' memory; block h is host h's own)
 *   O:  [host_end-host_begin][B][Hq][c][d] out, dims->dtype
 *   lse: [host_end-host_begin][B][Hq][c] out, fp32
 *   workspace: device, >= ra_ring_workspace_size(cfg, 0) bytes, 256-byte aligned
 * Step s: every simulated host h folds block (h - s) mod N into its state on
 * `compute` while `comm` copies the block it needs at step s+1 into the other
 * half of its receive double buffer ([P1] 计算与通信重叠; [P3] 隐藏通信).
 * When all N hosts are simulated the copy is the ring send: host h's next
 * block is what host h-1 holds now.  After N steps ra_finalize runs on
 * `compute`.  Work on `comm` is ordered after everything already queued on
 * `compute` when the call is made (inputs produced there are safe to pass),
 * and the call's last use of `comm` is ordered before its last work on
 * `compute`, so synchronising `compute` covers the whole call.
 * stats (host pointer) may be NULL. */
ra_status ra_ring_fwd(const ra_ring_cfg *cfg, const void *Q, const void *K, const void *V,
                      void *O, float *lse, void *workspace, size_t workspace_bytes,
                      void *compute_stream, void *comm_stream, ra_ring_stats *stats);

/* Ring backward ([P2] 5.2: the backward sweeps the ring again and
 * accumulates dQ, dK, dV from what the forward saved).
 * All N hosts (host_begin = 0, host_end = N):
 *   Q, O, dO: [N][B][Hq][c][d] (dims->dtype); lse: [N][B][Hq][c] fp32 from
 *   ra_ring_fwd; K, V: [N][B][Hkv][c][d].
 * bf16 inputs run on the MFMA kernels; fp32 inputs (small problems) on plain
 * fp32 kernels.  Causal zigzag needs bf16 and block_len % 256 == 0.  Every
 * refusal (RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_WORKSPACE) happens
 * before the first HIP call, so a refused call enqueues nothing.
 *   dQ: [N][B][Hq][c][d] fp32 out; dK, dV: [N][B][Hkv][c][d] fp32 out.
 * K/V rotate as in the forward (side-stream copies); the fp32 dK/dV
 * accumulators travel with their block: the step kernel adds its
 * contribution to the partial sum received from host h-1 and stores the sum
 * straight into host h+1's receive slot (a neighbour store), and after step
 * N-1 that store lands at the block's owner, i.e. in dK/dV.
 * A proper subset of hosts (e.g. one host's share, host_end - host_begin = 1):
 *   Q, O, dO: [na][B][Hq][c][d] and lse: [na][B][Hq][c] of the simulated
 *   hosts (na = host_end - host_begin); K, V: the pool [N][B][Hkv][c][d].
 *   dQ: [na][B][Hq][c][d] fp32, complete for the simulated hosts.
 *   dK, dV: [N][B][Hkv][c][d] fp32, the simulated hosts' contributions to
 *   every block (a real ring adds them to the running sums that pass
 *   through; over disjoint host subsets covering the ring they sum to the
 *   full gradient).  The call clears dQ, dK, dV first.  Blocks come from the
 *   pool by side-stream copies into the receive slots, as in ra_ring_fwd;
 *   RA_FLAG_ELIDE_SKIPPED_COPIES omits the copies of blocks a host skips. */
ra_status ra_ring_bwd(const ra_ring_cfg *cfg, const void *Q, const void *K, const void *V,
                      const void *O, const float *lse, const void *dO, float *dQ, float *dK,
                      float *dV, void *workspace, size_t workspace_bytes, void *compute_stream,
                      void *comm_stream, ra_ring_stats *stats);

/* ---------------------------------------------------------------------
 * Decoding against a ring-sharded KV cache
 * ------------------------------------------------------------------- */

/* [P2] 5.6 (the paper's Appendix C) runs autoregressive decoding on the
 * ring: the KV cache of a long context is spread over N hosts, one shard
 * each, and the newest query token of each sequence meets every shard
 * ([P3] 超长序列推理与KV Cache分发 describes the same split).  The new token
 * sees every cached key, so the result is softmax(scale q K^T) V over all
 * valid cached rows; each shard gives a partial (O, LSE) and the partials
 * combine with the LogSumExp merge ([P1] Online Softmax).
 *
 * dims: batch B sequences, heads_q / heads_kv (at most 16 query heads per
 *   KV head), head_dim 64 or 128, block_len c = rows per shard, dtype bf16
 *   (RA_ERR_UNSUPPORTED otherwise), scale (0: 1/sqrt(d)).
 * Workspace bytes for ra_ring_decode with n_hosts shards. */
ra_status ra_decode_workspace_size(const ra_dims *dims, int32_t n_hosts, size_t *bytes);

/* One decode step over n_hosts shards held on this GPU (all device pointers):
 *   q:      [B][Hq][d] bf16, the newest token of each sequence
 *   K, V:   [n_hosts][B][Hkv][c][d] bf16; shard h, sequence b holds
 *           kv_len[h * B + b] valid rows (clamped to [0, c]) at rows
 *           0 .. kv_len-1; rows past them are never read
 *   kv_len: [n_hosts][B] int32, device memory (read by the kernels, so it may
 *           change between calls without a host synchronisation)
 *   O:      [B][Hq][d] out, o_dtype RA_BF16 or RA_F32
 *   lse:    [B][Hq] fp32 out (natural log); a sequence with no valid row
 *           gets O = 0, lse = -inf
 *   workspace: >= ra_decode_workspace_size bytes, 256-byte aligned; holds
 *           the per-chunk partials, which are merged in host order.
 * Query head g uses KV head g / (Hq / Hkv).  With n_hosts = 1 and
 * o_dtype = RA_F32 the call is one host's share; ra_merge_lse (dims with
 * block_len = 1) combines such partials from several hosts.  Arguments are
 * checked before any HIP call; the work is queued on `stream`. */
ra_status ra_ring_decode(const ra_dims *dims, int32_t n_hosts, const void *q, const void *K,
                         const void *V, const int32_t *kv_len, void *O, int32_t o_dtype, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Allocation-free variant of ra_ring_decode, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * checks, kernels and results (bit for bit) as ra_ring_decode, without the
 * workspace: the per-chunk partials live in a fixed 32 MiB device array that
 * the library holds on every GPU it runs on until the process ends (looked up
 * once per device, on the first call with that device current; the call
 * runs on the current device, to which `stream` must belong).  A request
 * whose partials exceed 32 MiB (ra_decode_workspace_size reports the need)
 * returns RA_ERR_WORKSPACE before any HIP call.  Every call on one GPU shares
 * that array: calls that overlap in time on one GPU (concurrent streams, or
 * host threads without ordering) race and must not be issued; calls ordered
 * on one stream are safe.  Every partial a call reads is written by the same
 * call, so nothing needs clearing between calls.  No allocation, free or
 * allocating library routine is called. */
ra_status ra_ring_decode_noalloc(const ra_dims *dims, int32_t n_hosts, const void *q, const void *K,
                                 const void *V, const int32_t *kv_len, void *O, int32_t o_dtype,
                                 float *lse, void *stream);

/* ---------------------------------------------------------------------
 * Blockwise feedforward of the local block
 * ------------------------------------------------------------------- */

/* In the Blockwise Parallel Transformer the feedforward acts on each token
 * of the host's own block, so it runs locally after the ring, block by
 * block, and its activation stays within 2bch ([P2] 2, 5.2-5.3).  The
 * network is the standard two-layer feedforward
 *   Y = GELU(X W1^T) W2^T   (GELU with the exact Gaussian CDF),
 * computed over row blocks of `block_rows` rows; the GELU output of one row
 * block ([block_rows][f] bf16) is the only intermediate and lives in the
 * caller's workspace, beside fp32 split-K partial sums when a row block is
 * too small to give every CU a tile (ra_ffn_workspace_size covers both).  All device pointers, bf16, row-major:
 *   X [rows][h], W1 [f][h], W2 [h][f] (two linear layers' weights,
 *   out-features major), Y [rows][h] out.  h and f are multiples of 64.
 * Products accumulate in fp32; the GELU output is rounded to bf16 before
 * the second layer.  Arguments are checked before any HIP call. */
ra_status ra_ffn_workspace_size(int64_t block_rows, int32_t h, int32_t f, size_t *bytes);
ra_status ra_block_ffn(const void *X, const void *W1, const void *W2, void *Y, int64_t rows, int32_t h,
                       int32_t f, int64_t block_rows, void *workspace, size_t workspace_bytes,
                       void *stream);

/* ---------------------------------------------------------------------
 * Errors and version
 * ------------------------------------------------------------------- */
const char *ra_status_str(ra_status s);
const char *ra_last_error(void); /* thread-local detail of the last failure */
int32_t ra_version(void);        /* 100 * major + minor */

#ifdef __cplusplus
}
#endif
#endif /* RINGATTN_H */
