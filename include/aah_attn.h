/*
 * aah_attn.h -- C ABI of the per-head causal local-window attention library
 * (the execution branch of Asymmetric Attention Heads, AAH-v3) for AMD MI355X
 * (gfx950).
 *
 * Operation.  "Asymmetric Attention Heads: Structured Head-Wise Context
 * Allocation for Transformer Attention", section 5.8 (Head mapping and
 * execution): every head h has its own causal local window W_h; key t_k is
 * visible to query t_q iff t_q - W_h + 1 <= t_k <= t_q, and
 *     A = softmax(Q K^T * scale + M_W),   Y = A V
 * with the softmax scale 1/sqrt(d_h) of section 4.  W_h >= T is standard
 * causal attention (sections 5.2 and 5.8).  The pages bucket heads by window,
 * run each bucket and scatter the results back to head order (Figure 1); here
 * one launch runs every head and each work item writes its own (b, h) slice,
 * so head order is preserved without gather or scatter copies.  A bucket is
 * never silently run by another backend (section 7.7): unsupported inputs
 * return AAH_ERR_UNSUPPORTED.
 *
 * Conventions shared by every entry point:
 *   - Q, O, dO, dQ are dense row-major [B, H, T, d] tensors and K, V, dK, dV
 *     [B, H_kv, T, d] (d fastest), all of one dtype `dt`, device pointers
 *     aligned to 16 bytes.  LSE and the backward's D are fp32 [B, H, T].
 *   - H_kv (1 <= H_kv <= H, H_kv divides H) is the number of key/value heads:
 *     query head h reads key/value head h / G, G = H / H_kv, so the G query
 *     heads of a group are consecutive (grouped-query attention; H_kv = H is
 *     plain multi-head attention).  Windows and sinks stay per query head, and
 *     the gradients of a shared key/value head sum over its G query heads.
 *     "Asymmetric Attention Heads" section 3.3 sets the method beside grouped
 *     K/V sharing and appendix A.3 inserts it into a grouped-query model;
 *     "Autonomy-of-Heads" section 4 assigns query heads to KV groups.
 *   - `windows` is a HOST pointer to int32[H], one window per head, shared by
 *     every batch entry (section 5.8 maps one decision per head).  Each entry
 *     must be >= 1; entries above T act as T.  No lower clamp is applied: the
 *     pages' W_min = 512 belongs to the window controller, not to execution.
 *   - `sinks` is NULL or a HOST pointer to int32[H], each >= 0: head h also
 *     keeps its first sinks[h] keys visible to every later query, i.e. key t_k
 *     is visible to query t_q iff t_k <= t_q and (t_q - W_h < t_k or
 *     t_k < sinks[h]).  This is the sink + recent-window attention of a
 *     streaming head in "Autonomy-of-Heads: Data-Free Sparse Attention from
 *     Frozen Query-Key Geometry", section 5 (Deploying LLMs With AoH; section
 *     6.1 uses 128 sinks and a window of 256).  NULL, or all zeros, is the
 *     plain window.  Sinks past T - min(W_h, T) change nothing and are
 *     ignored; lse then covers the sink keys too.
 *   - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *     stream).  Calls only enqueue work on it and return; they never
 *     synchronise the device.  The first call for a new (B, H, T, dtype, d,
 *     windows, sinks) combination builds its work list on the host and
 *     uploads it on `stream` (a stream-ordered allocation filled by
 *     hipMemcpyAsync from pinned staging memory); later calls with the same
 *     combination reuse it, and a call on another stream first waits for that
 *     upload.  Work lists larger than 4 MiB are uploaded synchronously.
 *   - The library keeps at most 64 work lists per kind (forward / backward,
 *     split, decoding).  A new one beyond that replaces the least recently
 *     used, which is released in the order of the stream of the call that
 *     replaces it: a caller that runs calls on several streams concurrently
 *     with more distinct window vectors in flight than that must order those
 *     streams.  During HIP graph capture no work list is built (AAH_ERR_
 *     UNSUPPORTED for a combination not yet cached: run it once outside the
 *     capture); one used there is kept until aah_cache_clear(), since the
 *     graph refers to it.
 *   - The caller allocates and owns every tensor, the workspace and the
 *     stream.  The library owns only its cached work lists, released by
 *     aah_cache_clear(), and the staging memory they are uploaded through.
 *   - Every argument check runs before any HIP call; on an error nothing is
 *     written to any output and the call returns a status other than AAH_OK.
 *     aah_last_error_detail() then describes the failure (thread-local).
 *   - Supported: dt = AAH_BF16 with d in {32, 64, 128}; dt = AAH_F32 with d in
 *     {32, 64, 128}; any T >= 1 (ragged tails are masked) with T * d * 4 < 2^31
 *     (one head's slice is addressed with 32-bit offsets).
 *   - Empty problems: B = 0 or T = 0 (decoding: B = 0; the cache fill: B = 0 or
 *     T = 0) leave nothing to compute.  The call checks its other arguments
 *     (H >= 1, windows, sinks, H_kv, d, dt, scale) and returns AAH_OK without
 *     touching any tensor or workspace, which may then be NULL (an empty
 *     tensor has no storage).  aah_head_features has no empty case.
 */
#ifndef AAH_ATTN_H
#define AAH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AAH_ABI_VERSION 13

typedef enum {
  AAH_OK = 0,
  AAH_ERR_INVALID_ARG = 1,  /* null pointer, negative size (or H < 1), window < 1, misalignment (of any tensor or
                               workspace), non-finite scale */
  AAH_ERR_UNSUPPORTED = 2,  /* dtype / head dim combination without a kernel */
  AAH_ERR_WORKSPACE = 3,    /* workspace smaller than aah_attn_workspace_size() */
  AAH_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} aah_status;

typedef enum { AAH_BF16 = 0, AAH_F32 = 1 } aah_dtype;

typedef void* aah_stream_t;

/* One unit of work: a (batch*H + head) index, a row tile of the stationary
 * operand and the half-open range [lo, hi) of tiles of the streamed operand
 * it must visit.  Forward items: tile = query tile, [lo, hi) = key/value
 * tiles.  Backward items: tile = key/value tile, [lo, hi) = query tiles.
 * bh = -1 marks a padding slot that does nothing. */
typedef struct {
  int32_t bh;
  int32_t tile;
  int32_t lo;
  int32_t hi;
} aah_work_item;

/* ABI version of the loaded library (AAH_ABI_VERSION). */
int aah_abi_version(void);

/* Static name of a status code; never NULL. */
const char* aah_status_string(aah_status status);

/* Thread-local description of the last failed call on this thread ("" if none). */
const char* aah_last_error_detail(void);

/*
 * Forward pass (section 5.8).  Reads q, k, v [B,H,T,d] of dtype dt; writes
 * o [B,H,T,d] (dtype dt) and lse [B,H,T] (fp32): lse[b,h,i] is the natural log
 * of sum_j exp(scale * q_i . k_j) over the window of row i.  Accumulation and
 * softmax run in fp32 whatever dt is; bf16 outputs are rounded to nearest even.
 * Workspace is optional.  With workspace = NULL (or fewer bytes than
 * aah_attn_fwd_workspace_size reports) every work item writes its own rows.
 * A non-NULL workspace must be 256-byte aligned (AAH_ERR_INVALID_ARG otherwise,
 * whether or not the launch would split).
 * With a device workspace of at least that many bytes, a bf16
 * launch whose longest items hold more key tiles than L = max(24, total key
 * tiles / workgroups the device holds at once) splits those items' key ranges
 * into chunks of at most L tiles whose partial results (row max, row sum, fp32
 * accumulator) land in the workspace, and a second kernel on the same stream
 * merges them into o and lse.  That fills the device when B * H * ceil(T / 128)
 * is small (one sequence, few heads).  With sink keys the first chunk of an
 * item also visits its sink tiles.  The results agree within the bf16
 * bounds, not bitwise, since each chunk rounds its weights against its own
 * reference.  The workspace carries nothing between calls; calls that share one
 * must not run concurrently.
 */
aah_status aah_attn_fwd(const void* q, const void* k, const void* v,
                        const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T, int d,
                        aah_dtype dt, float scale, void* o, float* lse,
                        void* workspace, size_t workspace_bytes,
                        aah_stream_t stream);

/*
 * Workspace bytes with which aah_attn_fwd splits long items (see above) for
 * these windows and shape on the current device: 0 when it would not split
 * (fp32, enough work items already, or invalid arguments).  Queries
 * the device's occupancy and builds the split work list on first use per shape
 * (cached like the other work lists).
 */
size_t aah_attn_fwd_workspace_size(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                                   int d, aah_dtype dt);

/*
 * Workspace bytes with which the backward (aah_attn_bwd, and each of its two
 * steps) splits long items as the forward does, for these windows and shape
 * on the current device; 0 when it would not (fp32, enough work items,
 * invalid arguments).  Sink keys and grouped key/value heads split too (the
 * dK/dV chunks of a grouped item cut its query-tile range, each running every
 * query head of the group over its part).  Such a workspace
 * holds the usual rows first (so it also serves an unsplit call), then each
 * split kernel's partial sums; a merge launch after each split kernel adds
 * them in a fixed order (results stay deterministic, and agree with the
 * unsplit launch within the bf16 bounds).
 */
size_t aah_attn_bwd_split_workspace_size(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                                         int T, int d, aah_dtype dt);

/*
 * Forward pass with the attention diagnostics of "Asymmetric Attention Heads"
 * section 5.3 (the controller's head features include the attention entropy
 * and the output norm, taken from the most recent attention statistics).
 * Does exactly what aah_attn_fwd does (same o and lse) and also writes, for
 * every query row, row_entropy[b,h,i] = -sum_j p_ij ln p_ij over the row's
 * visible keys and row_onorm[b,h,i] = ||o_i||_2 (of the fp32 output before its
 * rounding to dt), both fp32 [B,H,T] device arrays, 4-byte aligned.  In bf16
 * the entropy is formed from the same rounded weights as lse: it is within
 * 2^-7 H + 2^-8 of the exact H.  Workspace: optional, as for aah_attn_fwd,
 * with aah_attn_fwd_diag_workspace_size bytes for a split launch; its chunks
 * also leave each row's sum of weights times their log-domain offsets, from
 * which the merge forms the entropy, and the merge takes the output norm of
 * the combined fp32 row.
 */
aah_status aah_attn_fwd_diag(const void* q, const void* k, const void* v, const int32_t* windows,
                             const int32_t* sinks, int B, int H, int H_kv, int T, int d, aah_dtype dt, float scale,
                             void* o, float* lse, float* row_entropy, float* row_onorm, void* workspace,
                             size_t workspace_bytes, aah_stream_t stream);

/*
 * Workspace bytes with which aah_attn_fwd_diag splits long items, as
 * aah_attn_fwd_workspace_size for aah_attn_fwd (a little more: four floats
 * of per-row partials instead of two); 0 when it would not split.
 */
size_t aah_attn_fwd_diag_workspace_size(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                                        int T, int d, aah_dtype dt);

/*
 * Per-head controller features ("Asymmetric Attention Heads" section 5.3):
 *   x_h = [mu(|q_h|), sigma(q_h), mu(|k_h|), sigma(k_h), mu(|v_h|), sigma(v_h), e_h, n_h, rho_h]
 * mu(|.|) is the mean of the absolute activations and sigma the population
 * standard deviation, both over batch, sequence and head dimension of head h;
 * e_h and n_h are the means over batch and rows of row_entropy and row_onorm
 * (from aah_attn_fwd_diag), and rho_h = min(W_h, T) / T is the window usage of
 * that forward pass, whose windows the caller passes here.  These three are
 * the previous-attention diagnostics: pass both row arrays NULL when there
 * are none yet, and all three are 0 (section 5.3 starts missing diagnostics
 * at zero).  With grouped
 * key/value heads the k and v entries of query head h are those of its
 * group's head.  Writes x to
 * features (device float[H * 9], row h = x_h; may be NULL) and smooths
 * features_ema (device float[H * 9], in/out; may be NULL):
 *   features_ema = init ? x : alpha * features_ema + (1 - alpha) * x,
 * with 0 <= alpha <= 1 (the pages use 0.9, initialised from the first x).  At
 * least one of features, features_ema must be given.  q, k, v as for the
 * forward, with B, T >= 1 (the statistics are means over tokens).  Workspace:
 * aah_head_features_workspace_size(B, H, T, d) bytes, 256-byte aligned,
 * scratch.  Deterministic: the same inputs give the same bits.
 */
size_t aah_head_features_workspace_size(int B, int H, int T, int d);

aah_status aah_head_features(const void* q, const void* k, const void* v, const float* row_entropy,
                             const float* row_onorm, const int32_t* windows, int B, int H, int H_kv, int T, int d,
                             aah_dtype dt, float alpha, int init, float* features, float* features_ema,
                             void* workspace, size_t workspace_bytes, aah_stream_t stream);

/*
 * Backward pass: gradients of sum(O * dout) with respect to q, k and v (dk, dv
 * [B, H_kv, T, d]: a shared head's gradient sums over its query heads), given
 * the forward's o and lse (the log-sum-exp saved by aah_attn_fwd with the same
 * scale, windows and sinks).  Writes dq, dk, dv [B,H,T,d] of dtype dt (each element
 * exactly once: no atomics, results are bitwise reproducible).  Needs a device
 * workspace of at least aah_attn_workspace_size(B, H, T, d, dt, 1) bytes,
 * 256-byte aligned; its contents on entry do not matter and are clobbered.
 * Runs aah_attn_bwd_dq and then aah_attn_bwd_dkdv on `stream`.
 */
aah_status aah_attn_bwd(const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse,
                        const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T, int d,
                        aah_dtype dt, float scale, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        aah_stream_t stream);

/*
 * The backward's two steps as separate calls, for callers that schedule or
 * time them.  Arguments mean what they mean for aah_attn_bwd and the same
 * checks apply.  The workspace carries two fp32 [B,H,T] arrays from the first
 * step to the second: nl2 = -lse log2(e) at byte 0, then nD = -D, with
 * D_i = dout_i . o_i, at the next 256-byte boundary after B*H*T floats.
 *   aah_attn_bwd_dq:   writes dq (query-stationary kernel) and, for every
 *     row, nl2 and nD into the workspace.
 *   aah_attn_bwd_dkdv: writes dk and dv (key-stationary kernel) from q, k,
 *     v, dout and the workspace rows; it must not start before
 *     aah_attn_bwd_dq has completed on the same workspace.  It only reads
 *     those rows, but a launch that splits (a workspace of
 *     aah_attn_bwd_split_workspace_size bytes) also writes its dK/dV partial
 *     sums past them, so two dK/dV calls that share a workspace must not run
 *     concurrently either.
 */
aah_status aah_attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                           int T, int d, aah_dtype dt, float scale, void* dq, void* workspace,
                           size_t workspace_bytes, aah_stream_t stream);

aah_status aah_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                             const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T, int d,
                             aah_dtype dt, float scale, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, aah_stream_t stream);

/*
 * Decoding over per-head trimmed K/V caches (bf16).
 *
 * One decoding step is section 5.8 for the newest position only: the token at
 * position p of query head h (window W_h) attends to positions
 * max(0, p - C_h + 1) .. p, where C_h = min(W_h, T_max) and T_max is the
 * maximum context the caches are built for, and, with sinks (a streaming head
 * of "Autonomy-of-Heads" section 5: sink tokens plus a recent window), also to
 * positions 0 .. min(sinks[h], p + 1) - 1.  Table 6 runs inference with
 * per-head windows, and AoH section 5 bounds a streaming head's decode-time
 * cache by its sinks and window.  With grouped key/value heads (H_kv < H,
 * G = H / H_kv) query head h reads key/value head h / G, and the caches hold
 * H_kv heads.
 *
 * Cache layout: kcache and vcache are device tensors [B, R, d] of dtype dt with
 * R = aah_kv_cache_rows(windows, sinks, H, H_kv, T_max).  Key/value head g
 * owns S_g sink rows followed by R_g ring rows, from row off_g (the sum of
 * S + R over the heads before g), where
 *   R_g = max over its query heads of C_h,
 *   S_g = max over its query heads of min(sinks[h], T_max - C_h)
 * (a sink at or past T_max - C_h is always inside the window).  Position t
 * lives in ring row off_g + S_g + (t mod R_g) and, if t < S_g, also in sink row
 * off_g + t.  Rows not yet written are never read.  Only dt = AAH_BF16 is
 * supported (AAH_ERR_UNSUPPORTED otherwise, and when one step's query rows,
 * H * d * 2 bytes, reach 2^31); d in {32, 64, 128}; sinks may be
 * NULL; windows, sinks, H_kv and stream as for the other calls.  Without sinks
 * and grouping head h simply owns C_h ring rows.
 */

/* R rows per batch entry (see above); -1 for invalid arguments. */
int64_t aah_kv_cache_rows(const int32_t* windows, const int32_t* sinks, int H, int H_kv, int T_max);

/* Workspace bytes aah_attn_decode needs: B*H_kv int32 merge counters (rounded
 * up to 256 bytes), then B * chunks * G * (2 + d) floats of partial results,
 * chunks = sum over key/value heads of ceil((S_g + R_g) / 256) (of
 * ceil((S_g + R_g) / 512) with grouped heads, H_kv < H); 0 for invalid
 * arguments. */
size_t aah_attn_decode_workspace_size(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                                      int T_max, int d, aah_dtype dt);

/*
 * Prefill into the caches: k, v [B,H_kv,T,d] hold positions 0 .. T - 1
 * (0 <= T <= T_max; T_max >= 1); writes the positions each key/value head keeps (its first
 * min(S_g, T) into the sink rows, its last min(R_g, T) into the ring) into
 * their rows.  Other rows are left as they are.
 */
aah_status aah_kv_cache_fill(const void* k, const void* v, const int32_t* windows, const int32_t* sinks, int B, int H,
                             int H_kv, int T, int T_max, int d, aah_dtype dt, void* kcache, void* vcache,
                             aah_stream_t stream);

/*
 * One decoding step.  q [B,H,d] and k_new, v_new [B,H_kv,d]: the new token of
 * every sequence; pos: DEVICE pointer to int32[B], the new token's position in
 * each sequence, 0 <= pos[b] < T_max (values outside are clamped into that
 * range), with every earlier position the step attends to already in the
 * cache.  Writes k_new / v_new into the rows of position pos[b] and
 * o [B,H,d] (dtype dt), lse [B,H] (fp32, natural log of sum_j exp(scale q . k_j)
 * over the attended positions).  Workspace: at least
 * aah_attn_decode_workspace_size bytes, 256-byte aligned.  Its first B*H_kv
 * int32 (the merge counters) must be zero before the first call that uses it;
 * every call leaves them zero again, the rest of it carries nothing between
 * calls.  Calls that share a workspace must not run concurrently.
 */
aah_status aah_attn_decode(const void* q, const void* k_new, const void* v_new, void* kcache, void* vcache,
                           const int32_t* pos, const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                           int T_max, int d, aah_dtype dt, float scale, void* o, float* lse, void* workspace,
                           size_t workspace_bytes, aah_stream_t stream);

/*
 * One decoding step that allocates nothing, for callers that cannot allocate
 * device memory when they call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments, caches, results and
 * status codes are those of aah_attn_decode, without the workspace.  Its merge
 * counters, plan tables and partial results live in one fixed device array
 * per GPU that the library holds until the process ends (8 MiB, allocated
 * when the library's code is loaded on that device, not by this call); a
 * small planning kernel rebuilds the tables from the windows and clears the
 * counters on every call, so the call reads no host memory after it returns
 * and a captured graph replays the whole step.  No work list is cached.
 * Limits: H <= 256, and the step's counters, tables and partials
 * (B * H_kv * 4 bytes, (4 H_kv + 1 + 2 H) * 4 bytes, 32 bytes per chunk
 * of a batch entry, and B * chunks * (H / H_kv) * (2 + d) * 4 bytes, each
 * region rounded up to 256 bytes) must fit in the array; a larger step returns
 * AAH_ERR_UNSUPPORTED before any HIP call.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads) race.
 */
aah_status aah_attn_decode_noalloc(const void* q, const void* k_new, const void* v_new, void* kcache, void* vcache,
                                   const int32_t* pos, const int32_t* windows, const int32_t* sinks, int B, int H,
                                   int H_kv, int T_max, int d, aah_dtype dt, float scale, void* o, float* lse,
                                   aah_stream_t stream);

/* Workspace bytes needed by aah_attn_fwd (is_bwd = 0) or aah_attn_bwd (is_bwd != 0);
 * 0 for invalid arguments. */
size_t aah_attn_workspace_size(int B, int H, int T, int d, aah_dtype dt, int is_bwd);

/* Tile shape used by the kernels for (dt, d, is_bwd): rows of the stationary
 * operand per item and rows of the streamed operand per inner step. */
aah_status aah_tile_shape(aah_dtype dt, int d, int is_bwd, int* row_tile, int* col_tile);

/*
 * Host-only work-list builders (no HIP call; usable without a GPU).
 *
 * Forward: for each (b, h, query tile qt) with rows [qt*q_tile, min(T, (qt+1)*q_tile)),
 * the keys needed are [max(0, q0 - W + 1), q1 - 1], i.e. key tiles
 * [floor(max(0, q0 - W + 1) / kv_tile), floor((q1 - 1) / kv_tile) + 1).
 * Backward: for each (b, key/value head g, key tile kt) with keys [k0, k1),
 * bh = b * H_kv + g; in query head h the queries that see them are
 * [k0, min(T, k1 + W - 1)), i.e. query tiles
 * [floor(k0 / q_tile), floor((min(T, k1 + W - 1) - 1) / q_tile) + 1); the item's
 * [lo, hi) is the union over the group's query heads, its cost their sum.
 * W = min(windows[h], T).  Tiles wholly outside every row's window are never
 * listed.  With sinks (NULL = none), S = min(sinks[h], T - W): a forward
 * item also visits the sink key tiles [0, min(ceil(S / kv_tile), lo)) before
 * [lo, hi) (implied, not stored); a backward item whose keys start below S
 * runs to the last query tile, [floor(k0 / q_tile), ceil(T / q_tile)).
 * Items are grouped into `n_queues` queues (key/value groups -- the G query
 * heads of one key/value head, or one head when H_kv = H -- are dealt to
 * queues longest-total-first, each to the least-loaded queue); each queue is
 * sorted by item cost (tiles visited, sink tiles included) descending, ties
 * by (group, tile, bh) ascending; the
 * output interleaves the queues so that slot s belongs to queue s % n_queues,
 * padding short queues with bh = -1 slots.  With n_queues = 8 this matches
 * the round-robin placement of workgroups on MI355X's eight XCDs, so the
 * items of one head share an L2.
 *
 * Writes up to `capacity` items to `items` (may be NULL when capacity = 0)
 * and always stores the full slot count in *n_items; returns
 * AAH_ERR_INVALID_ARG if capacity is too small (after setting *n_items).
 */
aah_status aah_plan_fwd(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                        int q_tile, int kv_tile, int n_queues,
                        aah_work_item* items, int64_t capacity, int64_t* n_items);

/*
 * Split forward work list (host only, no GPU): as aah_plan_fwd, but every
 * item of more than chunk_tiles window tiles becomes items over consecutive
 * near-equal sub-ranges of those tiles (the split launch of aah_attn_fwd); an
 * item's sink tiles belong to its first chunk, the one whose range starts at
 * the window's first tile.  slots[i] is item i's partial-result slot, -1 for
 * an item that writes its own rows; merges holds one record per split item:
 * (bh, q_tile_index, first slot, number of chunks).  Writes up to `capacity`
 * items and slots and up to `merge_capacity` records, stores the full counts
 * in *n_items and *n_merges, and returns AAH_ERR_INVALID_ARG if either
 * capacity is too small (after setting both counts).
 */
aah_status aah_plan_fwd_split(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                              int q_tile, int kv_tile, int n_queues, int chunk_tiles, aah_work_item* items,
                              int32_t* slots, int64_t capacity, int64_t* n_items, aah_work_item* merges,
                              int64_t merge_capacity, int64_t* n_merges);

/*
 * Split backward (dK/dV) work list, host only: as aah_plan_bwd, with every
 * key item whose steps (query tiles summed over the group's query heads, each
 * over its own range from lo) exceed chunk_tiles cut into items over
 * consecutive sub-ranges [c_lo, c_hi) of its range [lo, hi) with near-equal
 * steps, each running every head of the group over its part of the range;
 * slots and merge records (bh, key tile index, first slot, chunks) as for
 * aah_plan_fwd_split.
 */
aah_status aah_plan_bwd_split(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                              int q_tile, int kv_tile, int n_queues, int chunk_tiles, aah_work_item* items,
                              int32_t* slots, int64_t capacity, int64_t* n_items, aah_work_item* merges,
                              int64_t merge_capacity, int64_t* n_merges);

aah_status aah_plan_bwd(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                        int q_tile, int kv_tile, int n_queues,
                        aah_work_item* items, int64_t capacity, int64_t* n_items);

/*
 * Coverage of a window vector (section 5.10): the exact visible query/key
 * pair count of one batch entry, sum_h sum_{t=1}^{T} min(t, W_h) (plus, with
 * sinks, the sink keys each row sees before its window,
 * sum_t max(0, min(S_h, t - W_h))), and the Attention Coverage Ratio
 * sum_h T * W_h / (H * T^2) of the windows alone, with W_h = min(W_h, T).
 * sinks may be NULL.
 */
aah_status aah_window_stats(const int32_t* windows, const int32_t* sinks, int H, int T,
                            int64_t* pairs_per_batch, double* acr);

/* Free every cached device work list (synchronising the device).  Not
 * thread-safe against concurrent aah_attn_* calls that may be using them. */
void aah_cache_clear(void);

/* Number of work lists currently cached (all kinds together); each kind holds
 * at most 64 besides those pinned by graph capture. */
int64_t aah_cache_entries(void);

#ifdef __cplusplus
}
#endif

#endif /* AAH_ATTN_H */
