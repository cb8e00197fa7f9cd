/*
 * longflow.h -- C ABI of the LongFlow fused decode + score + evict library
 * (liblongflow.so, HIP for AMD Instinct MI355X / gfx950).
 *
 * What the library computes is defined on the LongFlow pages:
 *   - attention weights and output: LongFlow Guide (aifetchly blog),
 *     §Mathematical Derivation of the LongFlow Score, the alpha and o_t
 *     equations;
 *   - the token score ||c_{t,i}||_1 = alpha_{t,i} ||v_i||_1: same section, the
 *     c_{t,i} and Score equations; gist.science summary of arXiv 2603.11504,
 *     §2.1 (LongFlowScore);
 *   - the static buffer, initial fill, argmin eviction and in-place overwrite:
 *     LongFlow Guide, §Static Memory Pre-Allocation and In-Place Eviction,
 *     items 1-3; gist.science summary, §2.3 (static KV cache, one fused pass);
 *   - the variants selected in lf_config (l2 norm, the engine's deferred
 *     order, one victim per sequence): LongFlow Guide, §Mathematical
 *     Derivation (l1 or l2 norm of c_{t,i}) and §End-to-End Implementation:
 *     Building a LongFlow Engine (victim applied at the next call, scores
 *     summed over all heads).
 *
 * Unit of work: a "pair" is one (layer, sequence b, KV head h). Query head j
 * belongs to KV head j / G, G = num_q_heads / num_kv_heads. Pairs never
 * interact.
 *
 * One decode step of one pair, with n tokens cached (n <= budget):
 *   s_{g,i} = tau * <q_g, k_i> over the n cached tokens and the new token,
 *   alpha   = softmax over those n+1 tokens (per query head g),
 *   out_g   = sum_i alpha_{g,i} v_i (new token included),
 *   if n < budget (or mode FULL): the new token is appended at slot n;
 *   else: score_i = ||v_i||_1 * sum_g alpha_{g,i} for i in [sink_size, budget),
 *         the slot with the smallest score (lowest index on ties) is
 *         overwritten in place by k_new, v_new, ||v_new||_1.
 * ||v||_1 is kept per slot in a float32 sidecar, computed once when the token
 * is stored, from the stored (dtype-rounded) values.
 *
 * Variants (lf_config.order / scope / norm; 0 selects the behaviour above):
 *   LF_NORM_L2          the sidecar and the score use ||v||_2 instead.
 *   LF_ORDER_DEFERRED   the engine's order. Below the budget the token is
 *                       appended. At the budget it first replaces the slot
 *                       chosen by the PREVIOUS step (budget-1 if none was
 *                       chosen yet, e.g. right after a full prefill); the
 *                       replaced token leaves the softmax. When the buffer is
 *                       full after the write, the step scores the cached
 *                       slots (sinks and the slot just written excluded) and
 *                       keeps the argmin as the next victim.
 *   LF_SCOPE_SEQUENCE   one victim per (layer, sequence): the argmin of the
 *                       score summed over the sequence's KV heads, in head
 *                       order; every KV head of the sequence evicts that slot.
 *
 * Conventions for every call:
 *   - The handle owns all cache memory (K, V, ||v||_1, fill counters): one
 *     device allocation made by lf_cache_create, freed by lf_cache_destroy,
 *     never resized. No call allocates device memory after create.
 *   - The caller owns every I/O pointer. They are contiguous DEVICE buffers in
 *     cfg.dtype (float32 or bfloat16) unless stated, and must stay valid until
 *     the work queued on `stream` has completed.
 *   - The cache lives on the device that was current at lf_cache_create.
 *     Every later call on the handle runs there and leaves the caller's
 *     current device as it found it.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are stream-ordered and asynchronous; the library never
 *     synchronises the device and never copies device -> host.
 *   - Arguments are validated on the host before anything is queued. A call
 *     that returns any error other than LF_ERR_HIP has changed nothing.
 *     LF_ERR_HIP means the HIP runtime refused a launch or copy; calls that
 *     queue several (lf_prefill_fill, lf_seq_reset, lf_cache_snapshot) may
 *     have queued some before it, so the layer's contents are then
 *     undefined until it is filled again.
 *   - Inputs must be finite; NaN or Inf make the results undefined.
 *   - A handle is not thread-safe; serialise its calls on one stream.
 */
#ifndef LONGFLOW_H
#define LONGFLOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lf_cache lf_cache; /* opaque */

typedef enum {
  LF_OK = 0,
  LF_ERR_INVALID_ARG = 1, /* null pointer, out-of-range index, bad config   */
  LF_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, group, sizes    */
  LF_ERR_CAPACITY = 3,    /* prefill longer than the budget; FULL cache full */
  LF_ERR_OOM = 4,         /* the one device allocation failed               */
  LF_ERR_HIP = 5,         /* a HIP runtime or launch error                  */
  LF_ERR_SCRATCH = 6      /* lf_decode_step_noalloc: the launch needs more
                             workspace than the static scratch array holds  */
} lf_status;

typedef enum { LF_DTYPE_F32 = 0, LF_DTYPE_BF16 = 1 } lf_dtype;

typedef enum {
  LF_MODE_EVICT = 0, /* LongFlow: `budget` slots, score + argmin + in-place write */
  LF_MODE_FULL = 1   /* full-KV baseline: capacity `budget`, never evicts         */
} lf_mode;

typedef enum {
  LF_ORDER_SAME_STEP = 0, /* score -> argmin -> overwrite within one step         */
  LF_ORDER_DEFERRED = 1   /* overwrite the previous step's victim, then choose    */
} lf_order;

typedef enum {
  LF_SCOPE_KV_HEAD = 0,  /* one victim per (sequence, KV head)                    */
  LF_SCOPE_SEQUENCE = 1  /* one victim per sequence, scores summed over KV heads  */
} lf_scope;

typedef enum { LF_NORM_L1 = 0, LF_NORM_L2 = 1 } lf_norm;

typedef struct {
  int32_t num_layers;   /* >= 1                                                  */
  int32_t batch;        /* sequences, >= 1                                       */
  int32_t num_q_heads;  /* multiple of num_kv_heads; G = num_q_heads/num_kv_heads */
  int32_t num_kv_heads; /* >= 1                                                  */
  int32_t head_dim;     /* 64 or 128                                             */
  int32_t budget;       /* slots per pair (EVICT) or capacity (FULL), >= 1; one
                           pair's K region (budget rounded up to 64, times
                           head_dim, times the element size) must stay under
                           4 GiB, else LF_ERR_UNSUPPORTED                         */
  int32_t sink_size;    /* slots [0, sink_size) are never evicted; < budget      */
  float softmax_scale;  /* tau; 0 selects 1/sqrt(head_dim)                      */
  int32_t dtype;        /* lf_dtype: of the cache and of q, k_new, v_new, out    */
  int32_t mode;         /* lf_mode                                               */
  int32_t order;        /* lf_order; must be 0 in FULL mode                      */
  int32_t scope;        /* lf_scope; must be 0 in FULL mode                      */
  int32_t norm;         /* lf_norm; must be 0 in FULL mode                       */
} lf_config;

/* Device addresses and strides of one layer's region (for tests, snapshots).
 *
 * K layout (16-slot tiles of 1 KB blocks). Each pair's K region holds
 * slots_padded/16 tiles of 16 slots x head_dim elements (16 * head_dim *
 * elem_bytes bytes). A row is cut into 16-byte chunks (E = 16/elem_bytes
 * elements each). Inside tile t, chunk k of slot 16t + r (r in 0..15) is
 * stored at byte offset
 *     1024 * (k / 4) + 64 * r + 16 * (k % 4),
 * so each 1 KB block holds 16 slots x 64 contiguous bytes of their rows.
 * V is row-major: element (slot i, dim d) of a pair is at i * head_dim + d. */
typedef struct {
  void* k;              /* [batch][num_kv_heads][slots_padded/16 tiles] cfg.dtype, tiled as above */
  void* v;              /* [batch][num_kv_heads][slots_padded][head_dim] cfg.dtype                */
  float* vnorm;         /* [batch][num_kv_heads][slots_padded] float32: ||v||_1 (or _2) */
  int32_t* fill;        /* [batch][num_kv_heads] int32: tokens held per pair        */
  int32_t* victim;      /* [batch][num_kv_heads] int32: LF_ORDER_DEFERRED's next
                           victim, -1 = none chosen (unused in the other order)   */
  int64_t pair_stride;  /* elements between consecutive pairs in k / v             */
  int32_t slots_padded; /* budget rounded up to a multiple of 64                    */
  int32_t elem_bytes;   /* 4 (float32) or 2 (bfloat16)                              */
} lf_view;

/* Bytes lf_cache_create would allocate for `cfg` (nothing is allocated).
 * Lets a caller size the batch to the device memory. The size follows from
 * the static buffer of `budget` slots per pair fixed up front (LongFlow
 * Guide, §Static Memory Pre-Allocation and In-Place Eviction). */
lf_status lf_cache_bytes(const lf_config* cfg, size_t* bytes);

/* Validate `cfg`, make the one device allocation on the current device, zero
 * it (every fill level starts at 0) and return the handle in *out. On error
 * *out is set to NULL and nothing stays allocated. This is the static
 * pre-allocation of LongFlow Guide, §Static Memory Pre-Allocation and
 * In-Place Eviction: one fixed buffer per pair, never resized or compacted. */
lf_status lf_cache_create(const lf_config* cfg, lf_cache** out);

/* Initial fill of one layer (LongFlow Guide, §Static Memory..., item 1).
 *   k, v          device, [batch][n_max][num_kv_heads][head_dim], cfg.dtype
 *   n_per_seq     HOST array [batch]; sequence b stores its first n_b rows in
 *                 slots 0..n_b-1 of each of its pairs; 0 <= n_b <= n_max.
 *                 n_b = -1 leaves sequence b exactly as it is (refill only
 *                 the sequences being recycled, see lf_seq_reset)
 * No victim is pending afterwards. Slots n_b..budget-1 keep what they held:
 * no step reads a slot before it has been written. Only the sequences being
 * filled are touched (and launched). k and v may be NULL when n_max = 0.
 * In FULL mode the call also sets the layer's launch order (longest
 * sequences first), which lf_seq_reset updates too; results do not depend
 * on it.
 * Errors: LF_ERR_CAPACITY if some n_b > budget; LF_ERR_INVALID_ARG on null
 * pointers, a bad layer, n_b > n_max or n_b < -1. */
lf_status lf_prefill_fill(lf_cache* c, int32_t layer, const void* k, const void* v,
                          const int32_t* n_per_seq, int32_t n_max, void* stream);

/* One fused decode step of every pair of one layer (the hot path): the
 * attention output (LongFlow Guide, §Mathematical Derivation of the LongFlow
 * Score, the alpha and o_t equations), the score alpha * ||v||_1 of every
 * cached token (same section, the c_{t,i} and Score equations; gist.science
 * summary, §2.1), and the argmin slot overwritten in place by the new token
 * (Guide, §Static Memory Pre-Allocation and In-Place Eviction, items 2-3),
 * in one pass over the cache (gist.science summary, §2.3).
 *   q             device [batch][num_q_heads][head_dim], cfg.dtype
 *   k_new, v_new  device [batch][num_kv_heads][head_dim], cfg.dtype
 *   out           device [batch][num_q_heads][head_dim], cfg.dtype; written
 *                 (bfloat16 outputs are rounded to nearest even from float32)
 *   evicted_slot  device [batch][num_kv_heads] int32; written: the slot whose
 *                 token was replaced this step, or -1 when the token was
 *                 appended
 * Accumulation is float32. Errors: LF_ERR_INVALID_ARG on null pointers or a
 * bad layer; LF_ERR_CAPACITY in FULL mode when a pair already holds
 * `budget` tokens; LF_ERR_HIP if the launch fails.
 *
 * The call queues kernel launches only (no memset, no host synchronisation)
 * and the kernels reset their own cross-workgroup counters, so it can be
 * captured into a HIP graph, alone or as part of a model step. The kernels
 * read fill levels and victims from device memory, so replays are exact.
 * The host-side bookkeeping advances once per call, not per replay: the
 * launch shape planned at capture time is kept; lf_fill_levels does not see
 * replays (read fill levels with lf_cache_snapshot); and the FULL-mode
 * capacity check cannot run inside a replay (a pair at capacity then stores
 * nothing). */
lf_status lf_decode_step(lf_cache* c, int32_t layer, const void* q, const void* k_new,
                         const void* v_new, void* out, int32_t* evicted_slot,
                         void* stream);

/* lf_decode_step without any allocation of its own, for callers that cannot
 * allocate device memory at step time: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same arguments, launches,
 * kernels and results as lf_decode_step (bit for bit); the only difference is
 * where the launch's cross-workgroup workspace lives (split-K partial states,
 * raw logits and arrival counters; the score vectors, new-token norms and
 * counters of LF_SCOPE_SEQUENCE). Here it comes from one static device array
 * of the library, 64 MiB per GPU, held by every GPU the library runs on until
 * the process ends, instead of the cache's own allocation. The array's
 * address is looked up, and its counters cleared, by the first
 * lf_cache_create on each device; the counters are back at zero after every
 * launch. The call itself allocates and frees nothing.
 *
 * Every call on one GPU shares that GPU's array: calls on one GPU whose work
 * may overlap (other streams, other handles, other threads) race and give
 * undefined results. Serialise them on one stream.
 *
 * Errors: those of lf_decode_step, and LF_ERR_SCRATCH (nothing queued) when
 * the launch's workspace does not fit in the array. The regions, each
 * rounded up to 256 bytes, must fit in 64 MiB - 64 KiB:
 *   - split-K launches need pairs * splits * (2G + G*head_dim) * 4 bytes of
 *     partial states, plus pairs * slots_padded * G * 4 bytes of logits
 *     (EVICT mode);
 *   - stream launches (lf_cache_set_stream) need the same with the cut pairs
 *     for `pairs` and 16 partial states per cut pair for `splits`;
 *   - LF_SCOPE_SEQUENCE needs pairs * (slots_padded + 1) * 4 bytes.
 * Split-K and stream launches also need at most 8192 pairs with a
 * workspace row, and LF_SCOPE_SEQUENCE batch <= 8192. Launches of whole
 * pairs with LF_SCOPE_KV_HEAD use no workspace and always fit. */
lf_status lf_decode_step_noalloc(lf_cache* c, int32_t layer, const void* q, const void* k_new,
                                 const void* v_new, void* out, int32_t* evicted_slot,
                                 void* stream);

/* Fill the view of one layer: where the static buffer of LongFlow Guide,
 * §Static Memory Pre-Allocation and In-Place Eviction, sits in device
 * memory. */
lf_status lf_cache_view(const lf_cache* c, int32_t layer, lf_view* view);

/* Snapshot of one layer (the static buffer of LongFlow Guide, §Static Memory
 * Pre-Allocation and In-Place Eviction) into caller-owned DEVICE buffers,
 * stream-ordered device-to-device copies (tests, checkpoints; the static
 * layout makes each a single contiguous copy):
 *   k, v    [batch][num_kv_heads][slots_padded*head_dim] cfg.dtype, in the
 *           layouts of lf_view (K tiled, V row-major)
 *   vnorm   [batch][num_kv_heads][slots_padded] float32
 *   fill    [batch][num_kv_heads] int32
 *   victim  [batch][num_kv_heads] int32
 * Any of the five may be NULL to skip it. */
lf_status lf_cache_snapshot(const lf_cache* c, int32_t layer, void* k, void* v, float* vnorm,
                            int32_t* fill, int32_t* victim, void* stream);

/* Launch-shape tuning of the fused pass (LongFlow Guide, §Fused
 * High-Performance Triton Attention Kernel: one pass over the cache per
 * step; these calls only choose how that pass is spread over workgroups and
 * never change what it computes beyond float32 rounding).
 *
 * Split-K. By default each launch picks how many workgroups share a
 * pair: 1 when the layer has at least as many pairs as the device has
 * compute units; otherwise about (compute units / pairs), at most
 * lf_cache_max_splits and 16, with at least 256 slots per split. The
 * workspace is sized at create for up to min(16, 512 / pairs) splits when
 * the layer has fewer than 256 pairs (none otherwise). A positive `splits`
 * forces that count (clamped to lf_cache_max_splits); 0 restores the
 * automatic choice. Results do not depend on the split count except for
 * float32 rounding of the output. */
lf_status lf_cache_set_splits(lf_cache* c, int32_t splits);
lf_status lf_cache_max_splits(const lf_cache* c, int32_t* max_splits);

/* Launch-shape tuning (as above): workgroup size of the decode launches. By
 * default a launch that holds at most one workgroup per compute unit uses 8
 * waves (512 threads) per workgroup when each workgroup streams at least 8
 * tiles of 16 slots, and any other launch 4 waves (two workgroups per
 * compute unit for large launches).
 * 4 or 8 forces that size (8 falls back to 4 where its LDS does not fit); 0
 * restores the automatic choice. Results do not depend on it except for
 * float32 rounding of the output. Errors: LF_ERR_INVALID_ARG for other
 * values. */
lf_status lf_cache_set_waves(lf_cache* c, int32_t waves);

/* Launch-shape tuning (as above): loop of the decode launches. By default a
 * launch whose workgroups each stream at most 1024 slots uses the
 * interleaved loop (each wave streams the K and the V of the same 16 slots
 * together, with its own online softmax), and longer streams the phased loop
 * (all K, then all V). 1 forces the phased loop, 2 the interleaved one, 0
 * restores the automatic choice.
 * Results do not depend on it except for float32 rounding of the output and
 * of the scores. Errors: LF_ERR_INVALID_ARG for other values. */
lf_status lf_cache_set_loop(lf_cache* c, int32_t loop);

/* Launch-shape tuning (as above): how a launch of the evicting main path
 * with no split (same-step order, one victim per KV head) spreads its pairs
 * over workgroups. With R workgroups resident on the device at once, the
 * pairs take ceil(pairs / R) rounds of whole pairs, and a part-full last
 * round leaves the device partly idle. R is the compute units for 8-wave
 * workgroups, and twice that for 4-wave ones unless LDS allows only one. By
 * default:
 *   - just past k whole rounds (k R < pairs <= (k + 0.25) R): a stream
 *     launch of R workgroups. Each takes its k whole pairs of those rounds
 *     in turn, then an equal run (at least 16 tiles of 16 slots) of the
 *     remaining pairs' tiles. A pair cut between workgroups is combined by
 *     the last of its parts to finish, as in split-K. Just past one round of
 *     the compute units this uses 8-wave workgroups; past rounds of two per
 *     compute unit, 4-wave ones. The cache holds workspace for the cut pairs
 *     of these bands on a 256-CU device (up to 512 of them), and a launch
 *     is taken only if they fit;
 *   - two rounds of 4-wave workgroups with the second 40-85% full:
 *     ceil(pairs / 2) workgroups, each taking two whole pairs in turn;
 *   - otherwise one workgroup per pair.
 * lf_cache_set_grid: a positive `workgroups` makes 4-wave launches take
 * whole pairs in turn on that many workgroups; -1 always keeps one
 * workgroup per pair (no stream launch either); 0 restores the automatic
 * choice.
 * lf_cache_set_stream: a positive `tiles` streams every pair with that many
 * tiles per workgroup, raised where a pair would be cut into more parts than
 * its workspace row holds; 0 restores the automatic choice. It takes effect
 * only where the layer's workspace holds every pair: with a split-K
 * workspace (below 256 pairs, then with lf_cache_set_splits 1), or where
 * the stream rows cover the layer.
 * Other launches (split-K, the variants, FULL mode) ignore both. Whole pairs
 * in turn give the results of one workgroup per pair bit for bit; a stream
 * launch differs only in float32 rounding of the cut pairs' outputs and
 * scores, as split-K does. Errors: LF_ERR_INVALID_ARG for workgroups < -1
 * or tiles < 0. */
lf_status lf_cache_set_grid(lf_cache* c, int32_t workgroups);
lf_status lf_cache_set_stream(lf_cache* c, int32_t tiles);

/* Host-side copy of the fill levels of one layer (tokens held per pair: the
 * initial fill of LongFlow Guide, §Static Memory Pre-Allocation and In-Place
 * Eviction, item 1, grows to the budget), [batch] int32 into the
 * caller's HOST array. Tracked on the host from the calls made (no device
 * access, no synchronisation). */
lf_status lf_fill_levels(const lf_cache* c, int32_t layer, int32_t* fill_host);

/* Recycle the regions of `count` sequences for new requests (continuous
 * batching over the static buffer, LongFlow Guide, §Static Memory
 * Pre-Allocation and In-Place Eviction: slots are reused in place, never
 * freed or compacted). In every layer, each listed sequence's pairs drop to 0
 * tokens with no pending victim; its rows are left as they are and are never
 * read again before being overwritten. Nothing is allocated or freed.
 *   seqs   HOST array [count] of sequence indices in [0, batch)
 * A later lf_prefill_fill with n_b = -1 for the other sequences loads the new
 * prompts; decode steps may also start from 0 tokens. A sequence that stays
 * idle keeps taking one token per decode step (its q, k_new, v_new rows are
 * the caller's to fill, its output is to be ignored). Stream-ordered; no
 * memset is queued (safe under graph capture). Errors: LF_ERR_INVALID_ARG on
 * a null handle, count < 0, seqs == NULL with count > 0, or an index out of
 * range. */
lf_status lf_seq_reset(lf_cache* c, const int32_t* seqs, int32_t count, void* stream);

/* Release the handle and its device memory (the static buffer of LongFlow
 * Guide, §Static Memory Pre-Allocation and In-Place Eviction, freed once).
 * NULL is a no-op. The caller must make sure no queued work still uses the
 * cache. */
void lf_cache_destroy(lf_cache* c);

/* Static string naming a status code. No page defines it: it names this
 * library's own error codes. */
const char* lf_status_str(lf_status s);

#ifdef __cplusplus
}
#endif

#endif /* LONGFLOW_H */
