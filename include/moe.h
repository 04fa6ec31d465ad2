/*
 * moe.h -- C ABI of the gfx950 routed-expert MoE FFN library (libmoe.so).
 *
 * One MoE FFN layer, per token: an int8 router scores all E experts; a
 * softmax top-K picks K of them and renormalises their coefficients over the
 * chosen set; each chosen expert runs a SwiGLU FFN whose weights are affine
 * 4-bit with one (scale, bias) pair per 64 inputs of a row; an always-on
 * shared expert is added with unit weight; the result is the weighted sum.
 *   BigMoeOnEdge (onecrewdev), section "re-routing at every token and layer":
 *     router scores -> top-K experts with coefficients -> weighted merge
 *     y = sum_j w_j * Expert_j(x); the shared path is not counted among K.
 *   Rockchip-NPU MoE streaming plan (cnblogs), §2.1/§2.5: affine 4-bit
 *     group-64 expert weights, 8-bit router; §2.4: the shared expert is fused
 *     with the weighted routed outputs; §6.2.2 and §9.5: a per-layer 16-slot
 *     LFU expert cache; §8.4: 128-token prefill chunks.
 *
 * Conventions for every function:
 *  - Returns moe_status; nothing throws across the ABI.  On a non-OK status
 *    moe_last_error() returns a message for the calling thread, and any
 *    output buffers are undefined.
 *  - "DEVICE" pointers are HIP device memory owned by the caller; "HOST"
 *    pointers are ordinary host memory owned by the caller.
 *  - `stream` arguments are hipStream_t values passed as void* (NULL = the
 *    default stream).  Work is enqueued on that stream; functions return
 *    without waiting for the GPU unless stated otherwise.
 *  - One host thread may use a given layer/stack object at a time.  Distinct
 *    objects may be used concurrently on distinct streams.
 *  - Calls on one object must run in order on the GPU (one stream, or streams
 *    ordered with events): every call reuses the object's device workspace
 *    (routing, activations, the fused kernel's counters, a streamed layer's
 *    expert table and slots).
 */
#ifndef MOE_H
#define MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1, /* bad argument or descriptor */
  MOE_ERR_NOMEM = 2,   /* device or pinned host allocation failed */
  MOE_ERR_HIP = 3,     /* a HIP runtime call failed */
  MOE_ERR_IO = 4,      /* an expert could not be brought into its cache slot */
  MOE_ERR_STATE = 5    /* call not valid in the object's current state */
} moe_status;

enum { MOE_ACT_F32 = 0, MOE_ACT_BF16 = 1 };        /* activation dtype of x / out */
enum { MOE_RESIDENT = 0, MOE_STREAMED = 1 };        /* where routed experts live */
/* Execution paths of a forward call:
 *   DECODE  three kernels per layer (router + shared gate/up | routed gate/up |
 *           down + combine), any T, fp32 or bf16, resident or streamed;
 *   FUSED   one kernel per layer for a single bf16 token on resident experts
 *           (its workgroups hand results to each other through device-scope
 *           flags and counters), for d_model <= 4096 when its LDS fits;
 *           MOE_ERR_INVALID otherwise;
 *   PREFILL grouped bf16 matrix-core GEMMs for 128-token chunks, on resident
 *           experts or on streamed experts through the layer's own LFU cache
 *           (moe_cache_attach; not a shared pool): each chunk's experts are
 *           taken in groups of at most the slot count (cached ones first,
 *           then least chosen first), the GEMMs run per group, and the call
 *           blocks the thread once per chunk to read its expert counts.
 * AUTO takes FUSED where it applies, PREFILL for T >= 16 bf16 layers (resident,
 * or streamed with an LFU cache) with d_model <= 4096 and no rmsnorm, DECODE
 * otherwise. */
enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_PREFILL = 2, MOE_PATH_FUSED = 3 };

typedef struct moe_layer moe_layer; /* opaque, owned by the library */
typedef struct moe_stack moe_stack; /* opaque, owned by the library */
typedef struct moe_lfu moe_lfu;     /* opaque host-only cache policy object */
typedef struct moe_lru moe_lru;     /* opaque host-only policy of a shared pool */
typedef struct moe_cache_pool moe_cache_pool; /* opaque expert cache shared by layers */

/*
 * Layer descriptor.  All weight pointers are HOST pointers in the canonical
 * layout below; moe_layer_create copies them, so the caller may free them as
 * soon as it returns.
 *
 * A 4-bit matrix with R rows (outputs) and C columns (inputs), C % 64 == 0:
 *   q  uint32 [R][C/8]  : nibble k (bits 4k..4k+3) of word j is q[row][8j+k]
 *   s  uint16 [R][C/64] : fp16 scale of the 64-column group
 *   b  uint16 [R][C/64] : fp16 bias of the 64-column group
 *   weight[row][col] = s[row][col/64] * q[row][col] + b[row][col/64]
 * Routed experts are stacked along a leading expert axis [E]:
 *   gate, up: R = d_ff, C = d_model;   down: R = d_model, C = d_ff.
 * The shared expert uses d_ff_shared (0 = no shared expert; pointers NULL).
 * Router: int8 [E][d_model], fp16 per-row scale [E], optional fp32 per-expert
 *   logit bias [E]:  logit_e = scale_e * sum_c W[e][c] * x[c] + bias_e.
 */
typedef struct {
  int32_t d_model;     /* multiple of 64, <= 8192 */
  int32_t n_experts;   /* E, 1..1024 */
  int32_t top_k;       /* K, 1..min(E, 64) */
  int32_t d_ff;        /* routed expert hidden size, multiple of 64 */
  int32_t d_ff_shared; /* shared expert hidden size, multiple of 64, or 0 */
  int32_t act_dtype;   /* MOE_ACT_F32 or MOE_ACT_BF16 */
  int32_t max_tokens;  /* largest n_tokens any forward call will pass (>= 1) */
  int32_t residency;   /* MOE_RESIDENT: all experts in HBM; MOE_STREAMED:
                          routed experts in pinned host memory, served through
                          a per-layer HBM slot cache (see moe_cache_attach) */
  const int8_t* router_w;
  const uint16_t* router_scale;
  const float* router_bias; /* may be NULL */
  const uint32_t* gate_q;
  const uint16_t* gate_s;
  const uint16_t* gate_b;
  const uint32_t* up_q;
  const uint16_t* up_s;
  const uint16_t* up_b;
  const uint32_t* down_q;
  const uint16_t* down_s;
  const uint16_t* down_b;
  const uint32_t* sh_gate_q;
  const uint16_t* sh_gate_s;
  const uint16_t* sh_gate_b;
  const uint32_t* sh_up_q;
  const uint16_t* sh_up_s;
  const uint16_t* sh_up_b;
  const uint32_t* sh_down_q;
  const uint16_t* sh_down_s;
  const uint16_t* sh_down_b;
} moe_layer_desc;

/* Validates the descriptor, repacks the weights into the library's device
 * layout and allocates the layer's device workspace.  Blocks until the copies
 * are done.  Errors: MOE_ERR_INVALID (shape limits above, NULL weights),
 * MOE_ERR_NOMEM, MOE_ERR_HIP. */
moe_status moe_layer_create(const moe_layer_desc* desc, moe_layer** out);

/* Frees everything the layer owns (waits for the device first). NULL is OK. */
moe_status moe_layer_destroy(moe_layer* layer);

/* out[t] = MoE(x[t]) for t < n_tokens.
 * x, out: DEVICE [n_tokens][d_model] of act_dtype, row-major; may not alias.
 * n_tokens: 0..max_tokens (0 is a no-op).
 * Resident layers: only enqueues work on `stream`.  Streamed layers: blocks
 * the calling thread until the routing of this call is known on the host,
 * then enqueues the cache fills and the compute that needs them.  With one
 * token (top_k <= 32) the router, routed gate/up and down kernels are all
 * enqueued first: the gate/up launch runs the top-K, writes the routing into
 * pinned host memory (the thread spins on it, up to about 2 s, then waits for
 * the stream) and computes the experts that are cached; the down kernel runs
 * when all were.  A miss then costs a fill kernel, a gate/up launch for the
 * missed experts and the down kernel again.  More tokens: one small
 * device->host copy and a stream synchronisation.  A one-token call with
 * reuse_previous right after another one-token call of the layer already
 * has its sets on the host and does not wait, unless the layer's device
 * expert table has to be uploaded in that call. */
moe_status moe_layer_forward(const void* x, moe_layer* layer, void* out, int32_t n_tokens, void* stream);

/* Optional controls of one forward call.  Every field may be 0/NULL. */
typedef struct {
  int32_t* topk_ids;          /* DEVICE [T][K] out: chosen experts, ascending */
  float* topk_w;              /* DEVICE [T][K] out: their coefficients */
  const int32_t* forced_ids;  /* DEVICE [T][K] in: use these (ascending, distinct,
                                 < E) expert sets instead of the top-K; the
                                 coefficients are renormalised from this call's
                                 logits over the given set */
  int32_t reuse_previous;     /* nonzero: use the expert sets of this layer's
                                 previous forward call (same n_tokens; a
                                 moe_layer_route call in between replaces
                                 them), with coefficients from this call's
                                 logits */
  int32_t path;               /* MOE_PATH_* (see above) */
  int32_t residual;           /* nonzero: out = act(x_in + y) where x_in is the
                                 `residual_src` tensor (stack glue) */
  const void* residual_src;   /* DEVICE [T][d_model] of act_dtype, or NULL */
  int32_t* sort_offsets;      /* DEVICE [ceil(T/128)][E+1] out (prefill path
                                 only): the grouping of each 128-token chunk,
                                 offsets into that chunk's part of sort_perm */
  int32_t* sort_perm;         /* DEVICE [T*K] out (prefill path only): chunk c
                                 fills entries [128*c*K, 128*c*K + C*K) with
                                 its pairs in (expert, token) order, each as
                                 (t - 128*c)*K + k (chunk-local token index) */
} moe_fwd_opts;

moe_status moe_layer_forward_ex(const void* x, moe_layer* layer, void* out, int32_t n_tokens,
                                const moe_fwd_opts* opts, void* stream);

/* For callers that cannot allocate device memory during a call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * out[t] = MoE(x[t]) as moe_layer_forward with MOE_PATH_DECODE on a resident
 * layer (same kernels, same results bit for bit), its per-call workspace
 * (logits, routing, activations) taken from a device array of the library,
 * 8 MiB per GPU, held until the process ends.  The call allocates nothing and
 * calls no allocating routine; the caller passes x and out as for
 * moe_layer_forward.  n_tokens is limited by the array: about 16 KB per token
 * for the bf16 d_model 2816 / 128-expert / K 8 layer; larger calls fail with
 * MOE_ERR_INVALID.  Every such call on one GPU shares the array, so calls
 * that overlap on one GPU (different streams, not ordered) race and give
 * undefined results.  Streamed layers: MOE_ERR_INVALID.  The layer's error
 * flags (moe_layer_check_errors) report as for its other calls. */
moe_status moe_layer_forward_noalloc(const void* x, moe_layer* layer, void* out, int32_t n_tokens, void* stream);

/* Router + softmax top-K only: ids DEVICE int32 [T][K] (ascending per token),
 * w DEVICE fp32 [T][K].  The gating of BigMoeOnEdge, section "re-routing at
 * every token and layer", and the Rockchip-NPU plan, section 2.1: a softmax
 * over all experts, the K largest kept, their weights renormalised. */
moe_status moe_layer_route(const void* x, moe_layer* layer, int32_t* ids, float* w, int32_t n_tokens,
                           void* stream);

/* Token->expert grouping of a [T][K] id array (ascending per row, < E):
 * counts[E], offsets[E+1] (exclusive scan), perm[T*K] = t*K+k ordered by
 * (expert, token), inv[T*K] = position of pair t*K+k in perm.  All DEVICE,
 * T <= max_tokens of the layer.  Rockchip-NPU plan §8.4 (one fetched expert
 * serves all rows of the chunk that chose it). */
moe_status moe_layer_sort(const int32_t* ids, moe_layer* layer, int32_t n_tokens, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, void* stream);

/* Bytes the layer keeps in device memory, and the per-expert byte size
 * (gate + up + down at 4.5 bits per weight, padded to 256 B).  A library
 * utility: no passage of the pages defines it. */
moe_status moe_layer_bytes(const moe_layer* layer, uint64_t* device_bytes, uint64_t* expert_bytes);

/* Waits for the device, then returns and clears the layer's sticky kernel
 * error flags in *flags (HOST); a library utility, no passage of the pages
 * defines it:
 *   bit 0  a forced expert id was outside 0..E-1 (it was replaced by 0);
 *   bit 1  a chosen expert was not resident (its output read as zero);
 *   bit 2  a workgroup gave up waiting for another one's results: a bounded
 *          wait of the fused kernel ran out (seconds; for example when
 *          another process holds most of the GPU);
 *   bit 3  an intermediate activation |silu(gate.x) * up.x| reached 65504,
 *          the largest fp16 value: bf16 layers on the DECODE and FUSED paths
 *          hand these activations between kernels as fp16, so such inputs are
 *          outside their range (the PREFILL path keeps them in bf16).
 * Any set bit means the output of some call since the last check is not
 * valid.  The forward calls return MOE_OK without waiting for the GPU, so
 * MOE_OK from a call does not prove that its output is valid: check the
 * flags after the calls whose outputs matter. */
moe_status moe_layer_check_errors(moe_layer* layer, int32_t* flags);

/* The path run by calls that pass MOE_PATH_AUTO (moe_layer_forward, a NULL
 * opts, and every layer call of moe_stack_forward); MOE_PATH_AUTO (the
 * default) picks per call as described at moe_fwd_opts.path.  The paths differ
 * in rounding: the fused kernel hands its intermediate activations between
 * workgroups as fp16 with 9 mantissa bits, the others as full fp16.  So a
 * streamed layer (always MOE_PATH_DECODE) is bit-identical to a resident one
 * set to MOE_PATH_DECODE.  A call the chosen path cannot serve fails with
 * MOE_ERR_INVALID, as with an explicit path.  MOE_ERR_INVALID for unknown
 * values. */
moe_status moe_layer_set_default_path(moe_layer* layer, int32_t path);

/* Per-kernel timing (a library utility: no passage of the pages defines it).
 * enable != 0 brackets every kernel the layer launches
 * with HIP events on the launch stream; 0 stops and discards the record.
 * moe_layer_profile_read waits for the device, then fills HOST arrays
 * launches[MOE_N_KERNELS] and total_ms[MOE_N_KERNELS] (index = MOE_KERNEL_*)
 * with the launches timed since the last read and their summed durations. */
enum {
  MOE_KERNEL_ROUTE_SHARED = 0,   /* router GEMV + shared gate/up (decode) */
  MOE_KERNEL_ROUTED_GATE_UP = 1, /* top-K + chosen experts' gate/up + SiLU*mul (decode) */
  MOE_KERNEL_DOWN_COMBINE = 2,   /* down projections + weighted combine (decode) */
  MOE_KERNEL_SORT = 3,           /* token->expert grouping (moe_layer_sort; prefill groups in its router launch) */
  MOE_KERNEL_PREFILL_GATE_UP = 4,
  MOE_KERNEL_PREFILL_DOWN = 5,
  MOE_KERNEL_PREFILL_COMBINE = 6,
  MOE_KERNEL_PREFILL_ROUTE = 7,  /* router + top-K of every token of a prefill call, and each chunk's grouping */
  MOE_KERNEL_TOPK = 8,           /* stand-alone softmax top-K */
  MOE_KERNEL_FUSED_LAYER = 9,    /* whole layer for one token in one launch */
  MOE_N_KERNELS = 10
};
moe_status moe_layer_profile(moe_layer* layer, int32_t enable);
moe_status moe_layer_profile_read(moe_layer* layer, int64_t* launches, double* total_ms);

/* ---- expert cache (MOE_STREAMED layers) --------------------------------
 * Rockchip-NPU plan §6.2.2/§6.2.3/§9.5: per-layer slots, LFU eviction; the
 * cache entry keeps a use count and a last-used tick.  Policy: a hit adds
 * one to the entry's count; a miss takes the lowest empty slot, else evicts
 * the entry with the least (count, last-used tick, slot) among entries not
 * chosen by the current call; a new entry starts at count 1; counts are
 * never aged.  Fills are copy kernels on the call's stream that read the
 * pinned host store over the host link (about 50 GB/s; DMA copies measured
 * 43 GB/s on one stream and far less on two) and write the slots and the
 * layer's device expert table. */

/* Allocates n_slots HBM slots (n_slots >= top_k * max_tokens is not required;
 * n_slots >= the number of distinct experts a single call can choose is:
 * calls needing more return MOE_ERR_STATE).  side_stream carries the
 * fetch-ahead copies (moe_cache_prefetch, moe_stack_set_prefetch); it may be
 * NULL, in which case the library creates one.  Errors: MOE_ERR_STATE if the
 * layer is not MOE_STREAMED or already has a cache. */
moe_status moe_cache_attach(moe_layer* layer, int32_t n_slots, void* side_stream);

typedef struct {
  uint64_t accesses;   /* one per (call, token, chosen expert) that was looked up */
  uint64_t hits;
  uint64_t misses;
  uint64_t evictions;  /* entries replaced (by a miss or a prefetch) */
  uint64_t h2d_bytes;  /* (misses + prefetches) * expert bytes */
  uint64_t h2d_ns;     /* span of each call's fills, first copy start to last copy end (GPU event
                          clock), summed */
  uint64_t prefetches;    /* experts placed ahead of use (moe_cache_prefetch) */
  uint64_t prefetch_used; /* of those, the ones a call then hit */
  uint64_t ahead_slots;   /* one-token calls: routed slots computed by the kernels queued before the
                             call's cache step (its hits, which the device expert table marks) */
} moe_cache_stats;

moe_status moe_cache_stats_get(const moe_layer* layer, moe_cache_stats* out);
/* Clears the counters; drop_contents != 0 also empties every slot. */
moe_status moe_cache_reset(moe_layer* layer, int32_t drop_contents);
/* HOST outputs [n_slots]: expert held by each slot (-1 = empty), use count. */
moe_status moe_cache_contents(const moe_layer* layer, int32_t* expert_of_slot, uint32_t* use_count);
/* Test hook: make expert `expert` unreadable (1) or readable (0).  A decode
 * call that needs to fill an unreadable expert returns MOE_ERR_IO before
 * enqueuing any expert compute and leaves the slot table unchanged.  A
 * prefill call returns MOE_ERR_IO at the group that needs it: the groups and
 * chunks before it have already stepped the cache and run, so the slot table
 * holds their experts and the call's output is incomplete. */
moe_status moe_cache_fail_expert(moe_layer* layer, int32_t expert, int32_t fail);

/* Fetch ahead into a layer's own (LFU) cache, Rockchip-NPU plan §8
 * ("readahead": predict the next layer's experts from the routing history
 * and start reading them during the current layer) and §9.5 item 2.  The
 * absent ones of experts[n] (HOST ids) are placed as described at
 * moe_lfu_prefetch and copied on the layer's side stream; the layer's next
 * call waits for those copies.  `stream` is the stream the layer's calls run
 * on: this call first waits for it, so no slot still in use is refilled.
 * Unreadable experts (moe_cache_fail_expert) are skipped.  MOE_ERR_STATE
 * without a per-layer cache. */
moe_status moe_cache_prefetch(moe_layer* layer, const int32_t* experts, int32_t n, void* stream);

/* ---- shared expert cache under a byte budget (LRU) ---------------------
 * BigMoeOnEdge, "the cache manages the expert working set": one cache keyed
 * by (layer, expert) for all layers, a byte budget for expert weights only,
 * least recently used entries evicted first, the working set in use
 * protected.  Here: budget_bytes / expert_bytes slots of one expert blob each
 * (moe_layer_bytes gives expert_bytes; every layer attached must have that
 * size).  Policy: a call's hits are touched first; each miss takes the
 * lowest empty slot, else evicts the entry (of any layer) with the oldest
 * last use, lower slot first on ties, never an entry chosen by the same
 * call; misses are placed in ascending expert order.  Fills are copy
 * kernels on the call's stream, as for per-layer caches.  Layers sharing a
 * pool must be called from one stream (or calls ordered), since a call may
 * refill a slot another layer used last.  The pool does no fetch-ahead:
 * side_stream is accepted for symmetry with moe_cache_attach and not used. */
moe_status moe_cache_pool_create(uint64_t budget_bytes, uint64_t expert_bytes, void* side_stream,
                                 moe_cache_pool** out);
/* The layers that use it keep running only after another cache is
 * attached. */
moe_status moe_cache_pool_destroy(moe_cache_pool* pool);
/* In place of moe_cache_attach.  The layer's key in the pool is the number
 * of layers attached before it.  MOE_ERR_STATE if the layer is not
 * MOE_STREAMED or has a cache; MOE_ERR_INVALID if its expert size or device
 * differs from the pool's or the pool cannot hold one call's experts. */
moe_status moe_cache_attach_pool(moe_layer* layer, moe_cache_pool* pool);
/* Drop the layer's cache (its own slots, or its entries in a pool) and its
 * counters; another cache may then be attached. */
moe_status moe_cache_detach(moe_layer* layer);
/* Totals over the pool (per-layer shares: moe_cache_stats_get). */
moe_status moe_cache_pool_stats(const moe_cache_pool* pool, moe_cache_stats* out);
/* HOST outputs [budget_bytes / expert_bytes]: key of the layer and expert
 * held by each slot (-1 = empty). */
moe_status moe_cache_pool_contents(const moe_cache_pool* pool, int32_t* layer_of_slot, int32_t* expert_of_slot);

/* ---- stack of layers (decode through many MoE layers) ------------------
 * h <- act(h + MoE_l(act(rmsnorm(h)))) for each layer l in order, where
 * rmsnorm(h) = h / sqrt(mean(h^2) + eps) with unit gain. */
moe_status moe_stack_create(moe_layer* const* layers, int32_t n_layers, float rms_eps, moe_stack** out);
/* h: DEVICE [n_tokens][d_model], updated in place.  reuse_mask: HOST
 * [n_layers] or NULL; nonzero entries make that layer reuse its previous
 * call's expert sets (see moe_fwd_opts.reuse_previous).  ids_out: DEVICE
 * [n_layers][n_tokens][K] or NULL. */
moe_status moe_stack_forward(void* h, moe_stack* stack, int32_t n_tokens, const uint8_t* reuse_mask,
                             int32_t* ids_out, void* stream);
/* Fetch ahead in a stack of streamed layers with per-layer caches: once a
 * layer's routing is back on the host (and its own fills are queued), the
 * next layer's `depth` most often chosen experts so far (ties to the lower
 * id) that are not in its cache are prefetched, so their copies overlap the
 * current layer's expert compute.  0 (the default) turns it off; depth is at
 * most 64. */
moe_status moe_stack_set_prefetch(moe_stack* stack, int32_t depth);
moe_status moe_stack_destroy(moe_stack* stack);

/* ---- host-only cache policy (no GPU needed) ----------------------------
 * The same policy object the streamed layers use, exposed for checking. */
moe_status moe_lfu_create(int32_t n_slots, moe_lfu** out);
/* chosen: HOST [n] distinct expert ids of one call.  slot_out[n], miss_out[n]
 * (HOST) receive the slot of each id and 1 where it was a miss. */
moe_status moe_lfu_step(moe_lfu* lfu, const int32_t* chosen, int32_t n, int32_t* slot_out, int32_t* miss_out);
moe_status moe_lfu_stats(const moe_lfu* lfu, moe_cache_stats* out);
/* Place the absent ones of experts[n] ahead of use, in ascending id order,
 * without counting an access: each takes the lowest empty slot, else evicts
 * as a miss would, but never an entry placed by the same prefetch nor one
 * the last call used (the working set; the guess is dropped when no other
 * slot is left); a new entry
 * starts at use count 0 with the last call's tick, and a later call's hit on
 * it counts in prefetch_used.  slot_out[n] (HOST): slot given, or -1 where
 * the expert was already present (or no slot was left). */
moe_status moe_lfu_prefetch(moe_lfu* lfu, const int32_t* experts, int32_t n, int32_t* slot_out);
moe_status moe_lfu_destroy(moe_lfu* lfu);
/* The shared pool's LRU policy: one call of the layer with key `layer`
 * (>= 0); arguments as moe_lfu_step. */
moe_status moe_lru_create(int32_t n_slots, moe_lru** out);
moe_status moe_lru_step(moe_lru* lru, int32_t layer, const int32_t* chosen, int32_t n, int32_t* slot_out,
                        int32_t* miss_out);
moe_status moe_lru_stats(const moe_lru* lru, moe_cache_stats* out);
moe_status moe_lru_destroy(moe_lru* lru);

/* ---- test hooks ----------------------------------------------------------
 * Dequantise matrix `which` (0 gate, 1 up, 2 down) of routed expert `expert`
 * (-1: the shared expert) on the GPU from the library's device layout, with
 * the same addressing as the GEMV kernels: host_out[r][c] =
 * fma(scale, q, bias) in fp32, [rows][cols] row-major (gate/up: d_ff x
 * d_model, down: d_model x d_ff).  Blocks; allocates a temporary device
 * buffer.  Checks the device repack against the canonical layout (an
 * all-q = 8 group gives 8*scale + bias; a one-hot nibble lands at its own
 * row and column). */
moe_status moe_debug_dequant(const moe_layer* layer, int32_t which, int32_t expert, float* host_out);
/* How long a streamed one-token call spins for its routing in host memory
 * before it waits for the stream instead (default 2 000 000 us).  0 makes
 * every such call take the waiting branch, which must give the same output. */
moe_status moe_debug_host_wait(moe_layer* layer, int64_t microseconds);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
