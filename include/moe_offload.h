/* moe_offload.h - C ABI of the expert-offload MoE layer step on one MI355X (gfx950).
 *
 * One MoE layer step: router GEMM, renormalised softmax top-k, per-step dedup of
 * the selected experts, hit/miss classification against one GPU slot cache shared
 * by all MoE layers and keyed by (layer, expert), LRU victim selection and slot
 * table update, miss fills from a pinned host expert pool into the cache slots on
 * a side stream in double-buffered groups, and the SwiGLU expert FFN over the
 * tokens gathered per expert; plus elastic resize of the cache at a safe point.
 *
 * Sources (the FreeToken pages):
 *  - FreeToken paper summary (agihunt.info, arXiv 2608.16157), memory-architecture
 *    paragraph: full expert pool in host memory, non-expert weights on the GPU, the
 *    rest of VRAM one elastic expert cache shared by all MoE layers with slots
 *    managed by the logical id (layer, expert).
 *  - same page, execution-layer paragraph: per layer one kernel does routing dedup,
 *    hit classification and LRU victim selection with no per-layer host sync; the
 *    cache is rebuilt at a scheduler safe point when the VRAM budget changes;
 *    weights are stored in their runtime layout so a load lands in its final place.
 *  - same page, problem paragraph: VRAM budgets change during a session.
 *  - same page, last paragraph: the host pool must be pinned and DMA-registered.
 *  - "FreeToken vs vLLM on one RTX 3090" report, "FreeToken exploits MoE sparsity":
 *    a fixed number of routed experts per token, an LRU expert cache, only selected
 *    experts fetched on demand.
 *  - "FreeToken：在消费级 NVIDIA GPU 上进行 MoE 推理", "FreeToken 解决的问题": while
 *    one group of experts computes, the next group transfers (double buffering).
 *
 * Conventions.
 *  - Every call returns moe_status.  Arguments are checked on the host before any
 *    work is enqueued; a call that fails changes no state.  No exception crosses
 *    the ABI.
 *  - Device buffers, the pinned host pool and the streams belong to the caller.
 *    The library owns only its opaque handle and the HIP events it creates; it
 *    never allocates device memory (the caller passes a workspace of
 *    moe_workspace_bytes()).  moe_host_pool_alloc() is a convenience wrapper
 *    around hipHostMalloc for callers without their own pinned allocator.
 *  - Streams are hipStream_t values passed as void*; NULL is the null stream.
 *  - All step calls are asynchronous and stream ordered; none synchronises the
 *    host and none allocates, so a caller may capture them into a hipGraph with
 *    stream capture.  moe_cache_snapshot, moe_plan_read and moe_stats synchronise.
 *  - Not thread-safe: one handle is driven from one host thread.
 *
 * Layouts (row-major).
 *  - x: [T][hidden] bf16 layer input.  y: [T][hidden] bf16 layer output.
 *  - w_router: [experts][hidden] bf16 router weights of the layer.
 *  - topk_idx: [T][top_k] int32, by descending router logit, ties to the lower id.
 *    topk_w: [T][top_k] fp32, renormalised softmax over the selected logits.
 *  - host pool: layers*experts blobs of blob_bytes, blob (l, e) at offset
 *    (l*experts + e)*blob_bytes.  A cache slot holds one blob, byte-identical.
 *  - blob, bf16 (wfmt 0): Wgu[I][2][H] (gate row i then up row i), WdT[I][H].
 *    fp8 (wfmt 1): e4m3fn codes Wgu[I][2][H], WdT[I][H], then fp32 scales
 *    s_gu[I][2][H/128], s_d[I/128][H]; one scale per 128 contraction elements.
 *    mxfp4 (wfmt 2): e2m1 codes two per byte (even element low nibble)
 *    Wgu[I][2][H/2], WdT[I][H/2], then e8m0 scales s_gu[I][2][H/32], s_d[I/32][H].
 *    H = hidden, I = inter.  WdT row i is column i of the down projection Wd[H][I].
 *  - shared expert (has_shared): one more blob in the same format, resident on the
 *    GPU, added to every token with weight 1; it is not cached and not pooled.
 */
#ifndef MOE_OFFLOAD_H
#define MOE_OFFLOAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_E_INVALID (-1)  /* bad shape, pointer, format, size or call order */
#define MOE_E_CAPACITY (-2) /* capacity below min(max_tokens*top_k, experts) or above max */
#define MOE_E_BUSY (-3)     /* resize or snapshot while a step is in flight */
#define MOE_E_HIP (-4)      /* a HIP runtime call failed; see moe_last_hip_error */
#define MOE_E_NOMEM (-5)    /* pinned host allocation failed */
#define MOE_E_HYBRID (-6)   /* hybrid decode: the host did not answer a step within ~2 s */
#define MOE_E_SCRATCH (-7)  /* workspace above the static workspace (moe_cache_create_static) */

#define MOE_FMT_BF16 0
#define MOE_FMT_FP8_E4M3_K128 1
#define MOE_FMT_MXFP4_K32 2

typedef struct moe_cache_s* moe_cache;

typedef struct {
  int32_t layers;     /* MoE layers sharing the cache */
  int32_t experts;    /* routed experts per layer, <= 1024 */
  int32_t top_k;      /* experts selected per token, 1..16 */
  int32_t hidden;     /* H, multiple of 256 */
  int32_t inter;      /* I, SwiGLU intermediate size, multiple of 128 */
  int32_t wfmt;       /* MOE_FMT_* */
  int32_t has_shared; /* 1: one GPU-resident shared expert per layer */
  int32_t max_tokens; /* largest T passed to any step call, 1..65536 (see below) */
  int64_t blob_bytes; /* must equal moe_blob_bytes(wfmt, hidden, inter) */
} moe_shape;

/* Plan of the last routed step, copied to the host (parity and tests). */
typedef struct {
  int32_t n_unique, n_hit, n_miss, layer;
  int64_t step;
  int32_t n_cpu, pad_;  /* misses computed in place by the CPU (hybrid decode) */
  int32_t* unique;    /* [n_unique] distinct experts, ascending */
  int32_t* slot;      /* [n_unique] cache slot of each, after the step */
  uint8_t* hit;       /* [n_unique] 1 = was cached before the step */
  int32_t* miss_key;  /* [n_miss] key = layer*experts + expert, ascending expert */
  int32_t* miss_slot; /* [n_miss] slot filled */
  int32_t* miss_victim; /* [n_miss] evicted key, or -1 for a free slot */
  int32_t* count;     /* [n_unique] assignments per distinct expert */
  int32_t* perm;      /* [T*top_k] assignment ids t*top_k+j grouped by expert, ascending t */
  int32_t* cpu_key;   /* [n_cpu] keys of the CPU misses, ascending expert (may be NULL) */
} moe_plan_host;      /* caller-owned arrays sized for min(max_tokens*top_k, experts) / T*top_k */

typedef struct {
  int64_t steps, hits, misses, bytes_filled;
  int64_t cpu_misses; /* misses computed in place by the CPU (hybrid decode) */
} moe_counters;

/* Bytes of one expert blob, or -1 for an unsupported shape. */
int64_t moe_blob_bytes(int32_t wfmt, int32_t hidden, int32_t inter);

/* Device workspace bytes for a cache of up to max_capacity slots. */
size_t moe_workspace_bytes(const moe_shape* shape, int32_t max_capacity);

/* Budget-driven cache size ("FreeToken vs vLLM on one RTX 3090", Runtime configurations: an
 * automatic cache; "FreeToken: az VRAM ile büyük MoE modelleri", "KV cache": a KV floor is
 * reserved first; "FreeToken：在消费级 NVIDIA GPU 上进行 MoE 推理": --offload-ratio r keeps the
 * fraction 1 - r of the experts on the GPU).  *capacity = the largest C with
 * C * blob_bytes + moe_workspace_bytes(shape, C) <= free_bytes - reserve_bytes (reserve: the
 * KV floor and anything else that must stay resident), at most layers * experts, at most the
 * slot limit of a handle (4,096), and at most floor((1 - offload_ratio) * layers * experts)
 * when 0 <= offload_ratio < 1 (a negative ratio: no such limit).  Host arithmetic only.
 * MOE_E_CAPACITY when not even the floor min(max_tokens * top_k, experts) fits;
 * MOE_E_INVALID for a bad shape or offload_ratio >= 1. */
moe_status moe_auto_capacity(const moe_shape* shape, uint64_t free_bytes, uint64_t reserve_bytes,
                             double offload_ratio, int32_t* capacity);

/* moe_auto_capacity over the current device's free memory as hipMemGetInfo reports it now
 * (the budget the pages size the automatic cache from: the VRAM left once the resident
 * weights are loaded, minus the KV floor in reserve_bytes).  *free_bytes (may be NULL)
 * receives the free byte count used.  MOE_E_HIP if the query fails; otherwise as
 * moe_auto_capacity. */
moe_status moe_auto_capacity_device(const moe_shape* shape, uint64_t reserve_bytes,
                                    double offload_ratio, int32_t* capacity,
                                    uint64_t* free_bytes);

/* Expert pool files in the runtime layout (the FreeToken paper summary, execution-layer
 * paragraph: weights merged ahead of time into the runtime layout load straight into their
 * final place).  A 64-byte header (magic "MOEPOOL1", int32 layers, experts, hidden, inter,
 * wfmt, pad, int64 blob_bytes, int64 blob count) and then the layers * experts blobs in key
 * order.  moe_pool_write stores a pool; moe_pool_read fills `pool` (host memory of
 * layers * experts * blob_bytes bytes, normally from moe_host_pool_alloc, so the blobs land
 * in pinned memory directly) with `threads` parallel readers.  MOE_E_INVALID on an I/O error,
 * a header that does not match `shape`, or a file of the wrong size. */
moe_status moe_pool_write(const char* path, const moe_shape* shape, const void* pool,
                          int32_t threads);
moe_status moe_pool_read(const char* path, const moe_shape* shape, void* pool, int32_t threads);

/* Pinned, device-accessible host memory for the expert pool (hipHostMalloc).
 * Returns MOE_E_NOMEM when the allocation fails.  Free with moe_host_pool_free. */
moe_status moe_host_pool_alloc(size_t bytes, void** out);
moe_status moe_host_pool_free(void* p);

/* Create a cache of `capacity` slots (slot i at slot_arena + i*blob_bytes) over the
 * pinned host pool.  slot_arena must hold max_capacity slots; workspace must be
 * moe_workspace_bytes(shape, max_capacity) bytes of device memory, 256-byte
 * aligned.  host_pool must come from hipHostMalloc (moe_host_pool_alloc).  The
 * cache starts empty; its state is initialised on `stream` (asynchronously).
 * Errors: MOE_E_INVALID, MOE_E_CAPACITY (capacity < min(max_tokens*top_k, experts)
 * or capacity > max_capacity), MOE_E_NOMEM (pool not device-accessible), MOE_E_HIP. */
moe_status moe_cache_create(const moe_shape* shape, int32_t capacity, int32_t max_capacity,
                            void* slot_arena, void* workspace, const void* host_pool,
                            void* stream, moe_cache* out);

/* For callers that cannot allocate device memory (code under hipGraph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_cache_create with the workspace taken from the
 * library's own static device array of 16 MiB per device (enough for the decode handles of
 * every shape here; moe_workspace_bytes(shape, max_capacity) must not exceed it, else
 * MOE_E_SCRATCH).  Allocates nothing, on the device or through any allocating library
 * routine; the handle's state is initialised on `stream` as with moe_cache_create.  The
 * array is shared by every call on the device and keeps the last handle's contents: at most
 * one live handle per device may hold it (a second create while one lives returns
 * MOE_E_BUSY; overlapping use would race); moe_cache_destroy gives it back.  Events are
 * created only when a step first joins two queues (groups >= 1 or prefetch). */
moe_status moe_cache_create_static(const moe_shape* shape, int32_t capacity,
                                   int32_t max_capacity, void* slot_arena,
                                   const void* host_pool, void* stream, moe_cache* out);

moe_status moe_cache_destroy(moe_cache cache);

/* Elastic resize at a safe point (no step in flight: the last routed step has had
 * its FFN issued).  Keeps the new_capacity most recently used experts; survivors in
 * slots >= new_capacity move into the holes below it, in ascending slot order; stamps
 * are kept.  Growing adds empty slots.  new_arena: NULL keeps the current arena
 * (slots >= new_capacity become unused; growing in place is limited to the slots the
 * current arena holds); otherwise a device buffer of new_capacity slots that receives
 * every surviving slot and becomes the arena, after which the old arena may be
 * released once `stream` has passed this call.  Stream ordered.
 * MOE_E_BUSY if a step is in flight, MOE_E_CAPACITY outside
 * [min(max_tokens*top_k, experts), max_capacity] (with prefetch on, the lower end is
 * min(max_tokens*top_k, experts) + experts; see moe_set_prefetch). */
moe_status moe_cache_resize(moe_cache cache, int32_t new_capacity, void* new_arena, void* stream);

/* Router GEMM + top-k + dedup + classification + LRU victims + slot-table update
 * for `layer` on `stream`.  x: [T][hidden] bf16; w_router: [experts][hidden] bf16.
 * topk_idx/topk_w may be NULL.  Writes the step plan into the workspace; the next
 * moe_fill_misses and moe_expert_ffn use it.
 * Steps of up to 8 tokens (decode) run one fused kernel and the weight-streaming FFN;
 * steps of more tokens (prefill chunks) run a tiled router (fp64 accumulation), a
 * one-workgroup plan and a scatter, then the matrix-core FFN; they need bf16 weights,
 * experts <= 256 and top_k <= 16 (MOE_E_INVALID otherwise).
 * MOE_E_INVALID if T > max_tokens, layer out of range, or the previous plan has
 * not had its FFN issued. */
moe_status moe_route_classify(moe_cache cache, int32_t layer, const void* x, int32_t T,
                              const void* w_router, int32_t* topk_idx, float* topk_w,
                              void* stream);

/* Copy the missed blobs of the last plan from the host pool into their slots on
 * `fill_stream`, in `groups` double-buffered groups (groups >= 1; group g holds the
 * misses [g*m/groups, (g+1)*m/groups) of the m misses, ascending expert).  Waits for
 * the plan and for the previous step's FFN (a victim slot may still be read). */
moe_status moe_fill_misses(moe_cache cache, int32_t groups, void* fill_stream);

/* SwiGLU expert FFN and combine for the last plan on `stream`: hit experts first,
 * then each fill group once its copy has landed.  y: [T][hidden] bf16.
 * shared_blob: the layer's shared-expert blob on the GPU, or NULL when
 * has_shared == 0.  MOE_E_INVALID if the fills of the plan were not issued. */
moe_status moe_expert_ffn(moe_cache cache, int32_t layer, const void* x, int32_t T,
                          const void* shared_blob, void* y, void* stream);

/* One whole layer step.  groups >= 1: moe_route_classify + moe_fill_misses(groups) on
 * fill_stream + moe_expert_ffn, hit experts computing while the misses transfer.
 * groups == 0: the same step in stream order on compute_stream alone (route/plan, fill of
 * every miss, one FFN over all the step's experts, combine); fill_stream is ignored.
 * Both give identical results. */
moe_status moe_layer_step(moe_cache cache, int32_t layer, const void* x, int32_t T,
                          const void* w_router, const void* shared_blob, int32_t* topk_idx,
                          float* topk_w, void* y, int32_t groups, void* compute_stream,
                          void* fill_stream);

/* Synchronous copies of the cache state: key_of[capacity], stamp[capacity] (64-bit step
 * of last use, -1 empty), slot_of[layers*experts] (-1 absent), occupancy n and the
 * step counter.  Any pointer may be NULL. */
moe_status moe_cache_snapshot(moe_cache cache, int32_t* key_of, int64_t* stamp,
                              int32_t* slot_of, int32_t* n_occupied, int64_t* step,
                              int32_t* capacity);

/* Sets the global step counter (the stamp the next layer step gives its experts; 64-bit, as
 * are the stamps) of an empty cache, e.g. to carry a session's clock over into a new handle.
 * Synchronous.  MOE_E_INVALID for step < 0 or a cache that holds any expert (their stamps
 * would no longer precede the counter); MOE_E_BUSY while a step is in flight. */
moe_status moe_cache_set_step(moe_cache cache, int64_t step);

/* Prefetch mode for steps of more than 8 tokens (prefill chunks), whose routing union
 * covers nearly every expert (FreeToken paper summary, agihunt.info / arXiv 2608.16157,
 * problem paragraph), streaming experts ahead so that transfers overlap compute
 * ("FreeToken：在消费级 NVIDIA GPU 上进行 MoE 推理", "FreeToken 解决的问题"): each moe_layer_step of layer l (l + 1 < layers) also plans a
 * prefetch step of layer l + 1 - an LRU step whose distinct set is every expert of l + 1,
 * with the slots of step l protected from eviction, taking its own step-counter value - and
 * copies its misses on fill_stream while step l's FFN runs; step l + 1's FFN waits for
 * them.  The caller's next layer step must then be layer l + 1.  Decode steps (T <= 8) never
 * prefetch.  enable: 0 or 1.  MOE_E_INVALID for a handle with max_tokens <= 8; MOE_E_BUSY
 * while a step or a prefetch is in flight (moe_cache_resize is MOE_E_BUSY too until the
 * prefetched layer's step has run); MOE_E_CAPACITY when enabling on a cache of fewer than
 * min(max_tokens*top_k, experts) + experts slots (the step's distinct experts stay protected
 * while every expert of the next layer comes in), and while prefetch is on moe_cache_resize
 * refuses to shrink below that floor. */
moe_status moe_set_prefetch(moe_cache cache, int32_t enable);

/* Hybrid decode: split each decode step's misses between PCIe fills and in-place CPU
 * compute (FreeToken paper summary, agihunt.info / arXiv 2608.16157: problem, execution-layer
 * and last paragraphs - a miss is either moved or computed by the CPU, the split q is a
 * closed form of measured bandwidths derived inside the fused routing kernel; the CPU path
 * exists for bf16 weights only, "FreeToken: az VRAM ile büyük MoE modelleri", "Tuzaklar").
 * b_cpu_mbps: the CPU's expert-weight rate, b_pcie_mbps: the fill rate, both MB/s; a step
 * with m misses (T <= 8) sends the last q of them (ascending expert id) to the CPU, q the
 * integer minimising max((m - q) / b_pcie, q / b_cpu), the smaller on a tie.  CPU misses take
 * no slot, evict nothing and are not stamped.  The route kernel posts them to a pinned
 * mailbox that a server thread of this handle polls; `threads` host threads (the server
 * and its team, which spin while idle) compute them from the host pool, and the combine
 * kernel adds their sum once the host has answered (after 2 s without an answer - see
 * moe_set_hybrid_timeout - it gives up and the next moe_stats / moe_cache_snapshot returns
 * MOE_E_HYBRID).  b_cpu_mbps = 0
 * turns the split off (and stops the threads).  bf16 weights only (MOE_E_INVALID
 * otherwise); MOE_E_BUSY while a step is in flight; MOE_E_NOMEM if the mailbox cannot be
 * pinned.  Choosing the mode is the caller's: the pages switch to the split only when the
 * CPU expert rate is at least 2.0x the offload rate. */
moe_status moe_set_hybrid(moe_cache cache, int32_t b_cpu_mbps, int32_t b_pcie_mbps,
                          int32_t threads);

/* The split the route kernel applies (same code): CPU misses of `misses`, or -1 for a
 * negative argument.  Host arithmetic, for checking the closed form. */
int32_t moe_miss_split(int32_t misses, int32_t b_cpu_mbps, int32_t b_pcie_mbps);

/* Mode choice per weight format ("FreeToken: az VRAM ile büyük MoE modelleri", "Tuzaklar": a
 * start-up probe prints each dtype's CPU expert rate and offload rate against a 2.0x
 * threshold; bf16 at 1.02x offloads, fp8 has no CPU path).  Returns 1 (hybrid decode: split
 * misses with moe_set_hybrid) when wfmt is bf16 - the only format with a CPU expert path - and
 * cpu_gbps >= 2.0 * fill_gbps with both rates positive; 0 (fill every miss) otherwise; -1 for
 * an unknown format or a negative or NaN rate.  Rates in GB/s as measured by the caller
 * (moe_cpu_expert_rate, and the fill rate from moe_profile_read).  Host arithmetic. */
int32_t moe_choose_mode(int32_t wfmt, double cpu_gbps, double fill_gbps);

/* Longest time the combine kernel waits for the host's answer to a hybrid step before it
 * gives up (ERR_HYBRID: moe_stats / moe_cache_snapshot then return MOE_E_HYBRID), measured on
 * the GPU's constant clock; default 2 s.  MOE_E_BUSY while a step is in flight. */
moe_status moe_set_hybrid_timeout(moe_cache cache, int64_t microseconds);

/* Failure-path testing: hold = 1 makes the hybrid server leave requests unanswered (the
 * combine then times out as above); hold = 0 resumes.  MOE_E_INVALID without hybrid decode. */
moe_status moe_hybrid_hold(moe_cache cache, int32_t hold);

/* Host-side counters of the hybrid server since moe_set_hybrid started it: requests
 * answered, CPU experts computed and the seconds spent computing them (zeros when hybrid
 * decode is off).  Any pointer may be NULL. */
moe_status moe_hybrid_read(moe_cache cache, int64_t* requests, int64_t* experts, double* busy_s);

/* The CPU expert FFN of the hybrid path, on host buffers (no GPU involved): for t < T,
 * y[t][:] += w[t] * FFN(x[t]) with the bf16 expert blob `blob` (shape's layout), x [T][hidden]
 * bf16, y [T][hidden] fp32, using `threads` host threads.  T in 1..8.  MOE_E_INVALID for a
 * non-bf16 shape or bad arguments. */
moe_status moe_cpu_expert_ffn(const moe_shape* shape, const void* blob, const void* x, int32_t T,
                              const float* w, float* y, int32_t threads);

/* Measured expert-weight rate of the CPU path: one token through each of the first n_blobs
 * blobs of `pool` (host memory, shape's layout), `reps` times, with `threads` host threads;
 * *gbps = blob bytes processed / wall time / 1e9 (the CPU rate of the mode choice). */
moe_status moe_cpu_expert_rate(const moe_shape* shape, const void* pool, int32_t n_blobs,
                               int32_t threads, int32_t reps, double* gbps);

/* Synchronous copy of the last plan (see moe_plan_host). */
moe_status moe_plan_read(moe_cache cache, moe_plan_host* out);

/* Synchronous read of the device-side counters. */
moe_status moe_stats(moe_cache cache, moe_counters* out);

/* Per-kernel timing of the library's own launches, for measurement.  One launch in every
 * `every` (>= 1) of each kind selected in `mask` is bracketed by a pair of timing events on
 * the stream it runs on (eager calls only: do not enable while a stream is captured).  A
 * timing event costs queue time, so sampling keeps the timed run close to an untimed one.
 * Kinds: route/plan kernel, fill kernel, first FFN stage (the gate/up kernel, or at one token
 * with bf16 weights and no shared expert the fused gate/up + down kernel), second FFN stage
 * (the down kernel with the combine when it follows; after a fused launch the combine alone).
 * moe_profile_enable resets the accumulators (mask 0 switches timing off); moe_profile_read
 * synchronises.  ffn_weight_bytes counts the expert-weight bytes the FFN kernels were given
 * (each processed expert blob once): the algorithmic bytes of the FFN, of which the gate/up
 * kernel reads exactly two thirds in every weight format and the fused kernel all. */
#define MOE_PROF_ROUTE 1
#define MOE_PROF_FILL 2
#define MOE_PROF_GATE_UP 4
#define MOE_PROF_DOWN 8
#define MOE_PROF_ALL 15
typedef struct {
  int64_t launches[4]; /* route, fill, gate/up, down */
  double ms[4];        /* summed event-pair durations, same order */
  int64_t fill_bytes, ffn_weight_bytes;
  int64_t gate_up_timed_bytes; /* algorithmic weight bytes of the timed first-stage FFN
                                  launches: two thirds of each blob for the gate/up kernel,
                                  the whole blob for the fused one-token kernel */
  int64_t fused_timed_bytes;   /* the part of gate_up_timed_bytes read by fused launches */
} moe_profile;

moe_status moe_profile_enable(moe_cache cache, int32_t mask, int32_t every);
moe_status moe_profile_read(moe_cache cache, moe_profile* out);

/* Measurement probes: the ceilings the kernels are judged against, timed with event pairs
 * that the kernel dispatch takes itself (as moe_profile_* does).  Synchronous.
 * moe_probe_stream_read: `reps` launches of a read-only streaming kernel, each reading
 * `bytes_per_launch` bytes of device memory once, in the decode FFN's access pattern (a
 * 256-thread workgroup per contiguous 96 KiB, 24 16-byte loads per thread all in flight;
 * `nontemporal` 1: streaming loads); launch r reads the r-th window of that size (cyclically)
 * within the first `span_bytes` of `buf`, so windows span_bytes/bytes_per_launch launches
 * apart - choose span far above the 256 MB last-level cache - are not cache-resident.  One
 * untimed launch first.  *avg_us = average launch duration.  `sink`: a device word that is
 * written only when a thread's loads fold to a fixed constant (it keeps the loads alive).
 * bytes_per_launch: a multiple of 16, at most span_bytes; buf 16-byte aligned.
 * moe_probe_empty_launch: `reps` launches of an empty kernel of `grid` 256-thread
 * workgroups; *avg_us = average duration (the fixed cost of a launch of that size). */
moe_status moe_probe_stream_read(const void* buf, uint64_t span_bytes, uint64_t bytes_per_launch,
                                 int32_t nontemporal, int32_t reps, void* sink, void* stream,
                                 double* avg_us);
moe_status moe_probe_empty_launch(int32_t grid, int32_t reps, void* stream, double* avg_us);
/* moe_probe_copy: `reps` launches of a plain copy kernel (16-byte loads and stores, every byte
 * read once and written once) of `bytes` from src to dst (device memory, 16-byte aligned, not
 * overlapping; bytes a multiple of 16); *avg_us = average launch duration.  The reference of
 * known read and write bytes for calibrating hardware byte counters. */
moe_status moe_probe_copy(const void* src, void* dst, uint64_t bytes, int32_t reps, void* stream,
                          double* avg_us);

const char* moe_status_string(moe_status s);

/* The hipError_t of the last MOE_E_HIP returned on this handle (0 if none). */
int32_t moe_last_hip_error(moe_cache cache);

#ifdef __cplusplus
}
#endif
#endif /* MOE_OFFLOAD_H */
