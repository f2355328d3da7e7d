/*
 * pmk.h -- C ABI of the persistent decode megakernel library (libpmk.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * One call runs one memory-bound LLM decode step of a whole decoder stack as a
 * single persistent kernel whose tile tasks synchronise through per-tile event
 * counters held in device memory instead of kernel boundaries ("Event Tensor: A
 * Unified Abstraction for Compiling Dynamic Megakernel", summary page, Core
 * method: an event marks that a group of tile tasks finished; notify() is an
 * atomic decrement and wait() spins until the count reaches zero; under static
 * scheduling each compute unit walks a precomputed task queue inside one
 * persistent main loop). Event counts and task queues are rebuilt on the device
 * from (batch, seq_lens) at every call, so batch size and per-request lengths
 * may change between calls with no recompilation or capture (same page, Core
 * method, two kinds of dynamism: shape dynamism).
 *
 * Conventions shared by every entry point:
 *  - All tensor arguments are device pointers (hipMalloc'd or equivalent) and
 *    stay owned by the caller. The library never copies or frees them.
 *  - Weights are row-major [out][in] in the model dtype (float32 or bfloat16
 *    as raw 16-bit patterns), or, for bfloat16 with weight_layout =
 *    PMK_TILES, in the tile layout that pmk_pack_weights writes; RMSNorm gains
 *    are always float32.
 *  - Calls are stream-ordered and asynchronous; `stream` is a hipStream_t
 *    passed as void* (NULL = the null stream). One handle serves one stream at a
 *    time: calls on one handle must not overlap.
 *  - Return value: 0 (PMK_OK) or a PMK_ERR_* code; no exception crosses the ABI.
 *    Errors the device detects (a request length out of range, an event wait
 *    that exceeded the watchdog) are recorded in a device error word. The
 *    device also copies it into a pinned host mirror, so once the step that
 *    hit the error has finished on the device, every later decode_step /
 *    moe_layer_step on the handle returns that code without launching, until
 *    pmk_get_device_error() has read and cleared it. A call made while that
 *    step is still running cannot know yet: it returns PMK_OK, and the device
 *    skips its step (the error word stays set).
 */
#ifndef PMK_H
#define PMK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PMK_ABI_VERSION 1

enum pmk_status {
  PMK_OK = 0,
  PMK_ERR_ARG = 1,          /* invalid argument (dims, null pointer, batch out of range) */
  PMK_ERR_OOM = 2,          /* device allocation failed */
  PMK_ERR_DEVICE = 3,       /* a HIP call failed (launch, copy, event) */
  PMK_ERR_TIMEOUT = 4,      /* device: an event wait exceeded the watchdog; the step was abandoned */
  PMK_ERR_SEQ = 5,          /* device: seq_lens[b] < 0 or >= max_seq; the step did not run */
  PMK_ERR_UNSUPPORTED = 6,  /* a shape this build does not implement (see pmk_strerror) */
  PMK_ERR_SCRATCH = 7       /* decode_step_static: the model's workspace exceeds its 64 MiB static scratch */
};

enum pmk_dtype { PMK_F32 = 0, PMK_BF16 = 1 };

/* Storage of the weight matrices: row-major, or 16-row tiles (see
 * pmk_pack_weights). The arithmetic, and so every output bit, is the same. */
enum pmk_weight_layout { PMK_ROWS = 0, PMK_TILES = 1 };

/* Model description. Dense stack when n_experts == 0, MoE layers otherwise. */
typedef struct pmk_model_desc {
  int32_t abi_version;       /* must be PMK_ABI_VERSION */
  int32_t dtype;             /* pmk_dtype: weights and KV cache */
  int32_t n_layers;
  int32_t hidden;            /* H, multiple of 8 */
  int32_t n_q_heads;         /* Hq, multiple of n_kv_heads */
  int32_t n_kv_heads;        /* Hkv */
  int32_t head_dim;          /* d; d * sizeof(dtype) must be 256 bytes (d = 128 bf16, d = 64 f32) */
  int32_t ffn_dim;           /* F (dense), multiple of 8 */
  int32_t n_experts;         /* E (0 = dense) */
  int32_t top_k;             /* k <= 8 */
  int32_t expert_ffn_dim;    /* Fe, multiple of 8 */
  int32_t max_batch;         /* largest batch (or MoE token count) a call may pass */
  int32_t max_seq;           /* KV cache slots per request; seq_lens[b] < max_seq */
  float rms_eps;             /* e.g. 1e-5 */
  float rope_theta;          /* e.g. 10000 */
  int32_t watchdog_ms;       /* event-wait limit before the step is abandoned; 0 = 2000 */
  int32_t weight_layout;     /* pmk_weight_layout; PMK_TILES: bfloat16 only, with H, Hq d, F and Fe multiples
                                of 32 and (Hq + 2 Hkv) d and E multiples of 16 (else PMK_ERR_UNSUPPORTED) */
  int32_t reserved[5];       /* zero */
} pmk_model_desc;

/* One layer's weights (device pointers, caller-owned). Dense layers use
 * w_gate/w_up/w_down; MoE layers use w_router and the w_exp_* tensors. */
typedef struct pmk_layer_weights {
  const float* attn_norm;    /* [H] */
  const void* w_qkv;         /* [(Hq + 2 Hkv) d][H]: the q rows, then k, then v */
  const void* w_o;           /* [H][Hq d] */
  const float* ffn_norm;     /* [H] */
  const void* w_gate;        /* [F][H] */
  const void* w_up;          /* [F][H] */
  const void* w_down;        /* [H][F] */
  const void* w_router;      /* [E][H] */
  const void* w_exp_gate;    /* [E][Fe][H] */
  const void* w_exp_up;      /* [E][Fe][H] */
  const void* w_exp_down;    /* [E][H][Fe] */
} pmk_layer_weights;

typedef struct pmk_weights {
  int32_t n_layers;                  /* must equal desc->n_layers */
  const pmk_layer_weights* layers;   /* host array of n_layers entries (copied at init) */
} pmk_weights;

/* Optional routing outputs of moe_layer_step (device pointers, caller-owned;
 * each may be NULL). All describe the last MoE layer of the call. */
typedef struct pmk_routing {
  int32_t* topk_idx;        /* [T][k]   experts by (logit desc, index asc) */
  float* topk_w;            /* [T][k]   softmax over the k selected logits */
  float* router_logits;     /* [T][E]   float32 logits the selection was taken on */
  int32_t* exp_indptr;      /* [E+1]    prefix sum of per-expert routed rows; last = T k */
  int32_t* tile_indptr;     /* [E+1]    prefix sum of ceil(count_e / moe_bm) row tiles */
  int32_t* sorted_tok;      /* [T k]    routed (token) ordered by expert, then token */
  int32_t* sorted_slot;     /* [T k]    the matching top-k slot j */
} pmk_routing;

typedef struct pmk_info {
  int32_t grid;              /* persistent workgroups (one per compute unit) */
  int32_t block;             /* threads per workgroup */
  int32_t lds_bytes;         /* dynamic LDS per workgroup */
  int32_t moe_bm;            /* row-tile size of the grouped GEMM (tile_indptr granularity) */
  int32_t attn_chunk;        /* KV positions per attention tile task */
  int32_t max_queue;         /* task-queue capacity per workgroup per layer */
  int64_t workspace_bytes;   /* device memory owned by the handle */
  int32_t arch;              /* 950 for gfx950 */
  int32_t reserved[7];
} pmk_info;

typedef struct pmk_handle pmk_handle;

/* Create a handle (Event Tensor summary, Core method, ETC compiler and
 * scheduling: the megakernel is compiled ahead of time and its runtime needs
 * only the counter tensors and the scheduler queue; the two kinds of dynamism
 * are handled at run time from symbolic batch/length dimensions). Validates
 * desc and every weight pointer, keeps the weight pointers (no copy), builds
 * the RoPE cos/sin table on the host in double and uploads it as float32,
 * allocates the workspace (activations, attention partials, event counters,
 * task queues, MoE routing arrays, error word and its pinned host mirror) for
 * max_batch and max_seq, and sizes the persistent grid to the device's compute
 * units (one workgroup per compute unit, as the per-SM queues of static
 * scheduling assume). The handle is owned by the caller until
 * decode_layer_destroy. Errors: PMK_ERR_ARG (null pointer, inconsistent
 * dims), PMK_ERR_UNSUPPORTED, PMK_ERR_OOM, PMK_ERR_DEVICE. */
int decode_layer_init(const pmk_model_desc* desc, const pmk_weights* weights, pmk_handle** out);

/* One decode step of the whole stack for `batch` requests (Event Tensor
 * summary, Experiments: the end-to-end decode step covers attention, RoPE, KV
 * cache, norm and MLP; Core method, ETC compiler and scheduling: static
 * scheduling with a per-compute-unit queue and a persistent main loop).
 *   hidden    float32 [batch][H], in/out: each request's input hidden state in,
 *             the stack's output out (no final norm, no vocabulary head).
 *   kv_cache  model dtype [L][2][max_batch][Hkv][max_seq][d] (K block, then V):
 *             slots 0..seq_lens[b]-1 hold request b's cached, already-rotated
 *             keys and values. The step writes the new K/V at slot seq_lens[b]
 *             (rounded to the cache dtype, nearest even) and attends over
 *             seq_lens[b] + 1 entries.
 *   seq_lens  int32 [batch], device: cached length of each request before the
 *             step. Not modified: the caller advances it.
 * Two launches (a queue/event prologue and the persistent kernel). Dense
 * handles only; a MoE handle runs the same step with routed experts.
 * Errors: PMK_ERR_ARG (batch outside [1, max_batch], null pointer), a pending
 * device error from an earlier step that has reached the host mirror
 * (PMK_ERR_SEQ, PMK_ERR_TIMEOUT; nothing is launched), PMK_ERR_DEVICE. */
int decode_step(pmk_handle* h, float* hidden, void* kv_cache, const int32_t* seq_lens, int32_t batch, void* stream);

/* decode_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. One
 * call does what decode_layer_init and decode_step do, with no handle: the
 * workspace (counters, queues, activations, the RoPE table, the layer-pointer
 * table) lives in a file-scope device array of 64 MiB that each GPU the
 * library runs on holds until the process ends. The call makes no hipMalloc,
 * hipFree or other allocation; it launches a clearing kernel, the RoPE-table
 * kernel, a host-to-device copy of weights->layers, the prologue and the
 * persistent kernel (fused schedule, per-tile events, the descriptor's
 * watchdog), all on `stream`.
 *   desc, weights  as for decode_layer_init; dense stacks only (n_experts = 0,
 *                  else PMK_ERR_UNSUPPORTED). weights->layers must stay
 *                  valid until the copy has run on the stream.
 *   hidden, kv_cache, seq_lens, batch, stream  as for decode_step.
 *   status   nullable device int32: set to 0 when the step starts and to the
 *            device error code (PMK_ERR_SEQ, PMK_ERR_TIMEOUT) if the step hits
 *            one; there is no handle to hold it for a later call.
 * Every call on a GPU shares that GPU's scratch, which keeps the last call's
 * contents (each call clears what must start at zero): calls that overlap on
 * one GPU, on any streams, race. Errors: PMK_ERR_ARG, PMK_ERR_UNSUPPORTED,
 * PMK_ERR_SCRATCH (the workspace for desc is larger than the scratch: fewer
 * layers, a smaller max_batch or max_seq), PMK_ERR_DEVICE. */
int decode_step_static(const pmk_model_desc* desc, const pmk_weights* weights, float* hidden, void* kv_cache,
                       const int32_t* seq_lens, int32_t batch, int32_t* status, void* stream);

/* One step of a stack of MoE decoder layers for `tokens` tokens, each its own
 * request (Event Tensor summary, Key observations, observation 2: attention,
 * then TopK, then grouping, then the grouped GEMM; Core method, two kinds of
 * dynamism: topk decides which expert's event each grouping task updates, each
 * expert counter starts at its routed-token count, and the exp_indptr prefix
 * sum decides which grouped-GEMM tiles an expert triggers). Arguments as for
 * decode_step; `routing` (nullable) receives the last layer's routing.
 * Requires a handle made with n_experts > 0. Errors as for decode_step. */
int moe_layer_step(pmk_handle* h, float* hidden, void* kv_cache, const int32_t* seq_lens, int32_t tokens,
                   const pmk_routing* routing, void* stream);

/* Synchronise the device, free the workspace (counter tensors, queues,
 * activations), the host error mirror and the handle (the runtime state that
 * decode_layer_init created; Event Tensor summary, Core method, ETC compiler
 * and scheduling). The caller's weights, caches and hidden states are not
 * touched. NULL is a no-op. Returns PMK_ERR_DEVICE if the synchronisation
 * failed (everything is freed anyway). */
int decode_layer_destroy(pmk_handle* h);

/* Static description of a status code. */
const char* pmk_strerror(int status);

/* Synchronise the handle's last stream and return the device error word
 * (PMK_OK, PMK_ERR_TIMEOUT, PMK_ERR_SEQ, or PMK_ERR_ARG for a task queue
 * that outgrew its capacity), then clear it and its host mirror, so later
 * calls run again. The watchdog behind PMK_ERR_TIMEOUT answers the pages'
 * open point on deadlocks inside a persistent megakernel (Event Tensor
 * summary, Critical analysis, systemic gaps: observability and debugging):
 * a wait that never ends becomes an error, and every workgroup leaves the
 * step. Errors: PMK_ERR_ARG (null handle), PMK_ERR_DEVICE. */
int pmk_get_device_error(pmk_handle* h);

/* Launch configuration and sizes of a handle: the persistent grid (one
 * workgroup per compute unit, each with its own static task queue; Event
 * Tensor summary, Core method, ETC compiler and scheduling) and the row-tile
 * size moe_bm of the grouped GEMM, which sets the granularity of tile_indptr
 * (same page, Core method, two kinds of dynamism: the per-expert prefix sum
 * over grouped-GEMM tiles decides which tiles an expert triggers).
 * `out` is caller-owned. Errors: PMK_ERR_ARG (null pointer). */
int pmk_query(const pmk_handle* h, pmk_info* out);

/* Per-launch timing of the persistent kernel with HIP events recorded on the
 * call's stream around that launch only. enable != 0 starts a new window;
 * pmk_timing_read synchronises, returns the summed milliseconds and the number
 * of timed launches since the window started. */
int pmk_timing_enable(pmk_handle* h, int enable);
int pmk_timing_read(pmk_handle* h, double* total_ms, int32_t* launches);

/* Schedule of a step (an ablation of the fused design; Event Tensor summary,
 * Evaluation: the gain of fine-grained pipelining over kernel boundaries):
 *   PMK_SCHED_FUSED      one persistent launch per step, stages chained by
 *                        events (the default);
 *   PMK_SCHED_PER_LAYER  one launch of the same persistent kernel per layer:
 *                        events inside a layer, a kernel boundary between layers;
 *   PMK_SCHED_PER_STAGE  one launch per stage of each layer (QKV, attention, O,
 *                        gate/up, down; MoE: router, routing, expert gate/up,
 *                        expert down, combine): every grid-wide event becomes
 *                        a kernel boundary;
 *   PMK_SCHED_BARRIER    one persistent launch per step with a grid-wide
 *                        barrier after every stage: no workgroup starts a task
 *                        of the next stage (nor its weight prefetch) before
 *                        every workgroup has finished the current one (the
 *                        pages' unfused megakernel).
 *   PMK_SCHED_PER_OP     one launch per operator of each layer, ten per layer
 *                        (320 per token for 32 layers, the unfused GPU
 *                        picture of the "Dataflow Is All You Need" summary,
 *                        Key observations, observation 1: K1-K10 per decoder
 *                        layer): RMSNorm, QKV projection, RoPE, KV append,
 *                        attention partials, partial merge, O projection +
 *                        residual, RMSNorm, gate/up + SwiGLU, down +
 *                        residual. The norms, RoPE, append and merge that the
 *                        other modes fuse into the projections run as ops of
 *                        their own (the projections then read the normalised
 *                        rows from memory). Dense handles only.
 * The same task code and results in every mode (per-step prologue included;
 * the per-op mode adds the separate norm, RoPE, append and merge tasks);
 * timing (pmk_timing_*) covers all persistent launches of a step. Applies to
 * later calls. Errors: PMK_ERR_ARG (null handle, unknown mode),
 * PMK_ERR_UNSUPPORTED (PMK_SCHED_PER_OP on a MoE handle). */
#define PMK_SCHED_FUSED 0
#define PMK_SCHED_PER_LAYER 1
#define PMK_SCHED_PER_STAGE 2
#define PMK_SCHED_BARRIER 3
#define PMK_SCHED_PER_OP 4
int pmk_set_schedule(pmk_handle* h, int32_t mode);

/* How the grouped expert GEMM tasks of a MoE layer reach workgroups (Event
 * Tensor summary, Core method: static and dynamic scheduling):
 *   PMK_MOE_STATIC   each workgroup runs a fixed share of the gate/up tasks,
 *                    then of the down tasks, each down task waiting on its
 *                    expert's counter (the default);
 *   PMK_MOE_DYNAMIC  workgroups pop task indices from one counter per layer:
 *                    first the gate/up tasks, then down tasks from a ready
 *                    queue that the last gate/up task of each expert fills
 *                    with that expert's down tasks when the expert's counter
 *                    reaches zero.
 *   PMK_MOE_DYNAMIC_XCD  the same tasks and ready queue, popped hierarchically
 *                    (the pages leave the GPU scheduler's hierarchy as future
 *                    work; Event Tensor summary, Limitations and future
 *                    work): one counter per XCD, each over the task indices
 *                    congruent to that XCD's id mod 8, so a workgroup's pops
 *                    stay on its own XCD's counter; a workgroup whose XCD
 *                    counter has run out steals from the others.
 * Same results in every mode. Ignored by dense handles; applies to later
 * calls. Errors: PMK_ERR_ARG (null handle, unknown mode). */
#define PMK_MOE_STATIC 0
#define PMK_MOE_DYNAMIC 1
#define PMK_MOE_DYNAMIC_XCD 2
int pmk_set_moe_scheduler(pmk_handle* h, int32_t mode);

/* The event-wait limit of later calls, in microseconds (100 ticks of the
 * device's 100 MHz clock each); 0 restores the limit set at init
 * (desc->watchdog_ms). A wait that exceeds it abandons the step: the device
 * error word takes PMK_ERR_TIMEOUT, the abort flag makes every workgroup leave
 * the step, and later steps are skipped until pmk_get_device_error has read
 * (and cleared) the word; the next step then re-arms every counter. For
 * callers with a latency budget and for tests of that path.
 * Errors: PMK_ERR_ARG (null handle, negative limit). */
int pmk_set_watchdog_us(pmk_handle* h, int32_t us);

/* Granularity of the dense chain's events (Event Tensor summary, Core method:
 * Event Tensor abstraction; Problem and motivation: a kernel boundary makes
 * every consumer wait for the whole producer stage although it often needs
 * only part of it):
 *   PMK_EVENTS_TILE   per tile: the QKV tiles of each KV group and batch
 *                     block, the attention of each KV group and block, and
 *                     the O, gate/up and down tiles of each 16-row block
 *                     (batches beyond 16 rows) each have an event; attention
 *                     (b, g) waits on group g's QKV tiles only, an O task on
 *                     the attention of the groups its K slice reads, a
 *                     block's stages on that block's events;
 *   PMK_EVENTS_GROUP  (the default) the same up to 16 rows; beyond, one batch
 *                     block (per-block events measured 1.6 % slower at 64
 *                     rows: the queues are static, so a block's tasks cannot
 *                     overtake another's anyway);
 *   PMK_EVENTS_STAGE  one event per stage: every attention task waits on all
 *                     QKV tiles, every O task on all attention.
 * Same results in every mode (an ablation of the subset waits). Applies to
 * later calls. Errors: PMK_ERR_ARG (null handle, unknown mode). */
#define PMK_EVENTS_TILE 0
#define PMK_EVENTS_GROUP 1
#define PMK_EVENTS_STAGE 2
int pmk_set_event_granularity(pmk_handle* h, int32_t mode);

/* Writes a copy of the bfloat16 matrix src [rows][cols] (row-major) into dst
 * in the tile layout that a handle with weight_layout = PMK_TILES reads. The
 * decode step reads each weight matrix once as a stream of 16-row groups
 * (the weight-streaming tile tasks of the persistent megakernel, Event Tensor
 * summary page, Core method). The tile layout cuts the matrix into 16-row x
 * 32-column tiles and stores them one after another, row group major, each
 * tile row-major (1 KiB), so that every wave-wide 16-byte-per-lane load of a
 * row group's k-step reads one contiguous 1 KiB block: element (r, c) is at
 *   ((r / 16) * (cols / 32) + c / 32) * 512 + (r % 16) * 32 + c % 32
 * of dst. A stack of matrices with the same cols (the experts of a layer,
 * [E][rows][cols]) packs as one matrix of E rows rows. dst has the same size
 * as src (rows * cols * 2 bytes) and is caller-owned; the copy is ordered on
 * `stream` (hipStream_t as void*, NULL = null stream) and src may be freed
 * once it has run.
 * Errors: PMK_ERR_ARG (null or unaligned (16-byte) pointer, rows not a
 * positive multiple of 16, cols not a positive multiple of 32, overlapping
 * src and dst), PMK_ERR_DEVICE (launch failed). */
int pmk_pack_weights(const void* src, void* dst, int64_t rows, int64_t cols, void* stream);

/* Task trace for profiling the schedule. `buf` is a caller-owned device buffer
 * of grid * entries_per_wg * 8 uint32 (grid from pmk_query); NULL detaches.
 * While attached, every call records, per workgroup w, at
 * buf[(w * entries_per_wg + i) * 8 + 0..7] for i >= 1:
 *   [0] task type | layer << 8 | (first task coordinate & 0xffff) << 16
 *   [1] low 32 bits of the 100 MHz device clock when the task was taken
 *   [2] the clock once its input event was satisfied
 *   [3] the clock once its inputs were staged in LDS
 *   [4] the clock once wave 0 had streamed its weights (attention: once
 *       wave 0 had gone through its KV positions)
 *   [5] the clock once the partial sums were reduced (attention: once every
 *       wave had)
 *   [6] the clock once the epilogue had stored its outputs (attention: once
 *       its outputs were issued)
 *   [7] the clock when it had finished and notified
 * (a phase the task does not have repeats the previous clock), and at entry
 * i = 0, element [0], the number of tasks recorded (tasks beyond
 * entries_per_wg - 1 are dropped). Each call overwrites the buffer.
 * Errors: PMK_ERR_ARG (null handle, entries_per_wg < 2 with a buffer). */
int pmk_trace_attach(pmk_handle* h, uint32_t* buf, int32_t entries_per_wg);

/* Streaming-read probe: the HBM read bandwidth that a kernel doing nothing
 * but reading reaches on this device, as the measured reference next to the
 * nominal peak for the decode step's bandwidth roofline (the pages measure
 * decode against the memory roofline: "Dataflow Is All You Need" summary
 * page, Experiments and results, 45-78 % of roofline on SN40; Problem and
 * motivation, ~21 % of HBM bandwidth used by GPU decode on H100). One
 * workgroup per compute unit, 8 waves,
 * 16 loads of 16 bytes per lane in flight (the decode GEMV engine's ring),
 * each wave streaming 16 KiB blocks of `buf` round-robin:
 *   pattern 0: contiguous 1 KiB per wave-wide load, non-temporal (the tile
 *              weight layout);
 *   pattern 1: 16 rows x 64 bytes per wave-wide load over rows of 8 KiB,
 *              through the caches (row-major bfloat16 weights with 4096
 *              columns).
 * Runs `reps` launches on `stream`, each timed with HIP events, and writes the
 * fastest in milliseconds to *ms_out (bandwidth = bytes / ms). `buf`: device,
 * 256-byte aligned, `bytes` a positive multiple of 1 MiB, only read; `sink`:
 * a device int that the probe may increment (it keeps the loads from being
 * optimised away). Synchronises the stream. Errors: PMK_ERR_ARG, PMK_ERR_DEVICE. */
int pmk_stream_probe(const void* buf, int64_t bytes, int32_t pattern, int32_t reps, int* sink, void* stream,
                     double* ms_out);

/* Cross-XCD message-passing litmus of the persistent kernel's synchronisation
 * scheme (the pages leave the deadlock and race debugging of event-driven
 * kernels open; Event Tensor summary, Critical analysis), made from the same
 * device primitives: a writer's device-coherent stores, a drain of its stores
 * and a relaxed agent-scope atomic decrement; readers on the eight XCDs that
 * spin on the counter (watchdog-bounded) and then read a block written once
 * through the caches, as the kernels stage activations, and a block rewritten
 * every round device-coherently, as they read split-K records. `rounds`
 * rounds, one writer each (workgroup round mod grid), eight readers each.
 *   work    device buffer, 256-byte aligned, of at least
 *           rounds * 4224 + 4352 bytes (blocks, counters, error word);
 *   result  device int32[8]: [0] the first round a reader saw a stale value
 *           (-1: none; the run stops there), [1] its element, [2] the value
 *           read, [3] the value written, [4] 0: the written-once block read
 *           through the caches, 1: the rewritten block read coherently;
 *           [5] 1 if a wait timed out (2 s); [6] rounds x readers checked;
 *           [7] stale values of the rewritten block read through the caches
 *           (counted, not a failure: the access the kernels avoid).
 * Asynchronous on `stream` (a cooperative launch of one workgroup per compute
 * unit). Errors: PMK_ERR_ARG, PMK_ERR_DEVICE. */
int pmk_event_litmus(void* work, int64_t bytes, int32_t rounds, int32_t* result, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PMK_H */
