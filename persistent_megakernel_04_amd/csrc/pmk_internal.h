// pmk_internal.h -- definitions shared by the host runtime (pmk_api.hip) and the
// device code (pmk_kernels.hip) of libpmk. Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pmk.h"

namespace pmk {

constexpr int kBlock = 512;              // threads per persistent workgroup: 8 wave64
constexpr int kWaves = kBlock / 64;
constexpr int kSubs = 8;                 // sub-counters of a hierarchical event
constexpr int kCtr = 16;                 // ints between two counters (64 bytes)
constexpr int kXcd = 8;                  // XCDs of the device (the per-XCD task queues of the dynamic MoE scheduler)
constexpr int kMq = 2 + kXcd;            // per layer: the central pop counter, the push counter, a pop counter per XCD
constexpr int kEvInts = (1 + kSubs) * kCtr;
constexpr int kMinChunk = 64;            // smallest attention chunk (KV positions per tile task)
constexpr int kPieceCost = 320;          // streamed attention: a piece's fixed cost in KV positions
constexpr int kMaxChunk = 256;           // largest attention chunk
constexpr int kMergeChunks = 8;          // chunks per request at most when the O-projection merges the partials
constexpr int kMergeFloats = 4096;       // O-projection inputs (batch rows x Hq d) that one merging pass stages
constexpr int kMoeBM = 16;               // token rows per grouped-GEMM tile (one MFMA row block)
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 512;
constexpr int kMaxNb = 16;               // batch rows per GEMV pass (MFMA M)
constexpr int kMaxBatchAll = 1024;       // largest max_batch (prologue LDS)
constexpr int kMaxHkv = 128;             // KV heads at most (the prologue's per-group tile counts)
constexpr int kMaxStages = 8;            // stages of a layer (MoE: QKV, attention, O, router, route, gate/up, down, combine)

// LDS layout (bytes): [xy: a GEMV pass's staged inputs (xs), then its outputs
// (ys) | red: cross-wave partial sums | misc]. Attention and routing use the xy
// region as scratch.
constexpr int kXyBytes = 147968;
constexpr int kRedBytes = 8192;
constexpr int kMiscBytes = 2048;
constexpr int kRopeBytes = 4096;         // the QKV tile's rotation rows, kept across the layers of a launch
constexpr int kLdsBytes = kXyBytes + kRedBytes + kMiscBytes + kRopeBytes;
constexpr int kXsBytes = 131584;         // staged inputs of a pass at most (the rest of xy holds ys)
constexpr int kYsFloats = 2048;          // outputs of a pass whose residual is loaded ahead (O, down)
constexpr int kRingK = 16;               // weight loads in flight per wave

// A dense GEMV stage's work split for one step: `ks` slices of the depth K
// times `tiles` row tiles, one task each. With ks > 1 every task stores its
// partial sums and the last task of a row tile to finish adds the slices (in
// slice order) and runs the stage's epilogue. Chosen so that a task's staged
// input rows (nb rows of its slice, 4 bytes per element: bfloat16 hi + lo, or
// float) and its outputs fit the xy region; ks = 1 whenever the whole depth
// fits, always so for a single row. kstep: the k elements of one weight load
// step (32 bfloat16 or 16 float); xpad: LDS row padding (elements). Slices
// are whole ring lengths (16 steps) but the last.
constexpr int kMaxKs = 8;                // K slices of a split stage at most
struct StageGeo {
  int ks, tiles, kr;    // kr: slice length (elements); the last slice ends at K
  int blk;              // > 1: the batch in blocks of 16 rows, each (tile, slice, block) a task of its own
};
__host__ __device__ inline StageGeo stage_geo(int K, int units, int urows, int nb, int avail, int kstep, int xpad) {
  const int grain = kRingK * kstep;
  for (int ks = 1;; ++ks) {
    int kr = (K + ks - 1) / ks;
    kr = (kr + grain - 1) / grain * grain;
    if (kr > K) kr = K;
    const int kse = (K + kr - 1) / kr;
    int tiles = avail / kse;
    if (tiles > units) tiles = units;
    if (tiles < 1) tiles = 1;
    const int rows = (units + tiles - 1) / tiles * urows;
    const long xs = (long)nb * ((kr + kstep - 1) / kstep * kstep + xpad) * 4;
    const long need = (xs + 15) / 16 * 16 + (long)rows * nb * 4;
    if (kse > kMaxKs) return StageGeo{0, 0, 0, 1};   // no split fits: passes over the batch instead
    if (need <= kXyBytes || kr <= grain) return StageGeo{kse, tiles, kr, 1};
  }
}

// The split of a dense stage for a batch of B rows on `avail` workgroups. Up
// to 16 rows: stage_geo for those rows. Beyond, the batch runs in blocks of
// 16 rows, each (row tile, K slice, block) a task of its own (blk > 1), with
// row tiles sized for about `mult` tasks per workgroup over all the blocks
// (tiles x slices ~ avail mult / blocks): the smallest mult of 1, 2, 4, ...
// whose tile outputs and 16-row input slices fit the LDS. Each tile's weights
// are still read once per block (by workgroups of one XCD, through its L2),
// but each block's inputs are staged by that many times fewer tiles, and a
// workgroup runs that many times fewer tasks, each with its own wait,
// staging, stores and notify. Where no K split fits: passes of rows over the
// whole depth (slice 1, one block).
// Whether a pass of split g (nb staged rows of its K slice, then its tile's
// outputs for them) fits the LDS region that holds it.
__host__ __device__ inline bool stage_fits(const StageGeo& g, int units, int urows, int nb, int kstep, int xpad) {
  const long xs = (long)nb * ((g.kr + kstep - 1) / kstep * kstep + xpad) * 4;
  const long rows = (long)(units + g.tiles - 1) / g.tiles * urows;
  return (xs + 15) / 16 * 16 + rows * nb * 4 <= kXyBytes;
}
__host__ __device__ inline StageGeo stage_split(int K, int units, int urows, int B, int avail, int kstep, int xpad) {
  StageGeo g{0, 0, 0, 1};
  if (B <= kMaxNb) {
    g = stage_geo(K, units, urows, B, avail, kstep, xpad);
  } else {
    const int nbk = (B + kMaxNb - 1) / kMaxNb;
    for (int mult = 1;; mult *= 2) {
      if (mult >= nbk) {   // one tile set per block: the split of 16 rows on the whole share
        g = stage_geo(K, units, urows, kMaxNb, avail, kstep, xpad);
        break;
      }
      const long av = (long)avail * mult / nbk;
      g = stage_geo(K, units, urows, kMaxNb, av > 1 ? (int)av : 1, kstep, xpad);
      // (stage_geo stops at its shortest slice whether or not the tile fits)
      if (g.ks && stage_fits(g, units, urows, kMaxNb, kstep, xpad)) break;
    }
    if (g.ks) g.blk = nbk;
  }
  if (g.ks == 0) g = StageGeo{1, avail < units ? avail : units, K, 1};
  return g;
}

// Split-K record layout of a dense stage, as the persistent kernel addresses
// it: task (row tile t, slice s, batch block k) stores its slice's partial sums
// (the tile's rows x nb, then nb sums of squares) at record
// ((k tiles + t) ks + s), records `stride` floats apart, a whole number of
// 16-byte units sized for the stage's largest tile. nb: rows of the block (16
// for every block of a batch beyond 16 rows).
__host__ __device__ inline int kpart_stride(int units, int urows, int tiles, int nb) {
  return ((units + tiles - 1) / tiles * urows * nb + 16 + 3) & ~3;
}

// Floats of split-K records a stage of depth K needs at most, over every
// batch (stage_split: nb = min(batch, 16) rows per block, its blocks) and
// every grid share the prologue may give the stage (the whole grid, or the
// grid less the workgroups of up to a quarter of it that take attention tasks
// of their own: avail in [grid - grid / 4, grid] for QKV and O).
__host__ __device__ inline long kpart_need(int K, int units, int urows, int max_batch, int grid, bool attn_share,
                                           int kstep, int xpad) {
  long need = 0;
  const int lo = attn_share ? grid - grid / 4 : grid;
  // every batch up to 16, then one batch per count of 16-row blocks (the split
  // depends on the block count alone)
  for (int B = 1;; B = B < kMaxNb ? B + 1 : B + kMaxNb) {
    const int Bc = B < max_batch ? B : max_batch;
    for (int avail = lo; avail <= grid; ++avail) {
      const StageGeo g = stage_split(K, units, urows, Bc, avail, kstep, xpad);
      if (g.ks <= 1) continue;
      const long ext = (long)g.blk * g.tiles * g.ks * kpart_stride(units, urows, g.tiles, Bc < kMaxNb ? Bc : kMaxNb);
      if (ext > need) need = ext;
    }
    if (Bc >= max_batch) break;
  }
  return need;
}

// Task types of the per-workgroup queue (one layer's worth; replayed per layer).
enum TaskType : int {
  T_QKV = 1,      // y = tile: RMSNorm1 + QKV rows + RoPE + KV append
  T_ATTN = 2,     // y = b, z = kv group g, w = chunk: split-K GQA attention (+ merge by the last chunk)
  T_O = 3,        // y = tile: O-projection rows + residual
  T_GU = 4,       // y = tile: RMSNorm2 + gate/up rows + SwiGLU
  T_DOWN = 5,     // y = tile: down-projection rows + residual (dense layer output)
  T_ROUTER = 6,   // y = row tile, z = token block: RMSNorm2 + router logits
  T_ROUTE = 7,    // top-k, gates, expert grouping, expert-event arming (one workgroup)
  T_MGU = 8,      // this workgroup's share of the grouped gate/up GEMM tasks
  T_MDOWN = 9,    // this workgroup's share of the grouped down GEMM tasks
  T_COMBINE = 10, // this workgroup's share of the per-token gated combine (MoE layer output)
  T_ATTS = 11,    // x >> 8: piece | pieces << 12, y = b | g << 16, z..w: positions: streamed attention piece
  // the per-op schedule's separate operators (each a grid-stride share of its op per workgroup)
  T_NORM1 = 12,   // u = RMSNorm(layer input; attn_norm)
  T_NORM2 = 13,   // u = RMSNorm(h1; ffn_norm)
  T_ROPE = 14,    // rotate q and k in place at each request's position
  T_APPEND = 15,  // k, v rounded into the cache at each request's slot
  T_MERGE = 16    // merge the attention chunks' partials of every (request, KV head) into o
};

// Events of one layer. Each event is a block of kEvInts ints: [0] is the
// counter that waiters spin on; [1 + x] (x < kSubs) are sub-counters for
// hierarchical notification (the last notifier of a sub-counter decrements
// [0]). Flat events are decremented at [0] directly.
enum EventId : int {
  EV_QKV = 0, EV_ATTN, EV_O, EV_GU, EV_DOWN, EV_ROUTER, EV_ROUTE, EV_MDOWN, EV_COUNT
};

struct LayerPtrs {
  const float* attn_norm;
  const void* w_qkv;
  const void* w_o;
  const float* ffn_norm;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* w_router;
  const void* w_exp_gate;
  const void* w_exp_up;
  const void* w_exp_down;
};

struct Dims {
  int L, H, Hq, Hkv, d, F, E, k, Fe;
  int max_batch, max_seq, max_chunks;
  float eps;
  int grid;
  int qkv_units;                     // (Hq + 2 Hkv) d / 2 rotation pairs
  int qkv_tiles, o_tiles, gu_tiles, down_tiles, router_tiles;
  int max_queue;
  int moe;                           // 1 = MoE layers
  int kstep, xpad;                   // GEMV: k elements per weight load step, LDS row padding (by dtype)
  int attn_mm;                       // 1: matrix-core attention (bfloat16 KV, head_dim 128, <= 8 heads per KV head)
  int merge_b;                       // largest batch whose attention partials the O-projection merges (0: none)
  int max_tiles;                     // MoE: bound on grouped-GEMM row tiles
  int tctr_stride;                   // split-K tile counters per stage: grid x batch blocks
  int max_down;                      // MoE: bound on grouped down tasks (row tiles x H slices)
  int wtiles;                        // 1: bfloat16 weights in the tile layout (pmk_pack_weights)
  long kpart_off[5];                 // split-K records: first float of each dense stage's region; [4] = total
};

// Device workspace (one allocation, carved by the host).
struct Workspace {
  // per-layer activations (each written once per step; see qkv_of in the kernels)
  float* qkv;          // [L][max_batch][(Hq + 2 Hkv) d]   rotated q, k; v
  float* o;            // [L][max_batch][Hq d]             merged attention output
  float* h1;           // [L][max_batch][H]                residual after attention
  float* act;          // [L][max_batch][F]                SwiGLU output (dense)
  float* hid;          // [L - 1][max_batch][H]            layer outputs feeding the next layer
  float* part;         // [max_batch][Hkv][max_chunks][G][d + 4]  attention partials (acc, max, sum, pad)
  float* mpart;        // [L][merge_b][Hkv][kMergeChunks][G][d + 4]  the same, per layer, when the O-projection merges
  float2* rope;        // [max_seq][d / 2]              (cos, sin)
  int* ev;             // [L][EV_COUNT][kEvInts]
  int* mctr;           // [L][max_batch][Hkv][kCtr]     attention merge counters
  int* chunk_base;     // [max_batch + 1]               prefix sum of chunks per request
  int4* queue;         // [grid][max_queue]
  int4* qev;           // [grid][max_queue]            each queued task's events (pmk_sched.h: task_events)
  int* qlen;           // [grid]
  int* err;            // [0] error word, [16] abort flag
  int* err_host;       // pinned, host-coherent mirror of the error word (written by the device when set)
  void* args;          // a copy of this step's StepArgs, written by the prologue
  float* kpart;        // split-K partial sums: per dense stage, [block tiles + tile][slice][rows nb + 16]
  int* tctr;           // [4][tctr_stride][kCtr] per (batch block, row tile): slices done (reset by the last one)
  int* bar;            // [L][kMaxStages][kEvInts]     stage barriers (barrier schedule only)
  // MoE
  float* logits;       // [max_batch][E]
  int* topk_idx;       // [max_batch][k]
  float* topk_w;       // [max_batch][k]
  int* exp_indptr;     // [E + 1]
  int* sorted_tok;     // [max_batch k]
  int* sorted_slot;    // [max_batch k]
  int* pos_of;         // [max_batch][k]  row of (t, j) in the grouped order
  int* tile_info;      // [max_tiles][2]  (expert, first grouped row) of each row tile
  int* moe_info;       // [0] gate/up tasks, [1] down tasks, [2] gate/up slices, [3] down slices, [4] tiles
  int* ectr;           // [L][E][kCtr]                  per-expert counters (gate/up -> down)
  int* tile_ptr;       // [E + 1]                       first row tile of each expert (tile_indptr)
  int* rq;             // [L][max_down]                 dynamic: ready down tasks, index + 1 (0: not yet pushed)
  int* mq;             // [L][kMq][kCtr]                dynamic: pop counter, push counter, per-XCD pop counters
  float* mact;         // [L][max_batch k][Fe]          expert SwiGLU rows, grouped order (per layer)
  float* mout;         // [max_batch k][H]              expert down rows, grouped order
  float* u;            // [max_batch][H]                per-op schedule: the RMSNorm output a projection reads
};

struct StepArgs {
  Dims dm;
  Workspace ws;
  const LayerPtrs* layers;   // device array [L]
  float* hidden;
  void* kv;
  const int32_t* seq_lens;
  int batch;
  int attn_chunk;                      // KV positions per attention task this step (set by the prologue)
  int attn_merge_o;                    // 1: O-projection inputs merge the attention partials (set by the prologue)
  int qkv_tiles;                       // QKV tiles this step, on workgroups 0.. (set by the prologue)
  int nblk;                            // event blocks of this step (set by the prologue; see pmk_sched.h)
  StageGeo geo[4];                     // QKV, O, gate/up, down split of this step (set by the prologue)
  unsigned long long watchdog_ticks;   // s_memrealtime ticks (100 MHz)
  pmk_routing rout;                    // optional routing outputs (device pointers)
  uint32_t* trace;                     // optional task trace [grid][trace_cap][8], caller-owned
  int trace_cap;                       // entries per workgroup (entry 0 is the header)
  int barrier;                         // 1: the barrier schedule (the prologue arms ws.bar)
  int moe_dyn;                         // 1: grouped expert tasks popped from a per-layer queue; 2: per-XCD queues
  int per_op;                          // 1: the per-op schedule (norms, RoPE, append, merge as ops of their own)
  int ev_mode;                         // granularity of the dense chain's events (pmk_sched.h: EvMode)
};

// Which task paths an instantiation of the persistent kernel carries: all of
// them (the ablation schedules, float32 weights), or, for the fused bfloat16
// kernel, those of a dense decoder layer or those of a MoE layer only. A dense
// handle never queues routing, grouped-expert or combine tasks, and a MoE
// handle never queues dense gate/up or down tasks; dropping the other kind's
// code halves the fused kernel (about 360 to 170 KB of instructions) and frees
// registers, which took 2-3 % off the batch-1 and batch-4 steps.
// KP_TILES (added to either): bfloat16 weights in the 16-row tile layout that
// pmk_pack_weights writes, streamed with non-temporal loads.
enum KernelPaths : int { KP_ALL = 0, KP_DENSE = 1, KP_MOE = 2, KP_TILES = 4 };

// What one launch of the persistent kernel runs: layers [l0, l1), and of
// their queue entries only the task types whose bit (1 << type) is set;
// barrier: a grid-wide barrier after every stage of every layer.
struct RunSpec {
  int l0, l1;
  unsigned types;
  int barrier;
};
constexpr unsigned kAllTypes = 0xffffffffu;

// Launch wrappers (defined in pmk_kernels.hip).
hipError_t launch_prologue(const StepArgs& a, hipStream_t s);
hipError_t launch_main(const StepArgs& a, int dtype, hipStream_t s, RunSpec rs);
hipError_t prepare_main(int dtype, int wtiles);
hipError_t launch_pack(const void* src, void* dst, long rows, long cols, hipStream_t s);

}  // namespace pmk
