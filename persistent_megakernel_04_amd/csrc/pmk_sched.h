// pmk_sched.h -- one decode step's schedule as plain functions of the model's
// dimensions and (batch, seq_lens): the work split of every stage, each
// workgroup's task queue, and the event tensor -- which counters a task waits
// on, which it notifies, and the count every counter is armed with.
//
// This is the runtime instantiation of the layer's dependency template, whose
// batch and length dimensions stay symbolic until a step supplies them (Event
// Tensor summary page, Core method: Event Tensor abstraction, tile tasks and
// events with in/out edges; two kinds of dynamism: shape dynamism). The device
// prologue calls these functions every step; tests/host/sched_check.cpp calls
// the same functions on the host and replays the schedule they describe.
//
// The event tensor of a dense layer (flat counters are one int each, 64 bytes
// apart; hierarchical events are kEvInts ints, a counter [0] and kSubs
// sub-counters that spread the notifies of many producers):
//   QKV[blk][g]   flat: the QKV row tiles holding the rotation units of KV group g
//                 (its query heads, its key head, its value head) for batch
//                 block blk; the attention of (request b, group g) waits on
//                 QKV[blk(b)][g] alone;
//   ATTN[blk][g]  flat: the attention of the requests of block blk for group
//                 g; an O-projection task whose K slice covers heads of groups
//                 g0..g1 waits on ATTN[blk][g0..g1] alone;
//   O[blk], GU[blk], DOWN[blk]  hierarchical: the row tiles of the stage for
//                 block blk (gate/up waits on O of its block, down on GU, the
//                 next layer's QKV on DOWN);
//   ROUTER, ROUTE, MDOWN  the MoE chain (router logits, routing, grouped down).
// A batch block is 16 request rows; blocks get events of their own when every
// dense stage splits its tasks by block (batches beyond 16 whose every stage
// has a K split), so one block's stages can run ahead of another's. Otherwise
// there is one block.
#pragma once
#include "pmk_internal.h"

namespace pmk {

// Depth, units and rows per unit of the four dense stages.
__host__ __device__ inline void stage_dims(const Dims& dm, int st, int& K, int& U, int& R) {
  K = st == 0 ? dm.H : st == 1 ? dm.Hq * dm.d : st == 2 ? dm.H : dm.F;
  U = st == 0 ? dm.qkv_units : st == 1 ? dm.H : st == 2 ? dm.F : dm.H;
  R = (st == 0 || st == 2) ? 2 : 1;
}

// The handle's fixed dimensions from the model description and the device's
// compute-unit count (the persistent grid).
__host__ inline Dims dims_from_desc(const pmk_model_desc& desc, int grid) {
  auto cdiv = [](long a, long b) { return (int)((a + b - 1) / b); };
  Dims dm{};
  const bool moe = desc.n_experts > 0;
  dm.L = desc.n_layers; dm.H = desc.hidden; dm.Hq = desc.n_q_heads; dm.Hkv = desc.n_kv_heads;
  dm.d = desc.head_dim; dm.F = desc.ffn_dim; dm.E = desc.n_experts; dm.k = desc.top_k;
  dm.Fe = desc.expert_ffn_dim; dm.max_batch = desc.max_batch; dm.max_seq = desc.max_seq;
  // attention partial slots per (request, KV head): chunks of kMinChunk, or
  // streamed pieces of at least that many positions, one more when a range
  // starts inside a workgroup's share
  dm.max_chunks = cdiv(desc.max_seq, kMinChunk) + 1;
  dm.eps = desc.rms_eps;
  dm.grid = grid;
  dm.moe = moe ? 1 : 0;
  dm.kstep = desc.dtype == PMK_BF16 ? 32 : 16;
  dm.xpad = desc.dtype == PMK_BF16 ? 8 : 4;
  dm.attn_mm = desc.dtype == PMK_BF16 && dm.d == 128 && dm.Hq / dm.Hkv <= 8;
  dm.wtiles = desc.weight_layout == PMK_TILES ? 1 : 0;
  dm.merge_b = dm.max_batch < kMergeFloats / (dm.Hq * dm.d) ? dm.max_batch : kMergeFloats / (dm.Hq * dm.d);
  const int G = grid;
  auto mn = [](int a, int b) { return a < b ? a : b; };
  dm.qkv_units = (dm.Hq + 2 * dm.Hkv) * dm.d / 2;
  dm.qkv_tiles = mn(G, dm.qkv_units);
  dm.o_tiles = mn(G, dm.H);
  dm.gu_tiles = moe ? 0 : mn(G, dm.F);
  dm.down_tiles = moe ? 0 : mn(G, dm.H);
  dm.router_tiles = moe ? cdiv(dm.E, 16) : 0;
  dm.max_tiles = moe ? cdiv((long)dm.max_batch * dm.k, kMoeBM) + dm.E : 0;
  dm.max_down = dm.max_tiles * (dm.H / 16 > 1 ? dm.H / 16 : 1);
  // queue capacity: a dense stage's (tile, slice, block) tasks, slices and
  // tiles of a stage at most the grid, in groups of 8 per block; a
  // workgroup's attention share may also hold one piece of every (request, KV
  // head); + 16: the per-op schedule's norm, RoPE, append and merge entries
  const long attn_max = (long)dm.max_batch * dm.Hkv * dm.max_chunks;
  const int nblk = cdiv(dm.max_batch, kMaxNb);
  dm.tctr_stride = G * nblk;
  dm.max_queue = cdiv(dm.qkv_tiles, G) + cdiv(dm.o_tiles, G) + cdiv(attn_max, G) + dm.max_batch * dm.Hkv + 16 +
                 4 * (cdiv((long)(G + 8) * nblk, G) + 1);
  if (moe)
    dm.max_queue += cdiv((long)dm.router_tiles * cdiv(dm.max_batch, kMaxNb), G) + 4;
  else
    dm.max_queue += cdiv(dm.gu_tiles, G) + cdiv(dm.down_tiles, G);
  // split-K records: a region of its own for each dense stage, sized for
  // every batch and grid share (with events per KV group or per batch block,
  // one stage's tiles may still be reducing while a later stage's, or another
  // block's, store their slices)
  long off = 0;
  for (int st = 0; st < 4; ++st) {
    dm.kpart_off[st] = off;
    if (moe && st >= 2) continue;   // no dense gate/up or down stage
    int K, U, R;
    stage_dims(dm, st, K, U, R);
    off += (kpart_need(K, U, R, dm.max_batch, G, st <= 1, dm.kstep, dm.xpad) + 63) / 64 * 64;
  }
  dm.kpart_off[4] = off > 16 ? off : 16;
  return dm;
}

// First float of split-K record (stage st, tile index ti = block k x tiles +
// row tile, slice s), records rs floats apart.
__host__ __device__ inline long kpart_rec(const Dims& dm, int st, int ti, int ks, int s, int rs) {
  return dm.kpart_off[st] + ((long)ti * ks + s) * rs;
}

// This step's split and event-block count (set by plan_step).
struct Plan {
  int B;
  int ck;            // KV positions per attention chunk
  int merge;         // 1: the O-projection merges the chunk partials
  int stream;        // 1: attention streams equal shares of the laid-out positions
  int own;           // attention tasks on workgroups of their own (the last `own`)
  int total_attn;    // chunked attention tasks (sum over requests of chunks x Hkv)
  long share;        // streamed: positions (with each range's lead) per workgroup
  int nblk;          // event blocks (see above)
  int per_op;        // the per-op schedule
  int ev_mode;       // EVM_TILE, EVM_GROUP or EVM_STAGE (pmk_set_event_granularity)
  StageGeo geo[4];   // QKV, O, gate/up, down
};

// Granularity of the dense chain's events: per tile (KV group and batch
// block), per KV group only (one batch block), or one event per stage (every
// attention task waits on every group's QKV tiles, every O task on every
// group's attention: the stage-wide events of a plain megakernel).
enum EvMode : int { EVM_TILE = 0, EVM_GROUP = 1, EVM_STAGE = 2 };

__host__ __device__ inline int ceil_div_i(long a, long b) { return (int)((a + b - 1) / b); }


// What the step's split needs of the requests' lengths: for each chunk size
// kMinChunk << i (i < kChunkSizes), the chunks of all requests together and
// the most chunks of one request ((S + c) / c for a request with S cached
// positions: its new entry included), and the positions of all requests.
constexpr int kChunkSizes = 3;   // 64, 128, 256 = kMaxChunk
struct PlanAgg {
  long tasks[kChunkSizes];
  int max_nc[kChunkSizes];
  long positions;                // sum of S
};
__host__ __device__ inline void plan_agg_add(PlanAgg& g, int S) {
  for (int i = 0; i < kChunkSizes; ++i) {
    const int nc = (S >> (6 + i)) + 1;   // (S + c) / c, c = kMinChunk << i = 2^(6 + i)
    g.tasks[i] += nc;
    g.max_nc[i] = g.max_nc[i] > nc ? g.max_nc[i] : nc;
  }
  g.positions += S;
}
// The step's split from the lengths' aggregates: attention chunking,
// streaming and dedicated attention workgroups (every field but geo and nblk).
__host__ __device__ inline Plan plan_attention(const Dims& dm, int B, const PlanAgg& g, int per_op, int ev_mode) {
  static_assert(kMinChunk == 64 && kMaxChunk == kMinChunk << (kChunkSizes - 1), "chunk sizes");
  Plan p{};
  p.B = B;
  p.per_op = per_op;
  p.ev_mode = ev_mode;
  const int G = dm.grid;
  // Small batches whose O-projection inputs fit one merging pass take the
  // smallest chunk that keeps every request within 8 chunks and let the
  // O-projection merge the partials; otherwise the largest of 256/128/64
  // positions that still gives every workgroup a task, with the last chunk
  // of a request merging.
  int ci = kChunkSizes - 1, merge = 0;
  if (B <= dm.merge_b && !per_op) {
    int c = 0;
    while (c < kChunkSizes - 1 && g.max_nc[c] > kMergeChunks) ++c;
    if (g.max_nc[c] <= kMergeChunks) { ci = c; merge = 1; }
  }
  if (!merge)
    while (ci > 0 && g.tasks[ci] * dm.Hkv < G) --ci;
  p.ck = kMinChunk << ci;
  p.merge = merge;
  // Without the O-projection merge, the matrix-core attention streams its
  // positions: all (request, KV head) position ranges, laid end to end, are
  // cut into equal shares, one per workgroup (at least 64 positions), and each
  // piece of a range within a share is a task. The per-op schedule keeps chunk
  // partials, merged by an op of their own.
  p.stream = !merge && dm.attn_mm && !per_op;
  // cb[B]: positions (S + 1 each, streamed) or chunks
  const long acc = p.stream ? g.positions + B : g.tasks[ci];
  p.total_attn = (int)(acc * dm.Hkv);
  // streamed shares: every (request, KV head) range is laid out behind a lead
  // of kPieceCost positions (what a piece costs beyond its positions), so that
  // a share that starts a range holds fewer positions
  const long P = p.stream ? (long)dm.Hkv * (acc + (long)B * kPieceCost) : acc * dm.Hkv;
  const long sh = (P + G - 1) / G;
  p.share = ((sh + 15) / 16 * 16) < 64 ? 64 : (sh + 15) / 16 * 16;
  // A few attention tasks (at most a quarter of the grid) get workgroups of
  // their own, the last ones, which hold no QKV or O tile: their task comes
  // first in the layer, so its KV rows stream in while the QKV tiles run on
  // the other workgroups.
  p.own = (merge && p.total_attn <= G / 4 && !per_op) ? p.total_attn : 0;
  return p;
}
// One request's entry of cb (the prefix sum of positions S + 1, streamed, or
// of chunks ceil((S + 1) / ck)).
__host__ __device__ inline int plan_cb_term(const Plan& p, int S) { return p.stream ? S + 1 : (S + p.ck) / p.ck; }
// Dense stage st's split (stage_split): up to 16 rows, one pass over K
// slices that fit the LDS; beyond, blocks of 16 rows over larger row tiles
// (or, where no split fits, passes of rows over the whole depth).
__host__ __device__ inline StageGeo plan_geo(const Dims& dm, const Plan& p, int st) {
  if (dm.moe && st >= 2) return StageGeo{1, 1, 1, 1};   // MoE layers have no dense gate/up or down stage
  int K, U, R;
  stage_dims(dm, st, K, U, R);
  const int avail = st <= 1 ? dm.grid - p.own : dm.grid;
  return stage_split(K, U, R, p.B, avail, dm.kstep, dm.xpad);
}
// Events per block when every dense stage splits by block (MoE layers keep
// one block: their routed stages cover all tokens at once).
__host__ __device__ inline int plan_nblk(const Dims& dm, const Plan& p) {
  bool all_blocked = p.B > kMaxNb;
  for (int st = 0; st < 4; ++st)
    if (!(dm.moe && st >= 2) && p.geo[st].blk <= 1) all_blocked = false;
  return (all_blocked && !dm.moe && p.ev_mode == EVM_TILE) ? (p.B + kMaxNb - 1) / kMaxNb : 1;
}

// The step's split from (B, sl), serially: the composition of the parts above
// (the device prologue computes the same parts in parallel). cb[0..B]
// receives the prefix sum of the requests' positions (S + 1, streamed) or
// chunks.
__host__ __device__ inline Plan plan_step(const Dims& dm, int B, const int* sl, int* cb, int per_op,
                                          int ev_mode = EVM_TILE) {
  PlanAgg g{};
  for (int b = 0; b < B; ++b) plan_agg_add(g, sl[b]);
  Plan p = plan_attention(dm, B, g, per_op, ev_mode);
  int acc = 0;
  for (int b = 0; b < B; ++b) {
    cb[b] = acc;
    acc += plan_cb_term(p, sl[b]);
  }
  cb[B] = acc;
  for (int st = 0; st < 4; ++st) p.geo[st] = plan_geo(dm, p, st);
  p.nblk = plan_nblk(dm, p);
  return p;
}

// ---------------------------------------------------------------------------
// Event tensor layout (ints from the base of the event memory)
// ---------------------------------------------------------------------------
__host__ __device__ inline int ev_nbm(const Dims& dm) { return (dm.max_batch + kMaxNb - 1) / kMaxNb; }
__host__ __device__ inline long ev_layer_ints(const Dims& dm) {
  return 2L * ev_nbm(dm) * dm.Hkv * kCtr + (3L * ev_nbm(dm) + 3) * kEvInts;
}
// Offset of event (kind, blk, g) of layer l. QKV and ATTN: flat counters,
// consecutive over g (so a wait on groups g0..g1 reads one contiguous run);
// O, GU, DOWN: hierarchical, per block; ROUTER, ROUTE, MDOWN: one each.
__host__ __device__ inline long ev_off(const Dims& dm, int l, int kind, int blk = 0, int g = 0) {
  const long nbm = ev_nbm(dm), flat = nbm * dm.Hkv * kCtr, base = (long)l * ev_layer_ints(dm);
  switch (kind) {
    case EV_QKV: return base + ((long)blk * dm.Hkv + g) * kCtr;
    case EV_ATTN: return base + flat + ((long)blk * dm.Hkv + g) * kCtr;
    case EV_O: return base + 2 * flat + (long)blk * kEvInts;
    case EV_GU: return base + 2 * flat + (nbm + blk) * kEvInts;
    case EV_DOWN: return base + 2 * flat + (2 * nbm + blk) * kEvInts;
    case EV_ROUTER: return base + 2 * flat + (3 * nbm) * kEvInts;
    case EV_ROUTE: return base + 2 * flat + (3 * nbm + 1) * kEvInts;
    default: return base + 2 * flat + (3 * nbm + 2) * kEvInts;   // EV_MDOWN
  }
}
__host__ __device__ inline bool ev_flat(int kind) { return kind == EV_QKV || kind == EV_ATTN; }

// The event block of batch block k (or of request b: block b / 16), with
// `nblk` event blocks this step.
__host__ __device__ inline int ev_blk(int nblk, int k) { return nblk > 1 ? k : 0; }

// QKV rotation units in group-major order: KV group g owns the units of its G
// query heads, then of its key head, then of its value head (d / 2 units a
// head), so that a QKV row tile covers one group, or two at a boundary.
__host__ __device__ inline int qkv_unit(const Dims& dm, int up) {
  const int half = dm.d >> 1, G = dm.Hq / dm.Hkv, per = (G + 2) * half, g = up / per, r = up - g * per;
  if (r < G * half) return g * G * half + r;
  if (r < (G + 1) * half) return dm.Hq * half + g * half + (r - G * half);
  return (dm.Hq + dm.Hkv) * half + g * half + (r - (G + 1) * half);
}
// Row tile `tile` of `units` units split in `tiles`: first unit and count.
__host__ __device__ inline int2 tile_units(int tile, int units, int tiles) {
  // 32-bit when the products fit (every model shape here: the 64-bit
  // division is a long software sequence on the device)
  if ((unsigned long)(tiles + 1) * (unsigned)units <= 0xffffffffUL) {
    const unsigned u0 = (unsigned)tile * (unsigned)units / (unsigned)tiles;
    return make_int2((int)u0, (int)((unsigned)(tile + 1) * (unsigned)units / (unsigned)tiles - u0));
  }
  const int u0 = (int)((long)tile * units / tiles);
  return make_int2(u0, (int)((long)(tile + 1) * units / tiles) - u0);
}
// KV groups a QKV row tile covers (of `tiles` this step): x = first, y = last.
__host__ __device__ inline int2 qkv_tile_groups(const Dims& dm, int tiles, int tile) {
  const int per = (dm.Hq / dm.Hkv + 2) * (dm.d >> 1);
  const int2 u = tile_units(tile, dm.qkv_units, tiles);
  return make_int2(u.x / per, (u.x + (u.y > 0 ? u.y : 1) - 1) / per);
}
// KV groups whose query heads an O-projection K slice [k0, k0 + kn) reads.
__host__ __device__ inline int2 o_slice_groups(const Dims& dm, int k0, int kn) {
  const int gw = dm.Hq / dm.Hkv * dm.d;
  return make_int2(k0 / gw, (k0 + kn - 1) / gw);
}
// Notifiers of a hierarchical event with n notifiers indexed i (sub-counter
// i % kSubs), each `mult` times: the count of sub-counter x.
__host__ __device__ inline int sub_indexed(int n, int mult, int x) {
  return (n > x ? (n - x + kSubs - 1) / kSubs : 0) * mult;
}
// Tasks t < tiles that run on workgroup t % grid and notify sub-counter
// (t % grid) % kSubs: the count of sub-counter x.
__host__ __device__ inline int sub_tiles(int tiles, int grid, int x) {
  auto below = [x](int n) { return n > x ? (n - x + kSubs - 1) / kSubs : 0; };   // w < n with w % kSubs == x
  return (tiles / grid) * below(grid) + below(tiles % grid);
}
// Requests in batch block blk: [b0, b1).
__host__ __device__ inline int2 block_requests(const Plan& p, int blk) {
  if (p.nblk <= 1) return make_int2(0, p.B);
  const int b0 = blk * kMaxNb, b1 = b0 + kMaxNb < p.B ? b0 + kMaxNb : p.B;
  return make_int2(b0, b1);
}

// The count counter `sub` (0 for [0], 1 + x for sub-counter x; flat events
// have [0] only) of event (kind, blk, g) of a layer is armed with.
// QKV row tiles whose units meet KV group g.
__host__ __device__ inline int qkv_group_tiles(const Dims& dm, const Plan& p, int g) {
  int n = 0;
  for (int t = 0; t < p.geo[0].tiles; ++t) {
    const int2 gr = qkv_tile_groups(dm, p.geo[0].tiles, t);
    if (gr.x <= g && g <= gr.y) ++n;
  }
  return n;
}
// gtiles (nullable): qkv_group_tiles of every group, precomputed.
__host__ __device__ inline int ev_count(const Dims& dm, const Plan& p, const int* cb, int kind, int blk, int g,
                                        int sub, const int* gtiles = nullptr) {
  const int G = dm.grid;
  const int x = sub - 1;
  switch (kind) {
    case EV_QKV: {   // QKV row tiles covering group g, once per batch block they stand for
      if (sub != 0) return 0;
      const int n = gtiles ? gtiles[g] : qkv_group_tiles(dm, p, g);
      return n * (p.nblk > 1 ? 1 : p.geo[0].blk);
    }
    case EV_ATTN: {  // the attention tasks that finish (request, group g) of block blk
      if (sub != 0) return 0;
      const int2 r = block_requests(p, blk);
      if (p.merge || p.per_op) return cb[r.y] - cb[r.x];   // every chunk task notifies
      return r.y - r.x;                                    // one notify per request
    }
    case EV_O: case EV_GU: case EV_DOWN: {
      if (sub == 0) return 0;
      if (dm.moe && kind != EV_O) {   // MoE: DOWN is the combine, one slot per workgroup; no GU
        return kind == EV_DOWN ? sub_tiles(G, G, x) : 0;
      }
      const StageGeo& sg = p.geo[kind == EV_O ? 1 : kind == EV_GU ? 2 : 3];
      return sub_indexed(sg.tiles, p.nblk > 1 ? 1 : sg.blk, x);
    }
    case EV_ROUTER: {
      if (sub == 0 || !dm.moe) return 0;
      return sub_tiles(dm.router_tiles * ceil_div_i(p.B, kMaxNb), G, x);
    }
    case EV_ROUTE: return (sub == 0 && dm.moe) ? 1 : 0;
    default:   // EV_MDOWN: one notify per workgroup
      return (sub != 0 && dm.moe) ? sub_tiles(G, G, x) : 0;
  }
}

// The events a task waits on before it starts (the grouped expert tasks'
// data-dependent per-expert counters aside): `n` consecutive flat counters
// from (kind, blk, g0) of layer `layer` (QKV, ATTN), or one hierarchical event
// (n = 1); kind < 0: none. Task fields as queued: type, y, z, w; `nblk` event
// blocks, `o_kr` the O-projection's K slice length this step.
struct EvWait { int kind, layer, blk, g0, n; };
// ev_mode EVM_STAGE: attention and O tasks wait on every group.
__host__ __device__ inline EvWait task_wait(const Dims& dm, int nblk, int o_kr, int type, int y, int z, int w,
                                            int l, int ev_mode = EVM_TILE) {
  const bool all = ev_mode == EVM_STAGE;
  switch (type) {
    case T_QKV:   // the previous layer's down stage of this block (MoE: its combine)
      if (l == 0) break;
      return EvWait{EV_DOWN, l - 1, dm.moe ? 0 : ev_blk(nblk, w), 0, 1};
    case T_ATTN:   // (request y, group z): the QKV tiles of its block and group
      return EvWait{EV_QKV, l, ev_blk(nblk, y / kMaxNb), all ? 0 : z, all ? dm.Hkv : 1};
    case T_ATTS:   // a streamed piece of (request y & 0xffff, group y >> 16)
      return EvWait{EV_QKV, l, ev_blk(nblk, (y & 0xffff) / kMaxNb), all ? 0 : y >> 16, all ? dm.Hkv : 1};
    case T_O: {    // the attention of its block for the groups whose heads its K slice z reads
      const int K = dm.Hq * dm.d, k0 = z * o_kr, kn = (K < k0 + o_kr ? K : k0 + o_kr) - k0;
      const int2 gr = all ? make_int2(0, dm.Hkv - 1) : o_slice_groups(dm, k0, kn);
      return EvWait{EV_ATTN, l, ev_blk(nblk, w), gr.x, gr.y - gr.x + 1};
    }
    case T_GU: return EvWait{EV_O, l, ev_blk(nblk, w), 0, 1};
    case T_DOWN: return EvWait{EV_GU, l, ev_blk(nblk, w), 0, 1};
    case T_ROUTER: return EvWait{EV_O, l, 0, 0, 1};
    case T_ROUTE: return EvWait{EV_ROUTER, l, 0, 0, 1};
    case T_MGU: return EvWait{EV_ROUTE, l, 0, 0, 1};
    case T_COMBINE: return EvWait{EV_MDOWN, l, 0, 0, 1};
    default: break;
  }
  return EvWait{-1, 0, 0, 0, 0};
}

// A task's events as its queue entry carries them, so that the persistent
// kernel does no event arithmetic of its own (offsets into the event memory
// as if the task were in layer 0; layer l adds l ev_layer_ints):
//   x  the first counter the task waits on (a QKV task waits on the previous
//      layer's down event: x is layer -1's, and layer 0's QKV tasks wait on
//      nothing);
//   y  the counters past the first (a flat run) or kSubs (a hierarchical
//      event), | the awaited event's kind << 16; -1: no wait;
//   z  the counter the task notifies (of a hierarchical event, the
//      sub-counter its tile or workgroup takes); -1: none. A split tile's
//      slices notify only when they complete it;
//   w  consecutive flat counters it notifies (a QKV tile: the KV groups its
//      units cover).
// Attention tasks notify from their own code (the chunk or piece that
// finishes the request's group), at z.
__host__ __device__ inline int4 task_events(const Dims& dm, const Plan& p, int4 t, int wg) {
  const int type = t.x & 0xff;
  const long LI = ev_layer_ints(dm);
  int4 e = make_int4(0, -1, -1, 0);
  // layer 1's wait, moved back one layer (so that QKV's is layer -1's)
  const EvWait wt = task_wait(dm, p.nblk, p.geo[1].kr, type, t.y, t.z, t.w, 1, p.ev_mode);
  if (wt.kind >= 0) {
    e.x = (int)(ev_off(dm, wt.layer, wt.kind, wt.blk, wt.g0) - LI);
    e.y = (ev_flat(wt.kind) ? wt.n - 1 : kSubs) | (wt.kind << 16);
  }
  auto sub_of = [](int i) { return (1 + (i & (kSubs - 1))) * kCtr; };
  switch (type) {
    case T_QKV: {
      const int2 gr = qkv_tile_groups(dm, p.geo[0].tiles, t.y);
      e.z = (int)ev_off(dm, 0, EV_QKV, ev_blk(p.nblk, t.w), gr.x);
      e.w = gr.y - gr.x + 1;
      break;
    }
    case T_O: case T_GU: case T_DOWN:
      e.z = (int)ev_off(dm, 0, type == T_O ? EV_O : type == T_GU ? EV_GU : EV_DOWN, ev_blk(p.nblk, t.w)) +
            sub_of(t.y);
      e.w = 1;
      break;
    case T_ATTN: case T_ATTS: {
      const int b = type == T_ATTN ? t.y : (t.y & 0xffff), g = type == T_ATTN ? t.z : (t.y >> 16);
      e.z = (int)ev_off(dm, 0, EV_ATTN, ev_blk(p.nblk, b / kMaxNb), g);
      e.w = 1;
      break;
    }
    case T_ROUTER: e.z = (int)ev_off(dm, 0, EV_ROUTER) + sub_of(wg); e.w = 1; break;
    case T_ROUTE: e.z = (int)ev_off(dm, 0, EV_ROUTE); e.w = 1; break;
    case T_MDOWN: e.z = (int)ev_off(dm, 0, EV_MDOWN) + sub_of(wg); e.w = 1; break;
    case T_COMBINE: e.z = (int)ev_off(dm, 0, EV_DOWN) + sub_of(wg); e.w = 1; break;
    default: break;
  }
  return e;
}

// Pieces of (request b, KV head g) that streamed attention cuts its range into
// (the workgroups whose shares meet the range's positions), or the request's
// chunks: the count of its merge counter (the last piece or chunk merges).
__host__ __device__ inline int attn_pieces(const Dims& dm, const Plan& p, const int* cb, int b, int g) {
  int n = cb[b + 1] - cb[b];
  if (p.stream) {
    const long r0 = (long)dm.Hkv * (cb[b] + (long)b * kPieceCost) + (long)g * (n + kPieceCost) + kPieceCost;
    n = (int)((r0 + n - 1) / p.share - r0 / p.share) + 1;
  }
  return n;
}

// The task queue of workgroup w, in stage order (QKV, attention, O, then
// gate/up, down for dense layers, or router, routing, grouped gate/up,
// grouped down, combine for MoE layers; the per-op schedule interleaves its
// separate norm, RoPE, append and merge ops). push(int4) receives each task.
template <typename Push>
__host__ __device__ inline void build_queue(const Dims& dm, const Plan& p, const int* cb, int w, Push&& push) {
  const int G = dm.grid, B = p.B;
  const int aw0 = p.own ? G - p.own : G;
  // task i of a dense stage: row tile i / ks, K slice i % ks, on workgroup
  // i % G. In batch blocks, the blocks of one (tile, slice) go to workgroups 8
  // apart, which share an L2 (one XCD), so that they stream the same weights
  // together: groups of 8 (tile, slice) pairs, each group's blocks one after
  // another.
  auto stage_tasks = [&](int type, int st) {
    const StageGeo g = p.geo[st];
    const int TS = g.tiles * g.ks;
    if (g.blk <= 1) {
      for (int i = w; i < TS; i += G) push(make_int4(type, i / g.ks, i % g.ks, 0));
      return;
    }
    const int per = 8 * g.blk;
    for (int i = w; i < (TS + 7) / 8 * per; i += G) {
      const int grp = i / per, r = i - grp * per, ts = grp * 8 + (r & 7);
      if (ts < TS) push(make_int4(type, ts / g.ks, ts % g.ks, r >> 3));
    }
  };
  if (p.per_op) push(make_int4(T_NORM1, 0, 0, 0));
  stage_tasks(T_QKV, 0);
  if (p.per_op) {
    push(make_int4(T_ROPE, 0, 0, 0));
    push(make_int4(T_APPEND, 0, 0, 0));
  }
  if (p.stream) {   // this workgroup's share of the laid-out ranges
    // range (b, g) spans [seg0, seg0 + kPieceCost + S_b + 1): its lead, then its positions
    auto start = [&](int b) { return (long)dm.Hkv * (cb[b] + (long)b * kPieceCost); };
    const long share = p.share, hi = (long)(w + 1) * share < start(B) ? (long)(w + 1) * share : start(B);
    for (long pos = (long)w * share; pos < hi;) {
      int lo = 0, up = B;   // request b: start(b) <= pos < start(b + 1)
      while (up - lo > 1) {
        const int mid = (lo + up) >> 1;
        if (start(mid) <= pos) lo = mid; else up = mid;
      }
      const int len = cb[lo + 1] - cb[lo], span = len + kPieceCost;
      const int g = (int)((pos - start(lo)) / span);
      const long seg0 = start(lo) + (long)g * span, r0 = seg0 + kPieceCost, seg1 = seg0 + span;
      const long e = hi < seg1 ? hi : seg1, p0 = pos > r0 ? pos : r0;
      if (e > p0) {
        // pieces of a range are cut at multiples of the share: this is piece
        // w - r0 / share of (seg1 - 1) / share - r0 / share + 1
        const int piece = w - (int)(r0 / share), np = (int)((seg1 - 1) / share - r0 / share) + 1;
        push(make_int4(T_ATTS | (piece << 8) | (np << 20), lo | (g << 16), (int)(p0 - r0), (int)(e - r0)));
      }
      pos = e;
    }
  }
  for (int i = aw0 < G ? w - aw0 : w; !p.stream && i >= 0 && i < p.total_attn; i += (aw0 < G ? p.total_attn : G)) {
    int lo = 0, hi = B;   // find b: Hkv cb[b] <= i < Hkv cb[b + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (dm.Hkv * cb[mid] <= i) lo = mid; else hi = mid;
    }
    const int r = i - dm.Hkv * cb[lo], nc = cb[lo + 1] - cb[lo];
    push(make_int4(T_ATTN | (i << 8), lo, r / nc, r % nc));
  }
  if (p.per_op) push(make_int4(T_MERGE, 0, 0, 0));
  stage_tasks(T_O, 1);
  if (p.per_op) push(make_int4(T_NORM2, 0, 0, 0));
  if (!dm.moe) {
    stage_tasks(T_GU, 2);
    stage_tasks(T_DOWN, 3);
  } else {
    const int router_tasks = dm.router_tiles * ceil_div_i(B, kMaxNb);
    for (int i = w; i < router_tasks; i += G) push(make_int4(T_ROUTER, i % dm.router_tiles, i / dm.router_tiles, 0));
    if (w == G - 1) push(make_int4(T_ROUTE, 0, 0, 0));
    push(make_int4(T_MGU, 0, 0, 0));
    push(make_int4(T_MDOWN, 0, 0, 0));
    push(make_int4(T_COMBINE, 0, 0, 0));
  }
}

}  // namespace pmk
