// Host replay of a decode step's schedule (the functions of pmk_sched.h that
// the device prologue and the persistent kernel use): for a model shape, a
// batch and its lengths, build every workgroup's queue, arm every counter of
// the event tensor, and run the queues -- each workgroup takes its tasks in
// order, a task starts once the counters it waits on (task_wait) have reached
// zero, and a finished task notifies what the kernel's task notifies -- with
// the workgroups interleaved at random. Checked:
//  * no deadlock: some workgroup can always go on until every queue is done;
//  * every counter receives exactly its armed number of notifies (none goes
//    below zero, all end at zero);
//  * every consumer runs after every producer of the data it reads, with the
//    data each task reads and writes written out here from the tasks'
//    definitions (not from the event tensor): QKV rows per request and
//    rotation unit, attention output per request and KV group, h1, SwiGLU and
//    layer output rows per request, the MoE chain per token; including the
//    residual that O and down tasks load before their wait when the workgroup
//    has already seen an event that implies it is final.
//  * the split-K records of a tile, in use from its first slice task's store
//    to its last one's reduction, overlap no other tile's records in use and
//    lie inside their stage's region.
// The per-op schedule runs one launch per operator: the replay runs each
// launch's tasks (of one type) to completion before the next.
// With --fault drop|plus|minus, one notify is dropped, or one counter armed
// one too high or too low, and every such replay must report a failure; with
// --fault kpart, all dense stages address their split-K records from one base,
// and the replays where records of two tiles are in use at once must say so.
// Prints "ok <cases>" or the first failure.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <random>
#include <string>
#include <vector>

#include "../../persistent_megakernel_04_amd/csrc/pmk_sched.h"

using namespace pmk;

namespace {

struct Fail {
  std::string msg;
};

[[noreturn]] void fail(const std::string& m) { throw Fail{m}; }

pmk_model_desc make_desc(int dtype, int L, int H, int Hq, int Hkv, int d, int F, int E, int k, int Fe, int mb,
                         int ms) {
  pmk_model_desc x{};
  x.abi_version = PMK_ABI_VERSION;
  x.dtype = dtype;
  x.n_layers = L;
  x.hidden = H;
  x.n_q_heads = Hq;
  x.n_kv_heads = Hkv;
  x.head_dim = d;
  x.ffn_dim = F;
  x.n_experts = E;
  x.top_k = k;
  x.expert_ffn_dim = Fe;
  x.max_batch = mb;
  x.max_seq = ms;
  x.rms_eps = 1e-5f;
  x.rope_theta = 1e4f;
  return x;
}

struct Replay {
  Dims dm;
  Plan p;
  int L = 1;
  std::vector<int> sl, cb;
  std::vector<std::vector<int4>> q;
  std::vector<std::vector<int4>> qe;   // each task's events (task_events), as the kernel reads them
  std::map<long, int> ctr;           // counter (int offset in the event memory) -> count
  std::map<long, int> mctr;          // attention merge counters (l, b, g)
  std::map<long, int> slices;        // (stage, l, tile, block) -> slices done
  std::map<long, long2> held;        // (stage, l, tile, block) -> split-K records in use [x, y)
  std::map<long, int> done_tasks;    // (l, type) -> tasks done (MoE chain)
  // data produced so far, per layer: X and H1 rows [b][H] (+ per-row counts),
  // QKV units [b][qkv_units], attention output [b][Hkv], SwiGLU rows by the
  // gate/up tile that produced them [tile][b], the MoE routing
  std::vector<std::vector<uint8_t>> x_have, h1_have, qkv_have, o_have, act_have;
  std::vector<std::vector<int>> x_cnt, h1_cnt;
  std::vector<uint8_t> route_have;
  std::vector<std::vector<long>> seen;   // per workgroup, per wait kind: last event seen fired
  std::string fault;
  long fault_at = -1;                // the notify (by count) to drop
  long notifies = 0;

  // --- event tensor -------------------------------------------------------
  void arm() {
    const int nb = p.nblk, Hkv = dm.Hkv;
    for (int l = 0; l < L; ++l) {
      for (int kind : {EV_QKV, EV_ATTN})
        for (int b = 0; b < nb; ++b)
          for (int g = 0; g < Hkv; ++g) ctr[ev_off(dm, l, kind, b, g)] = ev_count(dm, p, cb.data(), kind, b, g, 0);
      for (int kind : {EV_O, EV_GU, EV_DOWN, EV_ROUTER, EV_ROUTE, EV_MDOWN}) {
        const int nbk = (kind == EV_O || kind == EV_GU || kind == EV_DOWN) ? nb : 1;
        for (int b = 0; b < nbk; ++b)
          for (int sub = 0; sub <= kSubs; ++sub)
            ctr[ev_off(dm, l, kind, b) + sub * kCtr] = ev_count(dm, p, cb.data(), kind, b, 0, sub);
      }
      for (int b = 0; b < p.B; ++b)
        for (int g = 0; g < Hkv; ++g) mctr[((long)l * p.B + b) * Hkv + g] = attn_pieces(dm, p, cb.data(), b, g);
    }
    if (fault == "plus" || fault == "minus") {   // a counter of layer 0 with a count > 0, off by one
      std::vector<long> offs;
      for (auto& kv : ctr)
        if (kv.second > 0 && kv.first < ev_layer_ints(dm)) offs.push_back(kv.first);
      const long o = offs[offs.size() / 2];
      ctr[o] += fault == "plus" ? 1 : -1;
    }
  }
  void notify(long off) {
    ++notifies;
    if (notifies == fault_at) return;   // the dropped notify
    auto it = ctr.find(off);
    if (it == ctr.end()) fail("notify of a counter that was never armed (offset " + std::to_string(off) + ")");
    if (--it->second < 0) fail("counter below zero (more notifies than armed) at offset " + std::to_string(off));
  }
  bool fired(long off, int counters) const {
    for (int i = 0; i < counters; ++i) {
      auto it = ctr.find(off + (long)i * kCtr);
      if (it == ctr.end()) fail("wait on a counter that was never armed (offset " + std::to_string(off) + ")");
      if (it->second != 0) return false;
    }
    return true;
  }
  // the wait of a task, as (offset, counters); counters 0: none -- from its
  // queue entry (task_events), as the kernel takes it
  std::pair<long, int> wait_of(int l, const int4& t, const int4& e) const {
    if (e.y < 0 || (l == 0 && (t.x & 0xff) == T_QKV)) return {0, 0};
    return {e.x + l * ev_layer_ints(dm), (e.y & 0xffff) + 1};
  }
  // the entry's notifies: w consecutive counters from z
  void notify_entry(int l, const int4& e) {
    if (e.z < 0) fail("a task that notifies has no counter in its queue entry");
    for (int i = 0; i < e.w; ++i) notify(e.z + l * ev_layer_ints(dm) + (long)i * kCtr);
  }
  static int wait_slot(int kind) {
    return kind == EV_QKV ? 0 : kind == EV_ATTN ? 1 : kind == EV_O ? 2 : kind == EV_GU ? 3 : kind == EV_DOWN ? 4 : 5;
  }

  // --- data ---------------------------------------------------------------
  void init_data() {
    const size_t B = p.B;
    auto mk = [&](std::vector<std::vector<uint8_t>>& v, size_t w) { v.assign(L, std::vector<uint8_t>(B * w, 0)); };
    mk(x_have, dm.H);
    mk(h1_have, dm.H);
    mk(qkv_have, dm.qkv_units);
    mk(o_have, dm.Hkv);
    mk(act_have, (size_t)(dm.moe ? 1 : p.geo[2].tiles));
    x_cnt.assign(L, std::vector<int>(B, 0));
    h1_cnt.assign(L, std::vector<int>(B, 0));
    route_have.assign(L, 0);
  }
  [[noreturn]] static void missing(const char* what, int l, int b, int i) {
    fail(std::string(what) + " read data not yet produced: layer " + std::to_string(l) + " request " +
         std::to_string(b) + " index " + std::to_string(i));
  }
  // rows [i0, i1) of request b in X (the layer input of layer l + 1) or H1 of layer l
  void need_rows(const std::vector<std::vector<uint8_t>>& v, const std::vector<std::vector<int>>& cnt, int l, int b,
                 int i0, int i1, const char* what) const {
    if (i0 == 0 && i1 == dm.H) {
      if (cnt[l][b] != dm.H) missing(what, l, b, -1);
      return;
    }
    for (int i = i0; i < i1; ++i)
      if (!v[l][(size_t)b * dm.H + i]) missing(what, l, b, i);
  }
  void put_rows(std::vector<std::vector<uint8_t>>& v, std::vector<std::vector<int>>& cnt, int l, int b, int i0, int i1) {
    for (int i = i0; i < i1; ++i) {
      uint8_t& f = v[l][(size_t)b * dm.H + i];
      if (f) fail("a row written twice in one step");
      f = 1;
      ++cnt[l][b];
    }
  }
  void need_x(int l, int b, int i0, int i1, const char* what) const {   // the layer input (the stack input is there)
    if (l > 0) need_rows(x_have, x_cnt, l - 1, b, i0, i1, what);
  }
  void need_units(int l, int b, int u0, int u1, const char* what) const {
    for (int u = u0; u < u1; ++u)
      if (!qkv_have[l][(size_t)b * dm.qkv_units + u]) missing(what, l, b, u);
  }
  // requests of batch block k of a stage (all of them when it is not split by block)
  int2 rows(int st, int k) const {
    if (p.geo[st].blk <= 1) return make_int2(0, p.B);
    const int b0 = k * kMaxNb;
    return make_int2(b0, b0 + kMaxNb < p.B ? b0 + kMaxNb : p.B);
  }
  // true for the slice task that completes (tile, block). A split tile's
  // records are in use from its first slice task's store to its last one's
  // reduction: no other tile's records may overlap them meanwhile, and they
  // lie inside the stage's region (the kernel's addressing, kpart_rec).
  bool stage_done(int st, int l, int tile, int blk) {
    const long key = (((long)st * L + l) * 65536 + tile) * 1024 + blk;
    const StageGeo& g = p.geo[st];
    const int cnt = ++slices[key];
    if (g.ks > 1) {
      int K, U, R;
      stage_dims(dm, st, K, U, R);
      const int nb = g.blk > 1 ? kMaxNb : (p.B < kMaxNb ? p.B : kMaxNb);
      const int rs = kpart_stride(U, R, g.tiles, nb);
      const int ti = tile + blk * g.tiles;
      const long r0 = kpart_rec(dm, st, ti, g.ks, 0, rs), r1 = kpart_rec(dm, st, ti + 1, g.ks, 0, rs);
      if (fault != "kpart" && r1 > dm.kpart_off[st + 1])
        fail("split-K records of stage " + std::to_string(st) + " tile " + std::to_string(ti) +
             " run past the stage's region");
      for (auto& h : held)
        if (h.first != key && h.second.x < r1 && r0 < h.second.y)
          fail("split-K records of stage " + std::to_string(st) + " layer " + std::to_string(l) + " tile " +
               std::to_string(ti) + " overlap records still in use (stage " + std::to_string(h.first / L / 65536 / 1024) +
               ")");
      if (cnt == 1) held[key] = make_long2(r0, r1);
      if (cnt == g.ks) held.erase(key);
    }
    return cnt == g.ks;
  }
  // the K slice [k0, k0 + kn) of task slice z of stage st
  int2 kslice(int st, int z) const {
    int K, U, R;
    stage_dims(dm, st, K, U, R);
    const int k0 = z * p.geo[st].kr, k1 = k0 + p.geo[st].kr < K ? k0 + p.geo[st].kr : K;
    return make_int2(k0, k1 - k0);
  }

  // Task t of workgroup w at layer l: check what it reads, record what it
  // writes, notify its events. Called when its wait has fired.
  void run(int w, int l, int4 t, const int4& e) {
    const int type = t.x & 0xff, Hkv = dm.Hkv, G = dm.Hq / Hkv, half = dm.d / 2;
    switch (type) {
      case T_QKV: {
        const int2 r = rows(0, t.w);
        for (int b = r.x; b < r.y; ++b) need_x(l, b, 0, dm.H, "QKV (its rows' RMSNorm)");
        if (!stage_done(0, l, t.y, t.w)) return;
        const int2 u = tile_units(t.y, dm.qkv_units, p.geo[0].tiles);
        for (int b = r.x; b < r.y; ++b)
          for (int up = u.x; up < u.x + u.y; ++up) {
            const int unit = qkv_unit(dm, up);
            qkv_have[l][(size_t)b * dm.qkv_units + unit] = 1;
          }
        const int2 gr = qkv_tile_groups(dm, p.geo[0].tiles, t.y);
        if (e.w != gr.y - gr.x + 1) fail("a QKV tile's entry notifies other than the groups its units cover");
        notify_entry(l, e);
        return;
      }
      case T_ATTN: case T_ATTS: {
        const int b = type == T_ATTN ? t.y : (t.y & 0xffff), g = type == T_ATTN ? t.z : (t.y >> 16);
        need_units(l, b, g * G * half, (g + 1) * G * half, "attention (its query heads)");
        need_units(l, b, dm.Hq * half + g * half, dm.Hq * half + (g + 1) * half, "attention (its key head)");
        need_units(l, b, (dm.Hq + Hkv) * half + g * half, (dm.Hq + Hkv) * half + (g + 1) * half,
                   "attention (its value head)");
        int& mc = mctr[((long)l * p.B + b) * Hkv + g];
        --mc;   // this chunk / piece of (b, g) is done
        if (p.merge || p.per_op) {   // every chunk notifies; the O-projection (or the merge op) merges
          if (mc == 0) o_have[l][(size_t)b * Hkv + g] = 1;
          notify_entry(l, e);
          return;
        }
        const int nc = type == T_ATTN ? cb[b + 1] - cb[b] : (t.x >> 20);
        if (nc == 1 || mc == 0) {   // the only, or the last, chunk / piece merges and notifies
          if (mc != 0) fail("a single-piece range whose merge counter was armed above one");
          o_have[l][(size_t)b * Hkv + g] = 1;
          notify_entry(l, e);
        }
        if (mc < 0) fail("attention merge counter below zero");
        return;
      }
      case T_O: {
        const int2 r = rows(1, t.w), ks = kslice(1, t.z);
        const int2 gr = o_slice_groups(dm, ks.x, ks.y);
        for (int b = r.x; b < r.y; ++b)
          for (int g = gr.x; g <= gr.y; ++g)
            if (!o_have[l][(size_t)b * Hkv + g]) missing("O-projection (attention of its K slice)", l, b, g);
        const int2 u = tile_units(t.y, dm.H, p.geo[1].tiles);
        for (int b = r.x; b < r.y; ++b) need_x(l, b, u.x, u.x + u.y, "O-projection (its residual)");
        if (!stage_done(1, l, t.y, t.w)) return;
        for (int b = r.x; b < r.y; ++b) put_rows(h1_have, h1_cnt, l, b, u.x, u.x + u.y);
        notify_entry(l, e);
        return;
      }
      case T_GU: {
        const int2 r = rows(2, t.w);
        for (int b = r.x; b < r.y; ++b) need_rows(h1_have, h1_cnt, l, b, 0, dm.H, "gate/up (its rows' RMSNorm)");
        if (!stage_done(2, l, t.y, t.w)) return;
        for (int b = r.x; b < r.y; ++b) act_have[l][(size_t)t.y * p.B + b] = 1;
        notify_entry(l, e);
        return;
      }
      case T_DOWN: {
        const int2 r = rows(3, t.w), ks = kslice(3, t.z);
        // the gate/up tiles whose rows (SwiGLU outputs) meet the K slice
        for (int gt = 0; gt < p.geo[2].tiles; ++gt) {
          const int2 gu = tile_units(gt, dm.F, p.geo[2].tiles);
          if (gu.x >= ks.x + ks.y || gu.x + gu.y <= ks.x) continue;
          for (int b = r.x; b < r.y; ++b)
            if (!act_have[l][(size_t)gt * p.B + b]) missing("down (its K slice of SwiGLU)", l, b, gt);
        }
        const int2 u = tile_units(t.y, dm.H, p.geo[3].tiles);
        for (int b = r.x; b < r.y; ++b) need_rows(h1_have, h1_cnt, l, b, u.x, u.x + u.y, "down (its residual)");
        if (!stage_done(3, l, t.y, t.w)) return;
        for (int b = r.x; b < r.y; ++b) put_rows(x_have, x_cnt, l, b, u.x, u.x + u.y);
        notify_entry(l, e);
        return;
      }
      // the MoE chain, per token (the grouped expert tasks' own per-expert
      // counters are data dependent and not part of this replay)
      case T_ROUTER: {
        const int b0 = t.z * kMaxNb, b1 = b0 + kMaxNb < p.B ? b0 + kMaxNb : p.B;
        for (int b = b0; b < b1; ++b) need_rows(h1_have, h1_cnt, l, b, 0, dm.H, "router (its tokens' RMSNorm)");
        ++done_tasks[(long)l * 64 + T_ROUTER];
        notify_entry(l, e);
        return;
      }
      case T_ROUTE: {
        if (done_tasks[(long)l * 64 + T_ROUTER] != dm.router_tiles * ceil_div_i(p.B, kMaxNb))
          fail("routing ran before every router task");
        route_have[l] = 1;
        notify_entry(l, e);
        return;
      }
      case T_MGU:
        if (!route_have[l]) missing("grouped gate/up (routing)", l, 0, 0);
        ++done_tasks[(long)l * 64 + T_MGU];
        return;
      case T_MDOWN:
        if (!route_have[l]) missing("grouped down (routing)", l, 0, 0);
        ++done_tasks[(long)l * 64 + T_MDOWN];
        notify_entry(l, e);
        return;
      case T_COMBINE: {
        if (done_tasks[(long)l * 64 + T_MDOWN] != dm.grid) fail("combine ran before every grouped down share");
        for (int b = w; b < p.B; b += dm.grid) put_rows(x_have, x_cnt, l, b, 0, dm.H);
        notify_entry(l, e);
        return;
      }
      default: return;   // the per-op schedule's separate ops: ordered by their launches
    }
  }

  // The early residual load of O / down tasks: before the task's wait, when
  // the workgroup has seen an event implying its residual rows are final (the
  // kernel's rule: O, the down event of the previous layer for its block or a
  // QKV event of its block in this layer; down, the O event of its block).
  void early_residual(int w, int l, int4 t) const {
    const int type = t.x & 0xff;
    if (type != T_O && type != T_DOWN) return;
    const int eb = ev_blk(p.nblk, t.w);
    bool early;
    if (type == T_O) {
      const long k = seen[w][0];
      early = l == 0 || seen[w][4] == ev_off(dm, l - 1, EV_DOWN, eb) ||
              (k >= ev_off(dm, l, EV_QKV, eb, 0) && k < ev_off(dm, l, EV_QKV, eb, dm.Hkv));
    } else {
      early = seen[w][2] == ev_off(dm, l, EV_O, eb);
    }
    if (!early) return;
    const int st = type == T_O ? 1 : 3;
    const int2 r = rows(st, t.w), u = tile_units(t.y, dm.H, p.geo[st].tiles);
    for (int b = r.x; b < r.y; ++b) {
      if (type == T_O) need_x(l, b, u.x, u.x + u.y, "O-projection's early residual load");
      else need_rows(h1_have, h1_cnt, l, b, u.x, u.x + u.y, "down's early residual load");
    }
  }

  // Replay all layers; launches: each a set of task types run to completion.
  void replay(std::mt19937& rng, const std::vector<unsigned>& launches) {
    const int W = dm.grid;
    seen.assign(W, std::vector<long>(8, -1));
    for (int l0 = 0; l0 < L; ++l0) {
      for (unsigned types : launches) {
        const bool fused = types == 0xffffffffu;
        const int l_end = fused ? L : l0 + 1;
        std::vector<int> pos(W, 0), lay(W, l0);
        auto next = [&](int w) -> int4* {   // the next task of w in this launch, skipping other types
          while (lay[w] < l_end) {
            if (pos[w] >= (int)q[w].size()) {
              pos[w] = 0;
              ++lay[w];
              continue;
            }
            int4& t = q[w][pos[w]];
            if ((types >> (t.x & 0xff)) & 1u) return &t;
            ++pos[w];
          }
          return nullptr;
        };
        for (;;) {
          // from a random workgroup on, the first one whose next task can start
          const int w0 = (int)(rng() % (unsigned)W);
          int w = -1;
          bool left = false;
          for (int i = 0; i < W && w < 0; ++i) {
            const int v = (w0 + i) % W;
            int4* t = next(v);
            if (!t) continue;
            left = true;
            const auto wt = wait_of(lay[v], *t, qe[v][t - q[v].data()]);
            if (wt.second == 0 || fired(wt.first, wt.second)) w = v;
          }
          if (!left) break;
          if (w < 0) {
            for (int v = 0; v < W; ++v)
              if (int4* t = next(v)) {
                char buf[200];
                std::snprintf(buf, sizeof buf, "deadlock: workgroup %d waits at layer %d on task type %d (%d, %d, %d)",
                              v, lay[v], t->x & 0xff, t->y, t->z, t->w);
                fail(buf);
              }
          }
          const int4* tp = next(w);
          const int4 t = *tp, e = qe[w][tp - q[w].data()];
          const auto wt = wait_of(lay[w], t, e);
          early_residual(w, lay[w], t);
          if (wt.second)   // record the event as seen, per wait kind (the kernel's cache)
            seen[w][wait_slot(e.y >> 16)] = wt.first;
          run(w, lay[w], t, e);
          ++pos[w];
        }
        if (fused) return;
      }
    }
  }

  void finish() const {
    for (auto& kv : ctr)
      if (kv.second != 0)
        fail("counter at offset " + std::to_string(kv.first) + " ends at " + std::to_string(kv.second) +
             " (fewer notifies than armed)");
    for (auto& kv : mctr)
      if (kv.second != 0) fail("attention merge counter ends at " + std::to_string(kv.second));
  }
};

struct Shape {
  const char* name;
  int dtype, H, Hq, Hkv, d, F, E, k, Fe;
};

// One replay; returns "" or the failure.
std::string check(const Shape& sh, int grid, int B, int max_seq, int lo, int hi, bool per_op, unsigned seed,
                  const std::string& fault, int L, int ev_mode) {
  Replay r;
  pmk_model_desc desc =
      make_desc(sh.dtype, L, sh.H, sh.Hq, sh.Hkv, sh.d, sh.F, sh.E, sh.k, sh.Fe, B < 16 ? 16 : B, max_seq);
  r.dm = dims_from_desc(desc, grid);
  if (fault == "kpart")   // every stage's split-K records from one base (one region shared by all stages)
    for (int st = 0; st < 4; ++st) r.dm.kpart_off[st] = 0;
  r.L = L;
  r.fault = fault;
  std::mt19937 rng(seed);
  r.sl.resize(B);
  for (int b = 0; b < B; ++b) r.sl[b] = lo + (int)(rng() % (unsigned)(hi - lo + 1));
  r.cb.resize(B + 1);
  r.p = plan_step(r.dm, B, r.sl.data(), r.cb.data(), per_op ? 1 : 0, ev_mode);
  r.q.resize(grid);
  r.qe.resize(grid);
  for (int w = 0; w < grid; ++w) {
    build_queue(r.dm, r.p, r.cb.data(), w, [&](int4 v) {
      r.q[w].push_back(v);
      r.qe[w].push_back(task_events(r.dm, r.p, v, w));
    });
    if ((int)r.q[w].size() > r.dm.max_queue) return "queue of workgroup " + std::to_string(w) + " above capacity";
  }
  r.arm();
  r.init_data();
  if (fault == "drop") {   // drop a notify from the middle of the first layer's
    long n = 0;
    for (auto& kv : r.ctr)
      if (kv.first < ev_layer_ints(r.dm)) n += kv.second;
    r.fault_at = n / 2 + 1;
  }
  std::vector<unsigned> launches;
  auto bit = [](int t) { return 1u << t; };
  if (per_op)
    launches = {bit(T_NORM1), bit(T_QKV), bit(T_ROPE), bit(T_APPEND), bit(T_ATTN), bit(T_MERGE), bit(T_O),
                bit(T_NORM2), bit(T_GU), bit(T_DOWN)};
  else
    launches = {0xffffffffu};
  try {
    r.replay(rng, launches);
    r.finish();
  } catch (const Fail& f) {
    return f.msg;
  }
  return "";
}

}  // namespace

// The plan's length aggregates (PlanAgg: the shift for a request's chunks)
// against their definitions: chunks of S cached positions plus the new entry
// at chunk size c are (S + c) / c, summed over the batch and maximised.
static bool check_aggregates() {
  for (int S = 0; S <= (1 << 20); ++S) {
    PlanAgg g{};
    plan_agg_add(g, S);
    for (int i = 0; i < kChunkSizes; ++i) {
      const int c = kMinChunk << i;
      if (g.tasks[i] != (S + c) / c || g.max_nc[i] != (S + c) / c) {
        std::printf("FAIL chunk count of %d positions at chunk %d\n", S, c);
        return false;
      }
    }
  }
  std::mt19937 rng(12345);
  for (int rep = 0; rep < 200; ++rep) {
    const int B = 1 + (int)(rng() % 1024);
    std::vector<int> sl(B);
    PlanAgg g{};
    long pos = 0, t[kChunkSizes] = {0, 0, 0};
    int mx[kChunkSizes] = {0, 0, 0};
    for (int b = 0; b < B; ++b) {
      sl[b] = (int)(rng() % 200000);
      plan_agg_add(g, sl[b]);
      pos += sl[b];
      for (int i = 0; i < kChunkSizes; ++i) {
        const int c = kMinChunk << i, nc = (sl[b] + c) / c;
        t[i] += nc;
        mx[i] = mx[i] > nc ? mx[i] : nc;
      }
    }
    bool ok = g.positions == pos;
    for (int i = 0; i < kChunkSizes; ++i) ok = ok && g.tasks[i] == t[i] && g.max_nc[i] == mx[i];
    if (!ok) {
      std::printf("FAIL aggregates of a batch of %d\n", B);
      return false;
    }
  }
  return true;
}

int main(int argc, char** argv) {
  std::string fault;
  for (int i = 1; i + 1 < argc; ++i)
    if (!std::strcmp(argv[i], "--fault")) fault = argv[i + 1];
  if (fault.empty() && !check_aggregates()) return 1;
  const Shape s8b{"8B", PMK_BF16, 4096, 32, 8, 128, 14336, 0, 0, 0};
  const Shape s70{"70B", PMK_BF16, 8192, 64, 8, 128, 28672, 0, 0, 0};
  const Shape stp{"70B TP share", PMK_BF16, 8192, 8, 1, 128, 3584, 0, 0, 0};
  const Shape s1{"tiny f32", PMK_F32, 256, 4, 2, 64, 688, 0, 0, 0};
  const Shape sf{"f32 mid", PMK_F32, 1024, 8, 2, 64, 4096, 0, 0, 0};
  const Shape smoe{"MoE", PMK_BF16, 2048, 32, 4, 128, 0, 128, 8, 768};
  struct Case { const Shape* sh; int grid, B, lo, hi; bool per_op; };
  std::vector<Case> cases;
  for (int B : {1, 2, 4, 8, 12, 16, 17, 33, 40, 64, 128}) cases.push_back({&s8b, 256, B, 0, 2100, false});
  for (int B : {1, 3, 16, 20}) cases.push_back({&s8b, 304, B, 500, 700, false});
  cases.push_back({&s8b, 256, 256, 16, 512, false});
  cases.push_back({&s8b, 256, 1024, 0, 24, false});
  for (int B : {1, 4, 20}) cases.push_back({&s8b, 256, B, 0, 900, true});
  for (int B : {1, 8, 12, 16, 20}) cases.push_back({&s70, 256, B, 100, 3000, false});
  for (int B : {1, 8}) cases.push_back({&stp, 256, B, 100, 3000, false});
  for (int B : {1, 3}) cases.push_back({&s1, 256, B, 0, 300, false});
  cases.push_back({&s1, 80, 3, 0, 300, true});
  for (int B : {1, 16}) cases.push_back({&sf, 256, B, 1, 300, false});
  for (int B : {1, 16, 128}) cases.push_back({&smoe, 256, B, 1, 2048, false});
  long n = 0;
  int faults_caught = 0, faults_tried = 0;
  for (const Case& c : cases) {
    const int ms = c.hi + 2;
    for (unsigned seed = 1; seed <= (fault.empty() ? 3u : 1u); ++seed) {
      // two layers: the second one's QKV waits on the first one's down stage;
      // the event granularity cycles through per tile, per group, per stage
      const int ev_mode = (int)((seed + c.B) % 3);
      const std::string e = check(*c.sh, c.grid, c.B, ms, c.lo, c.hi, c.per_op, seed * 7919u + c.B, fault, 2, ev_mode);
      ++n;
      if (fault.empty() && !e.empty()) {
        std::printf("FAIL %s grid %d batch %d lengths [%d, %d]%s seed %u event mode %d: %s\n", c.sh->name, c.grid, c.B,
                    c.lo, c.hi, c.per_op ? " per-op" : "", seed, ev_mode, e.c_str());
        return 1;
      }
      if (!fault.empty()) {
        ++faults_tried;
        if (!e.empty()) ++faults_caught;
        else if (fault != "kpart")
          std::printf("MISSED fault %s on %s grid %d batch %d\n", fault.c_str(), c.sh->name, c.grid, c.B);
      }
    }
  }
  if (!fault.empty()) {
    // a shared split-K region is a race only where two tiles' records are in
    // use at once: some of the cases must show it, not every one
    const bool ok = fault == "kpart" ? faults_caught > 0 : faults_caught == faults_tried;
    std::printf("%s %d of %d faults reported\n", ok ? "ok" : "FAIL", faults_caught, faults_tried);
    return ok ? 0 : 1;
  }
  std::printf("ok %ld\n", n);
  return 0;
}
