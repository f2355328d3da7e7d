// pmk_api.hip -- host runtime behind the C ABI of include/pmk.h: argument
// checks, workspace carving, the RoPE table, launch of the prologue and the
// persistent kernel, device-error readback and optional per-launch timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "pmk_internal.h"
#include "pmk_sched.h"

using namespace pmk;

struct pmk_handle {
  pmk_model_desc desc;
  int device = 0;
  Dims dm{};
  Workspace ws{};
  void* ws_base = nullptr;
  size_t ws_bytes = 0;
  LayerPtrs* d_layers = nullptr;
  hipStream_t last_stream = nullptr;
  unsigned long long watchdog_ticks = 0;
  unsigned long long watchdog_init = 0;   // the limit from the descriptor
  bool timing = false;
  uint32_t* trace = nullptr;
  int trace_cap = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> tev;
  int* err_host = nullptr;   // pinned host-coherent mirror of the device error word
  size_t tused = 0;
  int sched = PMK_SCHED_FUSED;
  int ev_mode = PMK_EVENTS_GROUP;
  int moe_sched = PMK_MOE_STATIC;
};

namespace {

int elem_bytes(int dtype) { return dtype == PMK_BF16 ? 2 : 4; }
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

int check_desc(const pmk_model_desc* d) {
  if (!d || d->abi_version != PMK_ABI_VERSION) return PMK_ERR_ARG;
  if (d->dtype != PMK_F32 && d->dtype != PMK_BF16) return PMK_ERR_ARG;
  if (d->n_layers < 1 || d->hidden < 8 || d->hidden % 8) return PMK_ERR_ARG;
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads) return PMK_ERR_ARG;
  if (d->head_dim < 2 || d->head_dim % 2) return PMK_ERR_ARG;
  if (d->max_batch < 1 || d->max_seq < 1) return PMK_ERR_ARG;
  if (!(d->rms_eps > 0.f) || !(d->rope_theta > 0.f)) return PMK_ERR_ARG;
  if (d->n_experts < 0) return PMK_ERR_ARG;
  if (d->weight_layout != PMK_ROWS && d->weight_layout != PMK_TILES) return PMK_ERR_ARG;
  if (d->n_experts == 0 && (d->ffn_dim < 8 || d->ffn_dim % 8)) return PMK_ERR_ARG;
  if (d->n_experts > 0 && (d->top_k < 1 || d->top_k > d->n_experts || d->expert_ffn_dim < 8 ||
                           d->expert_ffn_dim % 8))
    return PMK_ERR_ARG;
  // shapes this build implements
  if (d->head_dim * elem_bytes(d->dtype) != 256) return PMK_ERR_UNSUPPORTED;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PMK_ERR_UNSUPPORTED;
  if (d->n_kv_heads > kMaxHkv) return PMK_ERR_UNSUPPORTED;
  if (d->max_batch > kMaxBatchAll) return PMK_ERR_UNSUPPORTED;
  if (d->weight_layout == PMK_TILES) {
    // bfloat16 only; every matrix in whole 16-row groups and 32-column steps
    const int qd = d->n_q_heads * d->head_dim, qkv = (d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
    if (d->dtype != PMK_BF16 || d->hidden % 32 || qd % 32 || qkv % 16) return PMK_ERR_UNSUPPORTED;
    if (d->n_experts == 0 && d->ffn_dim % 32) return PMK_ERR_UNSUPPORTED;
    if (d->n_experts > 0 && (d->expert_ffn_dim % 32 || d->n_experts % 16)) return PMK_ERR_UNSUPPORTED;
  }
  // every GEMV depth must leave room for one staged input row in LDS (float32
  // inputs, or bfloat16 hi + lo pairs: 4 bytes per element either way)
  const int xrow_max = kXsBytes / 4 - 64;
  if (d->hidden > xrow_max || d->n_q_heads * d->head_dim > xrow_max) return PMK_ERR_UNSUPPORTED;
  if (d->n_experts == 0 && d->ffn_dim > xrow_max) return PMK_ERR_UNSUPPORTED;
  if (d->n_experts > 0) {
    // a grouped-GEMM tile stages all of its kMoeBM rows at once
    const int moe_k_max = kXsBytes / (4 * kMoeBM) - 8;
    if (d->n_experts > kMaxExperts || d->top_k > kMaxTopK || d->expert_ffn_dim > moe_k_max ||
        d->hidden > moe_k_max || d->expert_ffn_dim < 16 || d->hidden < 16)
      return PMK_ERR_UNSUPPORTED;
  }
  return PMK_OK;
}


// Stage shapes the LDS holds: one input row of the whole depth and a tile's
// outputs (a step may put its few attention tasks on workgroups of their own
// and the QKV and O tiles on the others, at least three quarters of the
// grid); event offsets within the 27-bit keys of the persistent kernel's
// seen-event cache. (The split-K record regions are sized in dims_from_desc.)
int check_fit(const Dims& dm) {
  const int G = dm.grid;
  for (int st = 0; st < 4; ++st) {
    if (dm.moe && st >= 2) continue;
    int K, U, R;
    stage_dims(dm, st, K, U, R);
    const int tiles_min = std::min(st <= 1 ? G - G / 4 : G, U);
    const long row_bytes = 4L * (ceil_div(K, dm.kstep) * dm.kstep + dm.xpad);
    if (row_bytes + 16 + 4L * ceil_div(U, tiles_min) * R > kXyBytes) return PMK_ERR_UNSUPPORTED;
  }
  if ((long)dm.L * ev_layer_ints(dm) >= (1L << 27)) return PMK_ERR_UNSUPPORTED;
  return PMK_OK;
}

// The workspace carved from `base` in 256-byte aligned parts (base nullptr:
// sizes only). Returns the bytes it takes, or 0 when a part (a layer's slice
// of a per-layer part) reaches 1 GiB: step intermediates are addressed with
// 32-bit byte offsets from one buffer base and stay below the kernels'
// out-of-range marker offset.
size_t carve(const Dims& dm, Workspace& ws, char* base) {
  struct Part { void** p; size_t bytes, per_layer; };
  Part parts[48];
  int n = 0;
  auto add = [&](void* p, size_t bytes, size_t per_layer = 0) { parts[n++] = Part{(void**)p, bytes, per_layer}; };
  const size_t B = (size_t)dm.max_batch, qkv_dim = (size_t)(dm.Hq + 2 * dm.Hkv) * dm.d, Gq = dm.Hq / dm.Hkv;
  const size_t TK = B * std::max(dm.k, 1), F = std::max(dm.F, 1), mb = std::max(dm.merge_b, 1);
  add(&ws.qkv, dm.L * B * qkv_dim * 4, B * qkv_dim * 4);
  add(&ws.o, dm.L * B * dm.Hq * dm.d * 4, B * dm.Hq * dm.d * 4);
  add(&ws.h1, dm.L * B * dm.H * 4, B * dm.H * 4);
  add(&ws.act, dm.L * B * F * 4, B * F * 4);
  add(&ws.hid, (size_t)std::max(dm.L - 1, 1) * B * dm.H * 4, B * dm.H * 4);
  add(&ws.part, B * dm.Hkv * dm.max_chunks * Gq * (dm.d + 4) * 4);
  add(&ws.mpart, dm.L * mb * dm.Hkv * kMergeChunks * Gq * (dm.d + 4) * 4, mb * dm.Hkv * kMergeChunks * Gq * (dm.d + 4) * 4);
  add(&ws.rope, (size_t)dm.max_seq * (dm.d / 2) * 8);
  add(&ws.ev, (size_t)dm.L * ev_layer_ints(dm) * 4);
  add(&ws.mctr, dm.L * B * dm.Hkv * kCtr * 4);
  add(&ws.chunk_base, (B + 1) * 4);
  add(&ws.queue, (size_t)dm.grid * dm.max_queue * 16);
  add(&ws.qev, (size_t)dm.grid * dm.max_queue * 16);
  add(&ws.qlen, (size_t)dm.grid * 4);
  add(&ws.err, 64 * 4);
  add(&ws.args, sizeof(StepArgs));
  add(&ws.kpart, (size_t)dm.kpart_off[4] * 4);
  add(&ws.tctr, (size_t)4 * dm.tctr_stride * kCtr * 4);
  add(&ws.bar, (size_t)dm.L * kMaxStages * kEvInts * 4);
  add(&ws.u, B * dm.H * 4);
  if (dm.moe) {
    add(&ws.logits, B * dm.E * 4);
    add(&ws.topk_idx, TK * 4);
    add(&ws.topk_w, TK * 4);
    add(&ws.exp_indptr, (size_t)(dm.E + 1) * 4);
    add(&ws.sorted_tok, TK * 4);
    add(&ws.sorted_slot, TK * 4);
    add(&ws.pos_of, TK * 4);
    add(&ws.tile_info, (size_t)dm.max_tiles * 2 * 4);
    add(&ws.moe_info, 64 * 4);
    add(&ws.ectr, (size_t)dm.L * dm.E * kCtr * 4);
    add(&ws.tile_ptr, (size_t)(dm.E + 1) * 4);
    add(&ws.rq, (size_t)dm.L * dm.max_down * 4);
    add(&ws.mq, (size_t)dm.L * kMq * kCtr * 4);
    add(&ws.mact, dm.L * TK * dm.Fe * 4, TK * dm.Fe * 4);
    add(&ws.mout, TK * dm.H * 4);
  }
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    if ((parts[i].per_layer ? parts[i].per_layer : parts[i].bytes) >= ((size_t)1 << 30)) return 0;
    if (base) *parts[i].p = base + off;
    off += align256(parts[i].bytes);
  }
  return off;
}


// ---------------------------------------------------------------------------
// decode_step_static: the no-allocation entry point. Its workspace (the
// handle's, plus the RoPE table and the layer-pointer table) is carved from
// `scratch`, a file-scope device array each GPU holds for the life of the
// process; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device (the array's name in
// host code is a host-side stand-in, not a device address).
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_scratch[kMaxDevices];   // scratch's device address, per device
int g_static_grid[kMaxDevices];

// Set-up on the current device, once: scratch's address and the grid.
int static_setup(int dev, char** ptr, int* grid) {
  if (dev < 0 || dev >= kMaxDevices) return PMK_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PMK_ERR_DEVICE;
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 1)
      return PMK_ERR_DEVICE;
    g_static_grid[dev] = cu;
    g_scratch[dev] = p;
  }
  *ptr = (char*)g_scratch[dev];
  *grid = g_static_grid[dev];
  return PMK_OK;
}

// The error word and abort flag cleared, and the caller's status word.
__global__ void static_clear(int* err, int32_t* status) {
  err[threadIdx.x] = 0;
  if (threadIdx.x == 0 && status) *status = 0;
}

// The RoPE table on the device, as decode_layer_init writes it on the host:
// angle p theta^(-2i/d) in double, cos and sin rounded to float.
__global__ void static_rope(float2* tab, int max_seq, int half, int d, double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= max_seq * half) return;
  const int p = idx / half, i = idx - p * half;
  const double phi = (double)p * pow(theta, -2.0 * i / (double)d);
  tab[idx] = make_float2((float)cos(phi), (float)sin(phi));
}

static_assert(sizeof(LayerPtrs) == sizeof(pmk_layer_weights), "the layer table is copied as the caller gives it");

}  // namespace

extern "C" {

const char* pmk_strerror(int s) {
  switch (s) {
    case PMK_OK: return "ok";
    case PMK_ERR_ARG: return "invalid argument";
    case PMK_ERR_OOM: return "device allocation failed";
    case PMK_ERR_DEVICE: return "HIP runtime call failed";
    case PMK_ERR_TIMEOUT: return "an event wait exceeded the watchdog; the step was abandoned";
    case PMK_ERR_SEQ: return "a request length is outside [0, max_seq); the step did not run";
    case PMK_ERR_SCRATCH:
      return "the model's workspace exceeds the 64 MiB static scratch of decode_step_static (fewer layers, a "
             "smaller max_batch or max_seq)";
    case PMK_ERR_UNSUPPORTED:
      return "shape not implemented: needs head_dim*sizeof(dtype) == 256, Hq/Hkv in {1,2,4,8}, Hkv <= 128, max_batch <= 1024, "
             "GEMV depths that fit one LDS input row, and for MoE E <= 512, top_k <= 8, H and Fe small enough "
             "for 16 staged rows; the tile weight layout needs bfloat16, H, Hq d, F and Fe multiples of 32, "
             "(Hq + 2 Hkv) d and E multiples of 16";
    default: return "unknown status";
  }
}

int decode_layer_init(const pmk_model_desc* desc, const pmk_weights* w, pmk_handle** out) {
  if (!out) return PMK_ERR_ARG;
  *out = nullptr;
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!w || w->n_layers != desc->n_layers || !w->layers) return PMK_ERR_ARG;
  const bool moe = desc->n_experts > 0;
  for (int l = 0; l < desc->n_layers; ++l) {
    const pmk_layer_weights& L = w->layers[l];
    if (!L.attn_norm || !L.w_qkv || !L.w_o || !L.ffn_norm) return PMK_ERR_ARG;
    if (!moe && (!L.w_gate || !L.w_up || !L.w_down)) return PMK_ERR_ARG;
    if (moe && (!L.w_router || !L.w_exp_gate || !L.w_exp_up || !L.w_exp_down)) return PMK_ERR_ARG;
  }
  pmk_handle* h = new (std::nothrow) pmk_handle();
  if (!h) return PMK_ERR_OOM;
  h->desc = *desc;
  if (hipGetDevice(&h->device) != hipSuccess) { delete h; return PMK_ERR_DEVICE; }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, h->device) != hipSuccess) { delete h; return PMK_ERR_DEVICE; }

  Dims& dm = h->dm;
  dm = dims_from_desc(*desc, prop.multiProcessorCount);
  rc = check_fit(dm);
  if (rc) { delete h; return rc; }
  Workspace& ws = h->ws;
  const size_t total = carve(dm, ws, nullptr);
  if (total == 0) { delete h; return PMK_ERR_ARG; }
  void* base = nullptr;
  if (hipMalloc(&base, total) != hipSuccess) { delete h; return PMK_ERR_OOM; }
  h->ws_base = base;
  h->ws_bytes = total;
  (void)carve(dm, ws, (char*)base);
  auto fail = [&](int code) {
    decode_layer_destroy(h);
    return code;
  };
  if (hipMemset(base, 0, total) != hipSuccess) return fail(PMK_ERR_DEVICE);
  // the device writes a detected error here as well, so that the next call
  // can return it without waiting for the stream
  if (hipHostMalloc((void**)&h->err_host, 64, hipHostMallocCoherent) != hipSuccess) {
    h->err_host = nullptr;
    return fail(PMK_ERR_OOM);
  }
  *(volatile int*)h->err_host = 0;
  ws.err_host = h->err_host;

  // RoPE table: angle pos * theta^(-2i/d) in double, cos/sin rounded to float
  {
    const int half = dm.d / 2;
    std::vector<float> tab((size_t)dm.max_seq * half * 2);
    for (int p = 0; p < dm.max_seq; ++p)
      for (int i = 0; i < half; ++i) {
        const double phi = (double)p * std::pow((double)desc->rope_theta, -2.0 * i / (double)dm.d);
        tab[((size_t)p * half + i) * 2] = (float)std::cos(phi);
        tab[((size_t)p * half + i) * 2 + 1] = (float)std::sin(phi);
      }
    if (hipMemcpy(ws.rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
      return fail(PMK_ERR_DEVICE);
  }
  // layer pointer table
  {
    std::vector<LayerPtrs> lp(dm.L);
    for (int l = 0; l < dm.L; ++l) {
      const pmk_layer_weights& L = w->layers[l];
      lp[l] = LayerPtrs{L.attn_norm, L.w_qkv, L.w_o, L.ffn_norm, L.w_gate, L.w_up, L.w_down,
                        L.w_router, L.w_exp_gate, L.w_exp_up, L.w_exp_down};
    }
    if (hipMalloc(&h->d_layers, sizeof(LayerPtrs) * dm.L) != hipSuccess) return fail(PMK_ERR_OOM);
    if (hipMemcpy(h->d_layers, lp.data(), sizeof(LayerPtrs) * dm.L, hipMemcpyHostToDevice) != hipSuccess)
      return fail(PMK_ERR_DEVICE);
  }
  // a valid argument block from the start (each step's prologue rewrites it)
  {
    StepArgs a0{};
    a0.dm = dm;
    a0.ws = ws;
    a0.layers = h->d_layers;
    a0.attn_chunk = kMaxChunk;
    a0.qkv_tiles = dm.qkv_tiles;
    a0.geo[0] = StageGeo{1, dm.qkv_tiles, dm.H, 1};
    a0.geo[1] = StageGeo{1, dm.o_tiles, dm.Hq * dm.d, 1};
    a0.geo[2] = StageGeo{1, std::max(dm.gu_tiles, 1), dm.H, 1};
    a0.geo[3] = StageGeo{1, std::max(dm.down_tiles, 1), std::max(dm.F, 1), 1};
    if (hipMemcpy(ws.args, &a0, sizeof(a0), hipMemcpyHostToDevice) != hipSuccess) return fail(PMK_ERR_DEVICE);
  }
  if (prepare_main(desc->dtype, dm.wtiles) != hipSuccess) return fail(PMK_ERR_DEVICE);
  const int wd = desc->watchdog_ms > 0 ? desc->watchdog_ms : 2000;
  h->watchdog_ticks = (unsigned long long)wd * 100000ull;   // s_memrealtime: 100 MHz
  h->watchdog_init = h->watchdog_ticks;
  *out = h;
  return PMK_OK;
}

static int run_step(pmk_handle* h, float* hidden, void* kv, const int32_t* seq_lens, int32_t batch,
                    const pmk_routing* rout, void* stream) {
  if (!h || !hidden || !kv || !seq_lens) return PMK_ERR_ARG;
  if (batch < 1 || batch > h->dm.max_batch) return PMK_ERR_ARG;
  // a device error of an earlier step that has reached the host mirror: the
  // step would be skipped on the device anyway
  const int pending = *(volatile int*)h->err_host;
  if (pending != 0) return pending;
  hipStream_t s = (hipStream_t)stream;
  StepArgs a{};
  a.dm = h->dm;
  a.ws = h->ws;
  a.layers = h->d_layers;
  a.hidden = hidden;
  a.kv = kv;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.qkv_tiles = h->dm.qkv_tiles;
  a.watchdog_ticks = h->watchdog_ticks;
  if (rout) a.rout = *rout;
  a.trace = h->trace;
  a.trace_cap = h->trace_cap;
  a.barrier = h->sched == PMK_SCHED_BARRIER;
  a.per_op = h->sched == PMK_SCHED_PER_OP;
  a.ev_mode = h->ev_mode;
  a.moe_dyn = !h->dm.moe ? 0 : h->moe_sched == PMK_MOE_DYNAMIC ? 1 : h->moe_sched == PMK_MOE_DYNAMIC_XCD ? 2 : 0;
  h->last_stream = s;
  if (launch_prologue(a, s) != hipSuccess) return PMK_ERR_DEVICE;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (h->timing) {
    if (h->tused == h->tev.size()) {
      hipEvent_t x, y;
      if (hipEventCreate(&x) != hipSuccess || hipEventCreate(&y) != hipSuccess) return PMK_ERR_DEVICE;
      h->tev.emplace_back(x, y);
    }
    e0 = h->tev[h->tused].first;
    e1 = h->tev[h->tused].second;
    ++h->tused;
    if (hipEventRecord(e0, s) != hipSuccess) return PMK_ERR_DEVICE;
  }
  const int L = h->dm.L;
  if (h->sched == PMK_SCHED_FUSED || h->sched == PMK_SCHED_BARRIER) {
    if (launch_main(a, h->desc.dtype, s, RunSpec{0, L, kAllTypes, a.barrier}) != hipSuccess) return PMK_ERR_DEVICE;
  } else {
    // the stages of a layer, in queue order; a per-layer schedule runs them all in one launch
    auto bit = [](int t) { return 1u << t; };
    std::vector<unsigned> stages = {bit(T_QKV), bit(T_ATTN) | bit(T_ATTS), bit(T_O)};
    if (h->dm.moe)
      for (int t : {T_ROUTER, T_ROUTE, T_MGU, T_MDOWN, T_COMBINE}) stages.push_back(bit(t));
    else
      for (int t : {T_GU, T_DOWN}) stages.push_back(bit(t));
    if (h->sched == PMK_SCHED_PER_LAYER) stages = {kAllTypes};
    if (h->sched == PMK_SCHED_PER_OP)   // ten operators per layer, each a launch of its own
      stages = {bit(T_NORM1), bit(T_QKV), bit(T_ROPE), bit(T_APPEND), bit(T_ATTN), bit(T_MERGE), bit(T_O),
                bit(T_NORM2), bit(T_GU), bit(T_DOWN)};
    for (int l = 0; l < L; ++l)
      for (unsigned types : stages)
        if (launch_main(a, h->desc.dtype, s, RunSpec{l, l + 1, types, 0}) != hipSuccess) return PMK_ERR_DEVICE;
  }
  if (e1 && hipEventRecord(e1, s) != hipSuccess) return PMK_ERR_DEVICE;
  return PMK_OK;
}

int pmk_set_moe_scheduler(pmk_handle* h, int32_t mode) {
  if (!h || mode < PMK_MOE_STATIC || mode > PMK_MOE_DYNAMIC_XCD) return PMK_ERR_ARG;
  h->moe_sched = mode;
  return PMK_OK;
}

int pmk_set_event_granularity(pmk_handle* h, int32_t mode) {
  if (!h || mode < PMK_EVENTS_TILE || mode > PMK_EVENTS_STAGE) return PMK_ERR_ARG;
  h->ev_mode = mode;
  return PMK_OK;
}

int pmk_set_schedule(pmk_handle* h, int32_t mode) {
  if (!h || mode < PMK_SCHED_FUSED || mode > PMK_SCHED_PER_OP)
    return PMK_ERR_ARG;
  if (mode == PMK_SCHED_PER_OP && h->dm.moe) return PMK_ERR_UNSUPPORTED;
  h->sched = mode;
  return PMK_OK;
}

int decode_step(pmk_handle* h, float* hidden, void* kv_cache, const int32_t* seq_lens, int32_t batch, void* stream) {
  return run_step(h, hidden, kv_cache, seq_lens, batch, nullptr, stream);
}

int decode_step_static(const pmk_model_desc* desc, const pmk_weights* w, float* hidden, void* kv_cache,
                       const int32_t* seq_lens, int32_t batch, int32_t* status, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (desc->n_experts > 0) return PMK_ERR_UNSUPPORTED;   // dense stacks only
  if (!w || w->n_layers != desc->n_layers || !w->layers || !hidden || !kv_cache || !seq_lens) return PMK_ERR_ARG;
  if (batch < 1 || batch > desc->max_batch) return PMK_ERR_ARG;
  for (int l = 0; l < desc->n_layers; ++l) {
    const pmk_layer_weights& L = w->layers[l];
    if (!L.attn_norm || !L.w_qkv || !L.w_o || !L.ffn_norm || !L.w_gate || !L.w_up || !L.w_down) return PMK_ERR_ARG;
  }
  int dev = 0, grid = 0;
  char* base = nullptr;
  if (hipGetDevice(&dev) != hipSuccess) return PMK_ERR_DEVICE;
  rc = static_setup(dev, &base, &grid);
  if (rc) return rc;
  const Dims dm = dims_from_desc(*desc, grid);
  rc = check_fit(dm);
  if (rc) return rc;
  Workspace ws{};
  const size_t wbytes = carve(dm, ws, nullptr);
  const size_t lbytes = align256(sizeof(LayerPtrs) * dm.L);
  // (a part of 1 GiB or more, carve's 0, is far beyond the scratch as well)
  if (wbytes == 0 || wbytes + lbytes > kStaticScratchBytes) return PMK_ERR_SCRATCH;
  (void)carve(dm, ws, base);
  LayerPtrs* layers = reinterpret_cast<LayerPtrs*>(base + wbytes);
  ws.err_host = status;   // the kernels copy a device error here
  hipStream_t s = (hipStream_t)stream;
  if (prepare_main(desc->dtype, dm.wtiles) != hipSuccess) return PMK_ERR_DEVICE;
  hipLaunchKernelGGL(static_clear, dim3(1), dim3(64), 0, s, ws.err, status);
  const int half = dm.d / 2, nrope = dm.max_seq * half;
  hipLaunchKernelGGL(static_rope, dim3((nrope + 255) / 256), dim3(256), 0, s, reinterpret_cast<float2*>(ws.rope),
                     dm.max_seq, half, dm.d, (double)desc->rope_theta);
  if (hipGetLastError() != hipSuccess) return PMK_ERR_DEVICE;
  if (hipMemcpyAsync(layers, w->layers, sizeof(LayerPtrs) * dm.L, hipMemcpyHostToDevice, s) != hipSuccess)
    return PMK_ERR_DEVICE;
  StepArgs a{};
  a.dm = dm;
  a.ws = ws;
  a.layers = layers;
  a.hidden = hidden;
  a.kv = kv_cache;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.qkv_tiles = dm.qkv_tiles;
  a.watchdog_ticks = (unsigned long long)(desc->watchdog_ms > 0 ? desc->watchdog_ms : 2000) * 100000ull;
  a.ev_mode = PMK_EVENTS_GROUP;
  if (launch_prologue(a, s) != hipSuccess) return PMK_ERR_DEVICE;
  if (launch_main(a, desc->dtype, s, RunSpec{0, dm.L, kAllTypes, 0}) != hipSuccess) return PMK_ERR_DEVICE;
  return PMK_OK;
}

int moe_layer_step(pmk_handle* h, float* hidden, void* kv_cache, const int32_t* seq_lens, int32_t tokens,
                   const pmk_routing* routing, void* stream) {
  if (!h) return PMK_ERR_ARG;
  if (!h->dm.moe) return PMK_ERR_ARG;
  return run_step(h, hidden, kv_cache, seq_lens, tokens, routing, stream);
}

int decode_layer_destroy(pmk_handle* h) {
  if (!h) return PMK_OK;
  int rc = PMK_OK;
  if (hipDeviceSynchronize() != hipSuccess) rc = PMK_ERR_DEVICE;
  for (auto& p : h->tev) {
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  if (h->d_layers) (void)hipFree(h->d_layers);
  if (h->ws_base) (void)hipFree(h->ws_base);
  if (h->err_host) (void)hipHostFree(h->err_host);
  delete h;
  return rc;
}

int pmk_set_watchdog_us(pmk_handle* h, int32_t us) {
  if (!h || us < 0) return PMK_ERR_ARG;
  h->watchdog_ticks = us == 0 ? h->watchdog_init : (unsigned long long)us * 100ull;
  return PMK_OK;
}

int pmk_pack_weights(const void* src, void* dst, int64_t rows, int64_t cols, void* stream) {
  if (!src || !dst || rows <= 0 || cols <= 0 || rows % 16 || cols % 32) return PMK_ERR_ARG;
  if (rows > INT64_MAX / 2 / cols) return PMK_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return PMK_ERR_ARG;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t n = (uintptr_t)(rows * cols * 2);
  if (s < d + n && d < s + n) return PMK_ERR_ARG;   // the two must not overlap
  if (launch_pack(src, dst, rows, cols, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return PMK_ERR_DEVICE;
  return PMK_OK;
}

int pmk_get_device_error(pmk_handle* h) {
  if (!h) return PMK_ERR_ARG;
  if (hipStreamSynchronize(h->last_stream) != hipSuccess) return PMK_ERR_DEVICE;
  int e = 0;
  if (hipMemcpy(&e, h->ws.err, 4, hipMemcpyDeviceToHost) != hipSuccess) return PMK_ERR_DEVICE;
  if (e != 0 && hipMemset(h->ws.err, 0, 64 * 4) != hipSuccess) return PMK_ERR_DEVICE;
  if (hipDeviceSynchronize() != hipSuccess) return PMK_ERR_DEVICE;
  *(volatile int*)h->err_host = 0;
  return e;
}

int pmk_query(const pmk_handle* h, pmk_info* out) {
  if (!h || !out) return PMK_ERR_ARG;
  std::memset(out, 0, sizeof(*out));
  out->grid = h->dm.grid;
  out->block = kBlock;
  out->lds_bytes = kLdsBytes;
  out->moe_bm = kMoeBM;
  out->attn_chunk = kMaxChunk;
  out->max_queue = h->dm.max_queue;
  out->workspace_bytes = (int64_t)h->ws_bytes;
  out->arch = 950;
  return PMK_OK;
}

int pmk_trace_attach(pmk_handle* h, uint32_t* buf, int32_t entries_per_wg) {
  if (!h) return PMK_ERR_ARG;
  if (buf && entries_per_wg < 2) return PMK_ERR_ARG;
  h->trace = buf;
  h->trace_cap = buf ? entries_per_wg : 0;
  return PMK_OK;
}

int pmk_timing_enable(pmk_handle* h, int enable) {
  if (!h) return PMK_ERR_ARG;
  if (h->tused && hipStreamSynchronize(h->last_stream) != hipSuccess) return PMK_ERR_DEVICE;
  h->timing = enable != 0;
  h->tused = 0;
  return PMK_OK;
}

int pmk_timing_read(pmk_handle* h, double* total_ms, int32_t* launches) {
  if (!h || !total_ms || !launches) return PMK_ERR_ARG;
  double sum = 0.0;
  for (size_t i = 0; i < h->tused; ++i) {
    if (hipEventSynchronize(h->tev[i].second) != hipSuccess) return PMK_ERR_DEVICE;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, h->tev[i].first, h->tev[i].second) != hipSuccess) return PMK_ERR_DEVICE;
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int32_t)h->tused;
  return PMK_OK;
}

}  // extern "C"
