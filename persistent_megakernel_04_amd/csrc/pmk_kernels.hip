// pmk_kernels.hip -- the per-step prologue and the persistent decode kernel.
//
// One decode step = two launches on the caller's stream:
//  1. pmk_prologue (one workgroup): reads (batch, seq_lens) on the device,
//     checks every length, picks the attention chunk size, writes each
//     persistent workgroup's task queue for one layer, and arms every event
//     counter of every layer. This is the runtime instantiation of a dependency
//     template whose batch and length dimensions are symbolic (Event Tensor
//     summary, Core method, two kinds of dynamism: shape dynamism), so a new
//     batch size or new lengths need no recompilation.
//  2. pmk_main (one workgroup per compute unit, cooperative launch so that all
//     are co-resident): every workgroup replays its queue for layer 0, 1, ...,
//     waiting on the events its tasks consume and notifying the events they
//     produce (same page, Core method, Event Tensor abstraction and ETC
//     compiler and scheduling: static scheduling with per-SM queues and a
//     persistent main loop). Each task issues the loads of its weights (or KV
//     entries) before it waits on its input event (same page, the optional
//     weight-prefetch pass), so HBM keeps streaming across dependencies.
//
// MoE layers (same page, Key observations, observation 2, and Core method, two
// kinds of dynamism: data-dependent events) run attention, then router logits,
// then one workgroup's top-k + grouping (which fills exp_indptr and the tile
// list and arms one counter per expert with that expert's gate/up task count),
// then grouped gate/up tasks that each notify their expert's counter, grouped
// down tasks that wait on their expert's counter, and a per-token combine.
//
// Deadlock freedom: each queue lists its tasks in stage order and every task
// only waits on events produced by earlier stages of the same layer or by the
// previous layer. All workgroups are resident, so by induction on (layer,
// stage) the earliest unfinished stage always has all its producers done. Every
// wait is bounded by a watchdog; on expiry the step is abandoned (error word +
// abort flag), so every wave exits.
#include "pmk_device.h"
#include "pmk_sched.h"

namespace pmk {

// ---------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------
struct Lds {
  void* xs;        // the xy region: a GEMV pass's input rows (MM<WT>::XT) then its outputs
                   // [R][nb] (see Pass::ys); attention and routing scratch
  float* red;      // cross-wave partial sums
  float* rstd;     // [kMaxNb] 1/rms of the staged rows
  float* ssp;      // [kMaxNb][kWaves] per-wave partial sums of squares
  int* flag;       // wait / last-arriver broadcast
  uint32_t* tclk;  // [8] phase clocks of the current task (trace): see the trace record layout
  int* seen;       // [8] per wait kind, the event offset this workgroup last saw fired (+ 1; 0: none)
  int* rope_key;   // [3] the QKV pass whose rotation rows rope holds: first unit + 1, first request, elements 32 + nb
  int* rope_pos;   // [kMaxNb] its requests' positions
  float2* rope;    // [kRopeBytes / 8] its (cos, sin) per element
};

__device__ __forceinline__ Lds lds_layout(char* base) {
  Lds s;
  s.xs = base;
  s.red = reinterpret_cast<float*>(base + kXyBytes);
  char* m = base + kXyBytes + kRedBytes;
  s.rstd = reinterpret_cast<float*>(m);                   // 16 floats
  s.ssp = reinterpret_cast<float*>(m + 64);               // 128 floats
  s.flag = reinterpret_cast<int*>(m + 64 + 512);          // 1 int
  s.tclk = reinterpret_cast<uint32_t*>(m + 64 + 512 + 16);   // 8 clocks
  s.seen = reinterpret_cast<int*>(m + 64 + 512 + 16 + 32);   // 8 ints
  s.rope_key = reinterpret_cast<int*>(m + 64 + 512 + 16 + 32 + 32);   // 4 ints
  s.rope_pos = reinterpret_cast<int*>(m + 64 + 512 + 16 + 32 + 48);   // 16 ints
  s.rope = reinterpret_cast<float2*>(m + kMiscBytes);
  return s;
}

struct Ctx {
  const StepArgs& a;
  int l, wg;
  Lds s;
  int* nev = nullptr;   // the counter this task notifies (attention: the request's group), resolved for layer l
};

// Per-layer activations. Each buffer is written once per step, by the stage
// that produces it, and read only after that stage's event; a reader's L2
// therefore never holds an older copy of its lines (the L2s are invalidated
// at every kernel start), and the staged reads use ordinary cached loads, so
// the workgroups of an XCD share one fetch of a row through their L2. The
// stack's input is the caller's hidden (layer 0 reads it) and its output goes
// back there (the last layer writes it).
__device__ __forceinline__ float* qkv_of(const StepArgs& a, int l) {
  return a.ws.qkv + (size_t)l * a.dm.max_batch * (a.dm.Hq + 2 * a.dm.Hkv) * a.dm.d;
}
__device__ __forceinline__ float* o_of(const StepArgs& a, int l) {
  return a.ws.o + (size_t)l * a.dm.max_batch * a.dm.Hq * a.dm.d;
}
__device__ __forceinline__ float* h1_of(const StepArgs& a, int l) { return a.ws.h1 + (size_t)l * a.dm.max_batch * a.dm.H; }
__device__ __forceinline__ float* act_of(const StepArgs& a, int l) {
  return a.ws.act + (size_t)l * a.dm.max_batch * a.dm.F;
}
__device__ __forceinline__ float* mpart_of(const StepArgs& a, int l) {
  return a.ws.mpart + (size_t)l * a.dm.merge_b * a.dm.Hkv * kMergeChunks * (a.dm.Hq / a.dm.Hkv) * (a.dm.d + 4);
}
__device__ __forceinline__ float* mact_of(const StepArgs& a, int l) {
  return a.ws.mact + (size_t)l * a.dm.max_batch * a.dm.k * a.dm.Fe;
}
__device__ __forceinline__ const float* hid_in(const StepArgs& a, int l) {
  return l == 0 ? a.hidden : a.ws.hid + (size_t)(l - 1) * a.dm.max_batch * a.dm.H;
}
__device__ __forceinline__ float* hid_out(const StepArgs& a, int l) {
  return l == a.dm.L - 1 ? a.hidden : a.ws.hid + (size_t)l * a.dm.max_batch * a.dm.H;
}

// x / d for a wave-uniform d > 0 and 0 <= x with x d < 2^32, by one
// multiply-high: with m = floor(2^32 / d) + 1 = (2^32 + e) / d, 0 < e <= d,
// x m / 2^32 = x / d + x e / (d 2^32), and the second term is below 1 / d,
// too small to carry x / d past the next integer.
// (d = 1: m wraps to 0 and `keep` adds x back, without a branch)
struct UDiv {
  uint32_t m, keep;
  __device__ __forceinline__ explicit UDiv(int d)
      : m(0xffffffffu / (uint32_t)d + 1u), keep(d == 1 ? 0xffffffffu : 0u) {}
  __device__ __forceinline__ int div(int x) const {
    return (int)(__umulhi((uint32_t)x, m) + ((uint32_t)x & keep));
  }
};

__device__ __forceinline__ size_t kv_off(const Dims& dm, int l, int which, int b, int g, int pos) {
  return (((((size_t)l * 2 + which) * dm.max_batch + b) * dm.Hkv + g) * (size_t)dm.max_seq + pos) * dm.d;
}

// Wait on an event (its [0] and kSubs sub-counters) or, with subs = 0, on a
// bare counter. Always a workgroup barrier, also with no event: every task
// begins with one before it writes LDS, since wave 0 may still be reading the
// previous GEMV pass's results in LDS when the other waves start the task.
__device__ __forceinline__ bool ctx_wait(const Ctx& c, const int* ev, int subs = kSubs) {
  if (!ev) {
    __syncthreads();
    return true;
  }
  const bool ok = wg_wait(ev, subs, c.a.ws.err, c.a.watchdog_ticks, c.s.flag);
  if (threadIdx.x == 0) c.s.tclk[1] = (uint32_t)now_ticks();
  return ok;
}

// ---------------------------------------------------------------------------
// The weight-streaming GEMV tile engine.
//
//   ys[j][m] = sum_k W[row(j)][k] * xs[m][k],  j < R, m < nb <= 16,
//   xs[m] = src row m (or src row gather[m]) * gain, rounded to the MFMA input
//   type; with `norm`, rstd[m] = 1 / sqrt(mean src[m]^2 + eps) (RMSNorm folded
//   into the GEMV: the epilogue multiplies by rstd).
//
// The R rows form RG = ceil(R / 16) row groups. Each wave streams its work
// items (row group x k range) row-group-major as 16-byte-per-lane loads (16
// rows x 64 contiguous bytes per load instruction, consecutive instructions
// walking along the same rows) through a register ring of 16 loads (16 KiB per
// wave). The ring is filled before the input event is awaited and refilled as
// it is consumed, flowing from one item into the next. Partial sums of waves
// that share a row group are added in LDS in wave order (deterministic).
// ---------------------------------------------------------------------------
enum RowMode : int { ROWS_CONTIG = 0, ROWS_QKV = 1, ROWS_PAIR = 2 };

struct GemvRows {
  int mode;
  const void* base;    // the matrix (CONTIG, QKV) or the first matrix (PAIR)
  const void* base2;   // PAIR: the second matrix
  int r0;              // CONTIG/PAIR: first row; QKV: first rotation unit
  int half;            // PAIR: rows taken from each matrix; QKV: head_dim / 2
  int ld;              // row stride of the matrix (elements)
  int k0;              // first column of the pass (a K slice)
  int qg, qh;          // QKV: query heads per KV group, query heads
};

// The rotation unit at group-major position `up` (qkv_unit of pmk_sched.h,
// from the fields a QKV pass carries).
__device__ __forceinline__ int qkv_unit_r(const GemvRows& rw, int up) {
  const int half = rw.half, G = rw.qg, per = (G + 2) * half, g = up / per, r = up - g * per;
  if (r < G * half) return g * G * half + r;
  if (r < (G + 1) * half) return rw.qh * half + g * half + (r - G * half);
  return (rw.qh + rw.qh / G) * half + g * half + (r - (G + 1) * half);
}

// Where row `row` of a weight matrix with `ld` columns starts at column k0:
// row-major, or (PK) in the tile layout: the matrix cut into 16-row x
// 32-column tiles, stored one after another (row group major), each tile
// row-major, so that one wave-wide load of a k-step reads a contiguous 1 KiB
// tile. For PK the returned pointer is that of the row's first 8 elements in
// the tile of column k0; a step advances it by one tile (512 elements).
template <typename WT, bool PK>
__device__ __forceinline__ const WT* wrow(const void* base, size_t row, int ld, int k0) {
  const WT* b = reinterpret_cast<const WT*>(base);
  if (PK) return b + (row >> 4) * 16 * (size_t)ld + (row & 15) * 32 + (size_t)(k0 >> 5) * 512;
  return b + row * ld + k0;
}

template <typename WT, bool PK>
__device__ __forceinline__ const WT* row_ptr(const GemvRows& rw, int j) {
  if (rw.mode == ROWS_QKV) {
    // local row 2u is (head h, i), 2u + 1 is (h, i + d/2): the two rows of a
    // rotation pair; units in KV-group-major order (qkv_unit)
    const int unit = qkv_unit_r(rw, rw.r0 + (j >> 1)), h = unit / rw.half, i = unit - h * rw.half;
    return wrow<WT, PK>(rw.base, (size_t)(h * 2 * rw.half + i + (j & 1) * rw.half), rw.ld, rw.k0);
  }
  if (rw.mode == ROWS_PAIR && j >= rw.half) return wrow<WT, PK>(rw.base2, (size_t)(rw.r0 + j - rw.half), rw.ld, rw.k0);
  return wrow<WT, PK>(rw.base, (size_t)(rw.r0 + j), rw.ld, rw.k0);
}

struct GemvIn {
  const float* src;    // float32 rows (written this step by other workgroups: device-coherent loads)
  int ld;              // row stride (elements)
  const int* gather;   // nullable: staged row m <- src row gather[m] (device-coherent)
  const float* gain;   // nullable: elementwise gain (RMSNorm weight)
  int norm;            // 1: rstd[m] = 1 / rms of the staged rows; 2: leave their raw sum of squares
  float eps;
  int merge_b0;        // >= 0: the rows are the attention outputs of requests merge_b0.. (merged from partials)
};

// Stage nb input rows into LDS as the MFMA input type, rows XS apart (SPLIT:
// each row as a hi part and a lo part, XS apart, rows 2 XS apart), zero
// beyond K up to Kp; per-row sum of squares -> rstd (when in.norm). Each wave
// takes an eighth of the rows' 256-element blocks, contiguous, eight blocks
// at a time: their loads (and the gains') are issued together with no branch
// between them, so each one waits only for itself. A wave's sum of squares
// over each row it touches is one wave reduction into that wave's slot, and
// the 8 slots are summed in order. The sources are per-layer activations:
// cached loads.
template <typename WT, bool SPLIT>
__device__ __forceinline__ void stage_rows(const GemvIn& in, int nb, int K, int Kp, int XS, const Lds& s) {
  typedef typename MM<WT>::XT XT;
  XT* xs = reinterpret_cast<XT*>(s.xs);
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int BPR = (Kp + 255) >> 8, NBK = nb * BPR;
  const auto src = rsrc(in.src);
  // no gain: a descriptor with an empty range reads zeros, replaced by ones below
  const auto grs = rsrc_n(in.gain ? (const void*)in.gain : (const void*)in.src, in.gain ? K * 4 : 0);
  const bool has_gain = in.gain != nullptr;
  // gathered rows: lane m holds the source row of staged row m
  const int gidx = (in.gather && lane < nb) ? ldci(in.gather + lane) : lane;
  if (lane == 0)
    for (int m = 0; m < nb; ++m) s.ssp[m * kWaves + wave] = 0.f;
  // wave w stages the contiguous blocks [w NBK / 8, (w + 1) NBK / 8), one row
  // segment at a time: a lane sums its squares over the segment, and the
  // wave adds them up once per segment
  const int wb1 = (wave + 1) * NBK / kWaves;
  for (int s0 = wave * NBK / kWaves; s0 < wb1;) {
    const int m = s0 / BPR, s1 = min(wb1, (m + 1) * BPR);
    const int srow = __builtin_amdgcn_readlane(gidx, m);
    float ssq = 0.f;
    for (int base = s0; base < s1; base += 8) {
      f4v v[8], gv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int blk = min(base + u, s1 - 1);   // past the segment: a valid block, not used
        const int k = (blk - m * BPR) * 256 + lane * 4;
        const int kc = min(k, K - 4);            // beyond K: a valid element, zeroed below
        v[u] = ldk4(src, (srow * in.ld + kc) * 4);
        gv[u] = ldk4(grs, kc * 4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int blk = base + u;
        if (blk >= s1) continue;
        const int k = (blk - m * BPR) * 256 + lane * 4;
        f4v x = k < K ? v[u] : f4v{0.f, 0.f, 0.f, 0.f};
        ssq += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
        x *= has_gain ? gv[u] : f4v{1.f, 1.f, 1.f, 1.f};
        if (k < Kp) {
          if (SPLIT)
            MM<WT>::put4_split(xs + (size_t)m * 2 * XS + k, xs + (size_t)m * 2 * XS + XS + k, x);
          else
            MM<WT>::put4(xs + (size_t)m * XS + k, x);
        }
      }
    }
    if (in.norm) {
      const float ss = wave_sum(ssq);
      if (lane == 0) s.ssp[m * kWaves + wave] += ss;
    }
    s0 = s1;
  }
  __syncthreads();
  if (in.norm && threadIdx.x < nb) {
    float ss = 0.f;
    for (int w = 0; w < kWaves; ++w) ss += s.ssp[threadIdx.x * kWaves + w];
    s.rstd[threadIdx.x] = in.norm == 2 ? ss : 1.0f / sqrtf(ss / (float)K + in.eps);
  } else if (!in.norm && threadIdx.x < nb) {
    s.rstd[threadIdx.x] = 1.0f;   // rows normalised by an op of their own (per-op schedule): no scale
  }
  __syncthreads();
}

// Stage the O-projection inputs of nb requests by merging their attention
// chunk partials (acc, max, sum per query head; the chunk tasks wrote them and
// notified) by log-sum-exp: o = sum_c acc_c 2^(m_c - M) / sum_c l_c 2^(m_c - M).
// Used when every request has at most 8 chunks and each thread stages at most
// two 4-element units, so all partial loads of a thread are in flight at once.
// The partials are this layer's (written once in the step): cached loads.
template <typename WT, bool SP>
__device__ __forceinline__ void stage_attn_merge(const StepArgs& a, int l, const GemvIn& in, int nb, int K, int Kp,
                                                 int XS, const Lds& s) {
  typedef typename MM<WT>::XT XT;
  XT* xs = reinterpret_cast<XT*>(s.xs);
  const Dims& dm = a.dm;
  const int d = dm.d, G = dm.Hq / dm.Hkv, DP = d + 4, ck = a.attn_chunk;
  const int K4 = Kp / 4;   // 4-element units per row (K = Hq d, a multiple of 4; zero beyond K)
  // this layer's partials: written once in the step, so read through the caches
  const auto pr = rsrc_n(mpart_of(a, l), dm.merge_b * dm.Hkv * kMergeChunks * G * DP * 4);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int unit = threadIdx.x + u * kBlock;
    if (unit >= nb * K4) continue;
    const int m = unit / K4, k = (unit - m * K4) * 4;
    f4v x = {0.f, 0.f, 0.f, 0.f};
    if (k < K) {
      const int b = in.merge_b0 + m;
      // the request's chunk count: for one request through the scalar cache,
      // so that the partial loads below issue at once
      const int nc = ((nb == 1 ? ldku(a.seq_lens + in.merge_b0) : *gp(a.seq_lens + b)) + ck) / ck;
      const int h = k / d, e = k - h * d, g = h / G, hh = h - g * G;
      const int base = ((b * dm.Hkv + g) * kMergeChunks * G + hh) * DP;
      f4v av[kMergeChunks], mv[kMergeChunks];
#pragma unroll
      for (int cc = 0; cc < kMergeChunks; ++cc) {
        // a chunk the request does not have reads past the buffer's range:
        // zeros, with no memory access
        const int o = cc < nc ? (base + cc * G * DP) * 4 : kNoRecord;
        av[cc] = ldk4(pr, o + e * 4);
        mv[cc] = ldk4(pr, o + d * 4);
      }
      float M = -INFINITY, L = 0.f;
#pragma unroll
      for (int cc = 0; cc < kMergeChunks; ++cc)
        if (cc < nc) M = fmaxf(M, mv[cc].x);
#pragma unroll
      for (int cc = 0; cc < kMergeChunks; ++cc) {
        if (cc < nc) {
          const float f = exp2f(mv[cc].x - M);
          L += mv[cc].y * f;
          x += av[cc] * f;
        }
      }
      x = x / L;
    }
    if (SP)
      MM<WT>::put4_split(xs + (size_t)m * 2 * XS + k, xs + (size_t)m * 2 * XS + XS + k, x);
    else
      MM<WT>::put4(xs + (size_t)m * XS + k, x);
  }
  __syncthreads();
}

// One wave's share of a GEMV pass: work items (row group, k-step range)
// streamed one after another. Tiles of fewer than 8 row groups split each row
// group's k range over 8 / RG waves (their partial sums are added in LDS);
// tiles of 8 or more give each wave whole row groups rg, rg + 8, ...
constexpr int kRing = 16;   // weight loads in flight per wave (16 KiB; 128 KiB per workgroup)

struct WaveItems {
  int n;        // items of this wave
  int rg0;      // row group of the first item
  int rg_step;  // row group step between consecutive items
  int ks_lo;    // every item covers k-steps [ks_lo, ks_lo + nks)
  int nks;
  int sl;       // the wave's k slice (0 when waves own whole row groups)
};

// Waves per row group's k range. Fewer than 8 row groups: 8 / RG waves each,
// or, when that leaves waves idle (RG = 3, 5, 6, 7) and the partial sums fit
// the cross-wave buffer, every wave takes one eighth of the k range of every
// row group. 8 or more row groups: waves own whole row groups.
__device__ __forceinline__ int k_split(int RG, int nb) {
  if (RG >= kWaves) return 1;
  if (kWaves % RG != 0 && RG * kWaves * nb * 16 <= kRedBytes / 4) return kWaves;
  return kWaves / RG;
}

__device__ __forceinline__ WaveItems wave_items(int RG, int NKS, int nb, int wave) {
  WaveItems it;
  const int ks = k_split(RG, nb);
  // slices of whole ring lengths, so that no wave pads its range with
  // dummy steps (the last slice ends at NKS). Where they cannot be equal, the
  // first slices take one ring length more: they go to waves 0-3, the first
  // wave on each SIMD, which win the issue arbitration over the second ones
  // (traced: the last wave of a task to finish its share is always one of
  // waves 4-7, and with the extra lengths on odd waves the down projection's
  // tasks ended ~4 us after their first wave at batch 1).
  const int NB = (NKS + kRing - 1) / kRing;
  auto slice = [&](int sl) {
    it.sl = sl;
    const int q = NB / ks, r = NB - q * ks, b0 = sl * q + min(sl, r), b1 = b0 + q + (sl < r ? 1 : 0);
    it.ks_lo = min(b0 * kRing, NKS);
    it.nks = min(b1 * kRing, NKS) - it.ks_lo;
  };
  if (ks == 1) {
    it.n = wave < RG ? (RG - wave + kWaves - 1) / kWaves : 0;
    it.rg0 = wave;
    it.rg_step = kWaves;
    it.sl = 0;
    it.ks_lo = 0;
    it.nks = NKS;
  } else if (ks * RG > kWaves) {   // every wave: its slice of every row group
    it.n = RG;
    it.rg0 = 0;
    it.rg_step = 1;
    slice(wave);
  } else {
    const bool busy = wave < RG * ks;
    it.n = busy ? 1 : 0;
    it.rg0 = busy ? wave / ks : 0;
    it.rg_step = 0;
    slice(wave % ks);
  }
  return it;
}

// Returns false if the wait was abandoned (nothing was computed). SP: the
// input rows are carried as bfloat16 hi + lo pairs, two MFMAs per chunk.
//
// Each wave fills its ring before the input event is awaited, so its first
// kRing steps stream in during the wait; the ring then flows from one item of
// the wave into the next. Every item is streamed as a whole number of ring
// lengths (steps past its end multiply a zero input and re-read its last
// step), which keeps the slot of a step fixed; the last block of the pass
// issues no refills. (Carrying the ring on into the next pass, so that a
// pass's last steps prefetch the next one, was measured slower: the workgroups
// that finish a stage early then take HBM bandwidth from the ones that gate
// the stage's event.)
template <typename WT, bool SP, bool PK>
__device__ __forceinline__ bool gemv(const Ctx& c, const GemvRows& rw, int R, int K, const GemvIn& in, int nb,
                                     const int* wait_ev, int wait_subs, float* ys) {
  typedef MM<WT> T;
  typedef typename T::XT XT;
  constexpr int D = kRing;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), grp = lane >> 4, mrow = lane & 15;
  const int NKS = (K + T::KSTEP - 1) / T::KSTEP, RG = (R + 15) >> 4;
  const int Kp = NKS * T::KSTEP, XS = Kp + T::XPAD;
  const int kmax = K - T::EPL, kg = grp * T::EPL;
  const WaveItems wi = wave_items(RG, NKS, nb, wave);
  const int nks = wi.nks, nks_c = nks > 0 ? nks - 1 : 0;
  const int nks_pad = nks > D ? (nks + D - 1) / D * D : D;
  auto item_rows = [&](int it) -> const WT* {
    const int rg = min(wi.rg0 + min(it, max(wi.n - 1, 0)) * wi.rg_step, RG - 1);
    return row_ptr<WT, PK>(rw, min(rg * 16 + mrow, R - 1));   // padded rows repeat a valid row
  };
  auto kofs = [&](int ks) {
    if constexpr (PK) return min(wi.ks_lo + ks, NKS - 1) * 512 + kg;
    else return min((wi.ks_lo + ks) * T::KSTEP + kg, kmax);
  };
  auto ldw = [&](const WT* p) {
    if constexpr (PK) return ldg16_nt(p);
    else return ldg16(p);
  };

  uint4 ring[D];
  const WT* cur = item_rows(0);
  const WT* nxt = item_rows(1);
  if (wi.n > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) ring[d] = ldw(cur + kofs(min(d, nks_c)));
  }
  if (!ctx_wait(c, wait_ev, wait_subs)) return false;
  if (in.merge_b0 >= 0)
    stage_attn_merge<WT, SP>(c.a, c.l, in, nb, K, Kp, XS, c.s);
  else
    stage_rows<WT, SP>(in, nb, K, Kp, XS, c.s);
  if (tid == 0) c.s.tclk[2] = (uint32_t)now_ticks();

  const XT* xrow = reinterpret_cast<const XT*>(c.s.xs) + (size_t)(mrow < nb ? mrow : 0) * (SP ? 2 : 1) * XS +
                   wi.ks_lo * T::KSTEP + kg;
  const bool xon = mrow < nb;
  const int KSPL = k_split(RG, nb);
  for (int it = 0; it < wi.n; ++it) {
    const bool has_next = it + 1 < wi.n;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    // the input fragments of the next k-step are read from LDS one step ahead
    uint4 xa_n = *reinterpret_cast<const uint4*>(xrow), xl_n = make_uint4(0, 0, 0, 0);
    if (SP) xl_n = *reinterpret_cast<const uint4*>(xrow + XS);
    // one k-step: the input fragment (zero past the item, or for a row >= nb)
    // times weights w, reading the next step's fragment ahead
    auto step = [&](int ks, const uint4 w) {
      const bool on = xon && ks < nks;
      uint4 xa = xa_n, xl = xl_n;
      const int xo = min(ks + 1, nks_c) * T::KSTEP;
      xa_n = *reinterpret_cast<const uint4*>(xrow + xo);
      if (SP) xl_n = *reinterpret_cast<const uint4*>(xrow + XS + xo);
      xa.x = on ? xa.x : 0u;
      xa.y = on ? xa.y : 0u;
      xa.z = on ? xa.z : 0u;
      xa.w = on ? xa.w : 0u;
      acc = T::mac(xa, w, acc);
      if (SP) {
        xl.x = on ? xl.x : 0u;
        xl.y = on ? xl.y : 0u;
        xl.z = on ? xl.z : 0u;
        xl.w = on ? xl.w : 0u;
        acc = T::mac(xl, w, acc);
      }
    };
    // Branch-free blocks, so the compiler's wait counts stay exact (a branch
    // here makes it wait for every load in flight before each MFMA).
    const int nrefill = has_next ? nks_pad : nks_pad - D;   // the last block of the pass refills nothing
    for (int ks0 = 0; ks0 < nrefill; ks0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int ks = ks0 + d;
        step(ks, ring[d]);
        // refill with the step kRing ahead: of this item, else of the next item
        const int nk = ks + D;
        const bool here = nk < nks_pad;
        ring[d] = ldw((here ? cur : nxt) + kofs(here ? min(nk, nks_c) : min(nk - nks_pad, nks_c)));
        // keep the refill here: left to itself the scheduler sinks all refills
        // to the end of the unrolled body, and the ring degrades to batches
        // that drain to zero loads in flight
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!has_next) {
#pragma unroll
      for (int d = 0; d < D; ++d) step(nks_pad - D + d, ring[d]);
    }
    // D[m][j] of this item's row group: lane (j + 16 * (m / 4)), element m % 4
    const int rg = wi.rg0 + it * wi.rg_step;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = grp * 4 + e, j = rg * 16 + mrow;
      if (KSPL == 1) {
        if (m < nb && j < R) ys[j * nb + m] = acc[e];
      } else if (m < nb) {
        c.s.red[((rg * KSPL + wi.sl) * nb + m) * 16 + mrow] = acc[e];
      }
    }
    cur = nxt;
    nxt = item_rows(it + 2);
  }
  if (tid == 0) c.s.tclk[3] = (uint32_t)now_ticks();
  __syncthreads();
  if (KSPL > 1) {   // add the k slices of each row group, in slice order
    for (int t = tid; t < RG * nb * 16; t += kBlock) {
      const int jj = t & 15, mm = (t >> 4) % nb, rg = (t >> 4) / nb;
      float sum = 0.f;
      for (int sl = 0; sl < KSPL; ++sl) sum += c.s.red[((rg * KSPL + sl) * nb + mm) * 16 + jj];
      const int j = rg * 16 + jj;
      if (j < R) ys[j * nb + mm] = sum;
    }
    __syncthreads();
  }
  if (tid == 0) c.s.tclk[4] = (uint32_t)now_ticks();
  return true;
}

// bfloat16 weights take their inputs as hi + lo pairs: a single bfloat16
// rounding of every activation (2^-9 relative) compounds through a deep stack
// beyond a 1e-2 output tolerance; the pair carries float32-level accuracy.
template <typename WT> struct SplitIn { static constexpr bool value = sizeof(WT) == 2; };

template <typename WT, bool PK>
__device__ __forceinline__ bool gemv_any(const Ctx& c, const GemvRows& rw, int R, int K, const GemvIn& in, int nb,
                                         const int* wev, int wsubs, float* ys) {
  return gemv<WT, SplitIn<WT>::value, PK>(c, rw, R, K, in, nb, wev, wsubs, ys);
}

// Bytes of one staged input row of depth K in LDS (bfloat16 hi + lo, or float).
template <typename WT>
__device__ __forceinline__ int xs_row_bytes(int K) {
  typedef MM<WT> T;
  const int Kp = ((K + T::KSTEP - 1) / T::KSTEP) * T::KSTEP;
  return (SplitIn<WT>::value ? 2 : 1) * (Kp + T::XPAD) * (int)sizeof(typename T::XT);
}

// Input rows per GEMV pass for depth K and R output rows: what the xy region
// holds (the rows, then the [R][nb] outputs), at most 16 (one MFMA row block).
template <typename WT>
__device__ __forceinline__ int pass_rows(int K, int R) {
  const int nb = (kXyBytes - 16) / (xs_row_bytes<WT>(K) + 4 * R);
  return nb < kMaxNb ? nb : kMaxNb;
}

// ---------------------------------------------------------------------------
// GEMV passes. Every projection of the step is a sequence of GEMV passes: the
// rows of one tile (or of one expert slice) against up to 16 staged input
// rows, then an epilogue that consumes the result. A task yields its passes in
// order (a batch wider than one pass takes several; a MoE share takes one per
// grouped task), and the main loop runs each through the one GEMV engine.
// ---------------------------------------------------------------------------
enum Epi : int { E_QKV = 0, E_O, E_GU, E_DOWN, E_ROUTER, E_MGU, E_MDOWN };

struct Pass {
  GemvRows rw;
  GemvIn in;
  int R, K, nb;     // output rows, depth of this pass (its K slice), input rows
  const int* wev;   // event the pass waits on (after its weights are in flight)
  int wsubs;        // its sub-counters (0: a bare counter)
  int epi;
  int b0;           // first batch row (dense, router) or first grouped row (MoE)
  int r0;           // first rotation unit (QKV), output row, or expert column
  int n;            // QKV: rotation units; GU / MoE gate-up: rows per matrix; else rows
  int e;            // MoE: expert
  int stage;        // dense stage 0..3 (QKV, O, gate/up, down), -1 otherwise
  int tile, slice, ks;   // row tile, K slice, slices of the stage (1: no split)
  int kfull;        // the stage's whole depth
  int rs;           // split-K record stride (floats): outputs of the stage's largest tile + 16
  int l;            // layer
  float* ys;        // the pass's outputs [R][nb] in LDS, after its staged inputs
};


// Pass p of a GEMV task; false once the task has no pass p. Dense stages take
// their split from this step's geometry: task (tile, K slice) covers all
// batch rows in one pass when the depth is split, else passes of what the LDS
// holds (a task whose stage is not split has slice 0).
// The XCD this workgroup runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ int xcd_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kXcd - 1); }

// One thread: the next grouped expert task index of layer l's dynamic queue,
// or n (the count of tasks) when none is left. Central: one counter for every
// workgroup. Per XCD: counter x hands out the indices x, x + 8, x + 16, ...;
// a workgroup takes its own XCD's next index, else steals the next index of
// another XCD's counter (reading each first, to skip exhausted ones without an
// atomic). Each counter hands out its gate/up indices (below the count of
// gate/up tasks) before its down indices, so a workgroup that waits on a down
// task's ready-queue slot implies that every gate/up task is held by a
// workgroup that runs it: the queue cannot deadlock.
__device__ __forceinline__ int moe_pop(const StepArgs& a, int l, int n) {
  int* mq = a.ws.mq + (size_t)l * kMq * kCtr;
  if (a.moe_dyn != 2) return min(atomic_add_relaxed(mq, 1), n);
  const int x = xcd_id();
  for (int s = 0; s < kXcd; ++s) {
    const int y = (x + s) & (kXcd - 1);
    int* cy = mq + (2 + y) * kCtr;
    if (s > 0 && y + kXcd * ldci(cy) >= n) continue;   // exhausted already
    const int i = y + kXcd * atomic_add_relaxed(cy, 1);
    if (i < n) return i;
  }
  return n;
}

template <typename WT, int KP>
__device__ __forceinline__ bool make_pass(const Ctx& c, const int4 task, int p, const int* wev, Pass& ps) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const LayerPtrs* Lp = a.layers + c.l;   // its fields are read with global loads (ldp)
  const int tile = task.y;
  if constexpr ((KP & 3) == KP_DENSE) {
    if (task.x != T_QKV && task.x != T_O && task.x != T_GU && task.x != T_DOWN) return false;
  } else if constexpr ((KP & 3) == KP_MOE) {
    if (task.x == T_GU || task.x == T_DOWN) return false;
  }
  ps.wev = p == 0 ? wev : nullptr;
  ps.wsubs = kSubs;
  ps.e = 0;
  ps.stage = -1;
  ps.l = c.l;
  ps.tile = tile;
  ps.slice = 0;
  ps.ks = 1;
  // grouped down task i = (row tile i / sd, H slice i % sd); waits on its expert's counter
  auto mdown = [&](int i) {
    const int sd = ldsu(a.ws.moe_info + 3), t = i / sd, sl = i - t * sd;
    const int e = ldsu(a.ws.tile_info + 2 * t), row0 = ldsu(a.ws.tile_info + 2 * t + 1);
    const int h0 = (int)((long)sl * dm.H / sd), R = (int)((long)(sl + 1) * dm.H / sd) - h0;
    ps.rw = GemvRows{ROWS_CONTIG, reinterpret_cast<const WT*>(ldp(&Lp->w_exp_down)) + (size_t)e * dm.H * dm.Fe,
                     nullptr, h0, 0, dm.Fe, 0, 0, 0};
    ps.in = GemvIn{mact_of(a, c.l) + (size_t)row0 * dm.Fe, dm.Fe, nullptr, nullptr, 0, 0.f, -1};
    ps.R = R; ps.K = dm.Fe; ps.kfull = dm.Fe; ps.nb = min(kMoeBM, ldsu(a.ws.exp_indptr + e + 1) - row0);
    ps.wev = a.ws.ectr + ((size_t)c.l * dm.E + e) * kCtr;
    ps.wsubs = 0;
    ps.epi = E_MDOWN; ps.b0 = row0; ps.r0 = h0; ps.n = R; ps.e = e;
  };
  // the K slice of a dense task, its rows per pass and first batch row
  int k0 = 0, kn = 0, b0 = 0, nbb = 0;
  auto dense = [&](int stage, int K, int R, int units, int urows) -> bool {
    const StageGeo g{ldku(&a.geo[stage].ks), ldku(&a.geo[stage].tiles), ldku(&a.geo[stage].kr),
                     ldku(&a.geo[stage].blk)};
    const bool one = g.ks > 1 || g.blk > 1;   // one pass of up to 16 rows: batch block task.w
    k0 = task.z * g.kr;
    kn = min(K, k0 + g.kr) - k0;
    nbb = one ? kMaxNb : pass_rows<WT>(kn, R);
    b0 = task.w * kMaxNb + p * nbb;
    if (b0 >= a.batch || (one && p > 0)) return false;
    ps.tile = tile + task.w * g.tiles;   // the split record and counter of (block, tile)
    ps.stage = stage;
    ps.slice = task.z;
    ps.ks = g.ks;
    ps.kfull = K;
    ps.K = kn;
    ps.R = R;
    ps.nb = min(nbb, a.batch - b0);
    ps.b0 = b0;
    // one record stride for every block of the stage (the last may be short),
    // a whole number of 16-byte units
    ps.rs = kpart_stride(units, urows, g.tiles, g.blk > 1 ? kMaxNb : ps.nb);
    return true;
  };
  switch (task.x) {
    case T_QKV: {   // RMSNorm1 + QKV rotation pairs of the tile
      const int2 u = tile_units(tile, dm.qkv_units, ldku(&a.geo[0].tiles));
      if (!dense(0, dm.H, 2 * u.y, dm.qkv_units, 2)) return false;
      ps.rw = GemvRows{ROWS_QKV, ldp(&Lp->w_qkv), nullptr, u.x, dm.d >> 1, dm.H, k0, dm.Hq / dm.Hkv, dm.Hq};
      ps.in = GemvIn{hid_in(a, c.l) + (size_t)b0 * dm.H + k0, dm.H, nullptr, ldp(&Lp->attn_norm) + k0,
                     ps.ks > 1 ? 2 : 1, dm.eps, -1};
      if constexpr ((KP & 3) == KP_ALL)
        if (a.per_op) ps.in = GemvIn{a.ws.u + (size_t)b0 * dm.H + k0, dm.H, nullptr, nullptr, 0, dm.eps, -1};
      ps.epi = E_QKV; ps.r0 = u.x; ps.n = u.y;
      break;
    }
    case T_O: {     // O-projection rows of the tile
      const int K = dm.Hq * dm.d;
      const int2 u = tile_units(tile, dm.H, ldku(&a.geo[1].tiles));
      if (!dense(1, K, u.y, dm.H, 1)) return false;
      ps.rw = GemvRows{ROWS_CONTIG, ldp(&Lp->w_o), nullptr, u.x, 0, K, k0, 0, 0};
      ps.in = GemvIn{o_of(a, c.l) + (size_t)b0 * K + k0, K, nullptr, nullptr, 0, 0.f, a.attn_merge_o ? b0 : -1};
      ps.epi = E_O; ps.r0 = u.x; ps.n = u.y;
      break;
    }
    case T_GU: {    // RMSNorm2 + gate and up rows of the tile
      const int2 u = tile_units(tile, dm.F, ldku(&a.geo[2].tiles));
      if (!dense(2, dm.H, 2 * u.y, dm.F, 2)) return false;
      ps.rw = GemvRows{ROWS_PAIR, ldp(&Lp->w_gate), ldp(&Lp->w_up), u.x, u.y, dm.H, k0, 0, 0};
      ps.in = GemvIn{h1_of(a, c.l) + (size_t)b0 * dm.H + k0, dm.H, nullptr, ldp(&Lp->ffn_norm) + k0,
                     ps.ks > 1 ? 2 : 1, dm.eps, -1};
      if constexpr ((KP & 3) == KP_ALL)
        if (a.per_op) ps.in = GemvIn{a.ws.u + (size_t)b0 * dm.H + k0, dm.H, nullptr, nullptr, 0, dm.eps, -1};
      ps.epi = E_GU; ps.r0 = u.x; ps.n = u.y;
      break;
    }
    case T_DOWN: {  // down-projection rows of the tile
      const int2 u = tile_units(tile, dm.H, ldku(&a.geo[3].tiles));
      if (!dense(3, dm.F, u.y, dm.H, 1)) return false;
      ps.rw = GemvRows{ROWS_CONTIG, ldp(&Lp->w_down), nullptr, u.x, 0, dm.F, k0, 0, 0};
      ps.in = GemvIn{act_of(a, c.l) + (size_t)b0 * dm.F + k0, dm.F, nullptr, nullptr, 0, 0.f, -1};
      ps.epi = E_DOWN; ps.r0 = u.x; ps.n = u.y;
      break;
    }
    case T_ROUTER: {  // RMSNorm2 + router rows [16 y, 16 y + 16) for the token block [16 z, 16 z + 16)
      const int bend = min(a.batch, (task.z + 1) * kMaxNb);
      const int nbr = pass_rows<WT>(dm.H, 16), br = task.z * kMaxNb + p * nbr;
      if (br >= bend) return false;
      const int r0 = tile * 16;
      ps.rw = GemvRows{ROWS_CONTIG, ldp(&Lp->w_router), nullptr, r0, 0, dm.H, 0, 0, 0};
      ps.in = GemvIn{h1_of(a, c.l) + (size_t)br * dm.H, dm.H, nullptr, ldp(&Lp->ffn_norm), 1, dm.eps, -1};
      ps.R = min(16, dm.E - r0); ps.K = dm.H; ps.kfull = dm.H; ps.nb = min(nbr, bend - br);
      ps.epi = E_ROUTER; ps.b0 = br; ps.r0 = r0; ps.n = ps.R;
      break;
    }
    case T_MGU: {   // grouped gate/up task i = (row tile i / sg, Fe slice i % sg)
      int i = c.wg + p * dm.grid;   // static: this workgroup's share
      const int nmgu = ldsu(a.ws.moe_info + 0);
      if (a.moe_dyn) {
        // dynamic: the next index of the layer's queue, gate/up tasks [0, nmgu),
        // then down tasks in the order their experts became ready
        if (threadIdx.x == 0) *c.s.flag = moe_pop(a, c.l, nmgu + ldsu(a.ws.moe_info + 1));
        __syncthreads();
        i = __builtin_amdgcn_readfirstlane(*c.s.flag);
        __syncthreads();
        if (i >= nmgu) {
          const int j = i - nmgu;
          if (j >= ldsu(a.ws.moe_info + 1)) return false;
          if (threadIdx.x < 64) {
            const int v = spin_nonzero(a.ws.rq + (size_t)c.l * dm.max_down + j, a.ws.err, a.watchdog_ticks);
            if (threadIdx.x == 0) *c.s.flag = v;
          }
          __syncthreads();
          const int v = __builtin_amdgcn_readfirstlane(*c.s.flag);
          __syncthreads();
          if (v == 0) return false;   // abandoned step
          mdown(v - 1);
          ps.wev = nullptr;           // ready once queued
          break;
        }
      } else if (i >= nmgu) {
        return false;
      }
      const int sg = ldsu(a.ws.moe_info + 2), t = i / sg, sl = i - t * sg;
      const int e = ldsu(a.ws.tile_info + 2 * t), row0 = ldsu(a.ws.tile_info + 2 * t + 1);
      const int f0 = (int)((long)sl * dm.Fe / sg), Rh = (int)((long)(sl + 1) * dm.Fe / sg) - f0;
      const size_t eo = (size_t)e * dm.Fe * dm.H;
      ps.rw = GemvRows{ROWS_PAIR, reinterpret_cast<const WT*>(ldp(&Lp->w_exp_gate)) + eo,
                       reinterpret_cast<const WT*>(ldp(&Lp->w_exp_up)) + eo, f0, Rh, dm.H, 0, 0, 0};
      // the tile's rows: its routed tokens' FFN inputs (RMSNorm2 of h1), gathered
      ps.in = GemvIn{h1_of(a, c.l), dm.H, a.ws.sorted_tok + row0, ldp(&Lp->ffn_norm), 1, dm.eps, -1};
      ps.R = 2 * Rh; ps.K = dm.H; ps.kfull = dm.H; ps.nb = min(kMoeBM, ldsu(a.ws.exp_indptr + e + 1) - row0);
      ps.epi = E_MGU; ps.b0 = row0; ps.r0 = f0; ps.n = Rh; ps.e = e;
      break;
    }
    case T_MDOWN: {  // static: this workgroup's share of the down tasks (dynamic: popped with the gate/up ones)
      const int i = c.wg + p * dm.grid;
      if (a.moe_dyn || i >= ldsu(a.ws.moe_info + 1)) return false;
      mdown(i);
      break;
    }
    default: return false;
  }
  ps.ys = reinterpret_cast<float*>(reinterpret_cast<char*>(c.s.xs) +
                                   (ps.nb * xs_row_bytes<WT>(ps.K) + 15) / 16 * 16);
  return true;
}

// The residual an O / down pass adds (hidden, resp. h1): thread t holds
// elements t, t + kBlock, ... of the [R][nb] tile (R nb <= kYsFloats). It is
// final once this workgroup has seen the event that produced it, so it is
// loaded before the pass's weights are waited on, and added into ys by the
// whole workgroup once the pass's sums are there.
constexpr int kResid = kYsFloats / kBlock;
__device__ __forceinline__ const float* resid_src(const StepArgs& a, const Pass& ps) {
  return ps.epi == E_O ? hid_in(a, ps.l) : h1_of(a, ps.l);
}
__device__ __forceinline__ void load_resid(const StepArgs& a, const Pass& ps, float (&r)[kResid]) {
  const float* res = resid_src(a, ps);
#pragma unroll
  for (int k = 0; k < kResid; ++k) {
    const int idx = threadIdx.x + k * kBlock;
    if (idx < ps.n * ps.nb) {
      const int j = idx / ps.nb, m = idx - j * ps.nb;
      r[k] = ldc(res + (size_t)(ps.b0 + m) * a.dm.H + ps.r0 + j);
    }
  }
}
__device__ __forceinline__ void add_resid(const Pass& ps, const float (&r)[kResid]) {
#pragma unroll
  for (int k = 0; k < kResid; ++k) {
    const int idx = threadIdx.x + k * kBlock;
    if (idx < ps.n * ps.nb) ps.ys[idx] += r[k];   // ys is [R][nb]: idx = j nb + m
  }
  __syncthreads();
}

// Split-K: store this slice's partial sums (ys, and for a normed stage the
// rows' raw sums of squares over the slice), count the slice done, and let
// the last slice task of the row tile add every slice, in slice order (its
// own from LDS), into ys and turn the sums of squares into 1 / rms over the
// whole depth. Returns whether this task is that last one (the others have
// nothing more to do for the tile).
//
// A record is the slice's n = R nb sums then, normed, its nb sums of squares,
// records rs floats apart (rs a multiple of 4). Records move as 16-byte
// units. The last task pulls the other slices' records into the staged-input
// region of LDS, which the pass no longer reads, with loads that go straight
// to LDS: one round trip to the coherence point for the whole tile, and no
// registers held (a loop of register loads paid one round trip per element
// group, which made these tasks the last of their stage by 5-15 us).
__device__ __forceinline__ bool reduce_slices(const Ctx& c, const Pass& ps) {
  const StepArgs& a = c.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), n = ps.R * ps.nb, rs = ps.rs;
  const bool normed = ps.in.norm != 0;
  const int nrec = n + (normed ? ps.nb : 0), U = (nrec + 3) >> 2;
  float* part = uptr(a.ws.kpart + kpart_rec(a.dm, ps.stage, ps.tile, ps.ks, 0, rs));
  const auto prs = rsrc_n(part, ps.ks * rs * 4);
  auto own = [&](int i) -> float { return i < n ? ps.ys[i] : (i < nrec ? c.s.rstd[i - n] : 0.f); };
  for (int u = tid; u < U; u += kBlock)
    stc4(prs, (ps.slice * rs + 4 * u) * 4, f4v{own(4 * u), own(4 * u + 1), own(4 * u + 2), own(4 * u + 3)});
  vm_drain();
  __syncthreads();
  if (tid == 0) {
    int* ctr = a.ws.tctr + ((size_t)ps.stage * a.dm.tctr_stride + ps.tile) * kCtr;
    const int last = atomic_add_relaxed(ctr, 1) == ps.ks - 1;
    if (last) stci(ctr, 0);   // every slice has counted: ready for this stage of the next layer
    *c.s.flag = last;
  }
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(*c.s.flag)) return false;
  // the other slices, in slice order, each in 1 KiB blocks (one wave load
  // each) below ys; lanes past a record load into their block's padding
  const int UB = (U + 63) >> 6;
  const int ys_off = (int)(reinterpret_cast<char*>(ps.ys) - reinterpret_cast<char*>(c.s.xs));
  char* land = reinterpret_cast<char*>(c.s.xs);
  const float* landf = reinterpret_cast<const float*>(land);
  if ((ps.ks - 1) * UB * 1024 <= ys_off) {
    for (int id = wave; id < (ps.ks - 1) * UB; id += kWaves) {
      const int oi = id / UB, blk = id - oi * UB, sl = oi + (oi >= ps.slice ? 1 : 0);
      ldc4_lds(prs, (sl * rs + (blk * 64 + lane) * 4) * 4, land + (oi * UB + blk) * 1024);
    }
    vm_drain();
    __syncthreads();
    for (int i = tid; i < nrec; i += kBlock) {
      float sum = 0.f;
      for (int sl = 0; sl < ps.ks; ++sl)
        sum += sl == ps.slice ? own(i) : landf[(sl - (sl > ps.slice ? 1 : 0)) * UB * 256 + i];
      if (i < n)
        ps.ys[i] = sum;
      else
        c.s.rstd[i - n] = 1.0f / sqrtf(sum / (float)ps.kfull + ps.in.eps);
    }
  } else {   // records too large for the free LDS: register loads, element by element
    for (int i = tid; i < nrec; i += kBlock) {
      float v[kMaxKs];
#pragma unroll
      for (int sl = 0; sl < kMaxKs; ++sl)
        v[sl] = (sl < ps.ks && sl != ps.slice) ? ldc(part + sl * rs + i) : 0.f;
      float sum = 0.f;
#pragma unroll
      for (int sl = 0; sl < kMaxKs; ++sl)
        if (sl < ps.ks) sum += sl == ps.slice ? own(i) : v[sl];
      if (i < n)
        ps.ys[i] = sum;
      else
        c.s.rstd[i - n] = 1.0f / sqrtf(sum / (float)ps.kfull + ps.in.eps);
    }
  }
  __syncthreads();
  return true;
}

// Wave 0 alone consumes a pass's result (ys[j][m], rstd[m] in LDS) and stores
// its outputs, while the other waves go on streaming the next pass's weights.
// `have_resid`: the O / down residual is already in ys. Consecutive lanes take
// consecutive outputs j of one batch row m, so each store instruction writes
// whole runs of a row: with the batch index fastest, one instruction wrote 16
// rows' 16-byte pieces, and such scattered device-coherent partial-line
// stores took a wave 5-13 us per tile at 16 rows.
// Threads t0, t0 + nt, ... of the workgroup take the outputs: wave 0 alone
// (t0 = lane, nt = 64), or, for the last slice task of a split tile, every
// wave (t0 = threadIdx.x, nt = kBlock). The MoE gate/up case notifies its
// expert from lane 0 of the calling wave and is only run by wave 0.
template <typename WT, int KP>
__device__ __forceinline__ void epilogue(const Ctx& c, const Pass& ps, bool have_resid, int t0, int nt) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const int nb = ps.nb, b0 = ps.b0, lane = threadIdx.x & 63;
  const float* ys = ps.ys;
  if constexpr ((KP & 3) == KP_DENSE) {
    if (ps.epi > E_DOWN) return;
  } else if constexpr ((KP & 3) == KP_MOE) {
    if (ps.epi == E_GU || ps.epi == E_DOWN) return;
  }
  switch (ps.epi) {
    case E_QKV: {   // RoPE at each request's position, then q/k/v out and the K/V append
      // The model's dimensions are held in registers for the whole epilogue
      // (read through `a`, they are reloaded after every store, which might
      // alias the argument block), and the index math is branch-free: element
      // (request m, tile unit ju) at index ju << sh | m (2^sh >= nb), the
      // unit's (head, pair) from multiply-high dividers set up once.
      const int Hq = dm.Hq, Hkv = dm.Hkv, d = dm.d, half = d >> 1, G = Hq / Hkv, per = (G + 2) * half;
      const int qkv_dim = (Hq + 2 * Hkv) * d, max_seq = dm.max_seq, mb = dm.max_batch, r0 = ps.r0;
      const int sh = nb <= 1 ? 0 : 32 - __builtin_clz(nb - 1), ni = ps.n << sh;
      float* const qkv = qkv_of(a, c.l);
      WT* const kvb = reinterpret_cast<WT*>(a.kv);
      const UDiv per_div(per), half_div(half);
      auto unit_hi = [&](int ju, int& h, int& i) {
        const int up = r0 + ju, g = per_div.div(up), r = up - g * per;
        const int hg = half_div.div(r);   // head within the group's run: G query heads, its key, its value
        i = r - hg * half;
        const int hq = g * G + hg, hkv = Hq + (hg - G) * Hkv + g;
        h = hg < G ? hq : hkv;
      };
      if constexpr ((KP & 3) == KP_ALL) {
        if (a.per_op) {   // the projection alone: RoPE and the append are ops of their own
          for (int idx = t0; idx < ni; idx += nt) {
            const int m = idx & ((1 << sh) - 1), ju = idx >> sh;
            if (m >= nb) continue;
            int h, i;
            unit_hi(ju, h, i);
            float* dst = qkv + (size_t)(b0 + m) * qkv_dim + h * d + i;
            stc(dst, ys[(2 * ju) * nb + m]);
            stc(dst + half, ys[(2 * ju + 1) * nb + m]);
          }
          break;
        }
      }
      // lane m < nb holds request b0 + m's position; the rotation rows of
      // eight items per lane are loaded together (one latency per eight
      // items, not two dependent ones per item). A workgroup takes the same
      // QKV pass in every layer of a launch, at the same positions: the
      // first layer's rows are kept in LDS (rope, keyed by the pass) and the
      // later layers read them there instead of from memory.
      // (a wave-uniform flag, so that a hit branches around the loads
      // instead of issuing them and selecting)
      const bool hit = __builtin_amdgcn_readfirstlane(c.s.rope_key[0] == r0 + 1 && c.s.rope_key[1] == b0 &&
                                                      c.s.rope_key[2] == ni * 32 + nb) != 0;
      const bool keep = !hit && ni <= kRopeBytes / 8;
      int posl;
      if (hit)
        posl = c.s.rope_pos[lane < nb ? lane : 0];
      else
        posl = *gp(a.seq_lens + b0 + (lane < nb ? lane : 0));
      if (keep && t0 < 64 && lane < nb) c.s.rope_pos[lane] = posl;   // the first wave of the pass: one per request
      const auto rrs = rsrc_n(a.ws.rope, max_seq * half * 8);
      for (int base = 0; base < ni; base += nt * 8) {
        float2 cs[8];
        int hs[8], is[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) unit_hi(min((base + t0 + nt * u) >> sh, ps.n - 1), hs[u], is[u]);
        if (hit) {
#pragma unroll
          for (int u = 0; u < 8; ++u) cs[u] = c.s.rope[min(base + t0 + nt * u, ni - 1)];
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int idx = base + t0 + nt * u, m = idx & ((1 << sh) - 1);
            const int pos = __shfl(posl, m, 64);
            cs[u] = ldk2(rrs, idx < ni && m < nb && hs[u] < Hq + Hkv ? (pos * half + is[u]) * 8 : kNoRecord);
          }
        }
        if (keep) {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int idx = base + t0 + nt * u;
            if (idx < ni) c.s.rope[idx] = cs[u];
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int idx = base + t0 + nt * u;
          if (idx >= ni) break;
          const int m = idx & ((1 << sh) - 1), ju = idx >> sh, h = hs[u], i = is[u];
          if (m >= nb) continue;
          const float r = c.s.rstd[m];
          float y1 = ys[(2 * ju) * nb + m] * r, y2 = ys[(2 * ju + 1) * nb + m] * r;
          const int bb = b0 + m, pos = __shfl(posl, m, 64);
          if (h < Hq + Hkv) {
            const float t1 = y1 * cs[u].x - y2 * cs[u].y, t2 = y2 * cs[u].x + y1 * cs[u].y;
            y1 = t1;
            y2 = t2;
          }
          float* dst = qkv + (size_t)bb * qkv_dim + h * d + i;
          stc(dst, y1);
          stc(dst + half, y2);
          if (h >= Hq) {   // the append: kv_off of (layer, K or V, request, KV head, pos)
            const int kvh = h - Hq, which = kvh >= Hkv ? 1 : 0, g = kvh - which * Hkv;
            WT* cp = kvb + ((((size_t)(c.l * 2 + which) * mb + bb) * Hkv + g) * (size_t)max_seq + pos) * d;
            Elem<WT>::put(cp + i, y1);
            Elem<WT>::put(cp + i + half, y2);
          }
        }
      }
      // the kept rows are read by this workgroup's next QKV pass, a later
      // task: every task starts with a workgroup barrier
      if (keep && t0 == 0) {
        c.s.rope_key[0] = r0 + 1;
        c.s.rope_key[1] = b0;
        c.s.rope_key[2] = ni * 32 + nb;
      }
      break;
    }
    case E_O:       // h1 = x + W_o o
    case E_DOWN: {  // x' = h1 + W_down act (the layer output, into hidden)
      const float* res = resid_src(a, ps);
      float* out = ps.epi == E_O ? h1_of(a, c.l) : hid_out(a, c.l);
      for (int idx = t0; idx < ps.n * nb; idx += nt) {
        const int m = idx / ps.n, j = idx - m * ps.n;
        const size_t o = (size_t)(b0 + m) * dm.H + ps.r0 + j;
        stc(out + o, (have_resid ? 0.f : ldc(res + o)) + ys[j * nb + m]);
      }
      break;
    }
    case E_GU:      // act = silu(gate) * up
    case E_MGU: {
      const int Rh = ps.n;
      float* out = ps.epi == E_GU ? act_of(a, c.l) : mact_of(a, c.l);
      const int ld = ps.epi == E_GU ? dm.F : dm.Fe;
      for (int idx = t0; idx < Rh * nb; idx += nt) {
        const int m = idx / Rh, j = idx - m * Rh;
        const float r = c.s.rstd[m];
        const float gt = ys[j * nb + m] * r, up = ys[(Rh + j) * nb + m] * r;
        stc(out + (size_t)(b0 + m) * ld + ps.r0 + j, gt / (1.0f + __expf(-gt)) * up);
      }
      if (ps.epi == E_MGU) {   // this task of expert e is done
        int* ec = a.ws.ectr + ((size_t)c.l * dm.E + ps.e) * kCtr;
        if (!a.moe_dyn) {
          wave_notify(ec, -1);
        } else {
          // the expert's last gate/up task queues the expert's down tasks
          vm_drain();
          const int left = __shfl(lane == 0 ? atomic_add_relaxed(ec, -1) : 0, 0, 64);
          if (left == 1) {
            const int t0 = ldci(a.ws.tile_ptr + ps.e), t1 = ldci(a.ws.tile_ptr + ps.e + 1);
            const int sd = ldci(a.ws.moe_info + 3), n = (t1 - t0) * sd;
            const int slot = __shfl(lane == 0 ? atomic_add_relaxed(a.ws.mq + ((size_t)c.l * kMq + 1) * kCtr, n) : 0, 0, 64);
            int* rq = a.ws.rq + (size_t)c.l * dm.max_down + slot;
            for (int i = lane; i < n; i += 64) stci(rq + i, t0 * sd + i + 1);
          }
        }
      }
      break;
    }
    case E_ROUTER: {
      for (int idx = t0; idx < ps.n * nb; idx += nt) {
        const int m = idx / ps.n, j = idx - m * ps.n;
        stc(a.ws.logits + (size_t)(b0 + m) * dm.E + ps.r0 + j, ys[j * nb + m] * c.s.rstd[m]);
      }
      break;
    }
    case E_MDOWN: {
      for (int idx = t0; idx < ps.n * nb; idx += nt) {
        const int m = idx / ps.n, j = idx - m * ps.n;
        stc(a.ws.mout + (size_t)(b0 + m) * dm.H + ps.r0 + j, ys[j * nb + m]);
      }
      break;
    }
    default: break;
  }
}

// ---------------------------------------------------------------------------
// Split-K GQA decode attention for (request b, KV head g, chunk ci): the G
// query heads of group g against positions [ci*ck, min((ci+1)*ck, S+1)).
// Lanes 16r..16r+15 of a wave hold one KV position (16 bytes each, so a 256-B
// row); a wave covers 4 positions per step and the workgroup 32; ITS steps
// cover the chunk. The cached rows are loaded before the QKV event is awaited
// (they do not depend on this step); the new position S uses this step's
// rotated k and v, rounded exactly as they were stored into the cache. A chunk
// writes its (acc, max, sum) partial; the workgroup that completes the last
// chunk of (b, g) merges all partials by log-sum-exp and notifies. A request
// with a single chunk writes its output directly.
// ---------------------------------------------------------------------------
template <typename KT> __device__ __forceinline__ void unpack_row(const uint4 r, float (&f)[16 / sizeof(KT)]);
template <> __device__ __forceinline__ void unpack_row<uint16_t>(const uint4 r, float (&f)[8]) {
  f[0] = bf_lo(r.x); f[1] = bf_hi(r.x); f[2] = bf_lo(r.y); f[3] = bf_hi(r.y);
  f[4] = bf_lo(r.z); f[5] = bf_hi(r.z); f[6] = bf_lo(r.w); f[7] = bf_hi(r.w);
}
template <> __device__ __forceinline__ void unpack_row<float>(const uint4 r, float (&f)[4]) {
  f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y); f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
}
// Device-coherent float row slice -> cache-dtype bits (rounded like the KV append).
template <typename KT> __device__ __forceinline__ uint4 pack_row(__amdgpu_buffer_rsrc_t r, int off);
template <> __device__ __forceinline__ uint4 pack_row<uint16_t>(__amdgpu_buffer_rsrc_t r, int off) {
  const f4v a = ldk4(r, off), b = ldk4(r, off + 16);
  return make_uint4((uint32_t)f2bf(a.x) | ((uint32_t)f2bf(a.y) << 16), (uint32_t)f2bf(a.z) | ((uint32_t)f2bf(a.w) << 16),
                    (uint32_t)f2bf(b.x) | ((uint32_t)f2bf(b.y) << 16), (uint32_t)f2bf(b.z) | ((uint32_t)f2bf(b.w) << 16));
}
template <> __device__ __forceinline__ uint4 pack_row<float>(__amdgpu_buffer_rsrc_t r, int off) {
  const f4v a = ldk4(r, off);
  return make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z), __float_as_uint(a.w));
}

// The end of an attention chunk task, once every wave has left its partial
// (acc[D], max, sum per query head; log2 units) in LDS at sw[wave][h][DP]:
// combine the 8 waves into this chunk's partial (or the output, for a request
// with a single chunk), then notify; without the O-projection merge, the last
// chunk task of (b, g) to finish merges all partials by log-sum-exp.
template <int D>
__device__ __forceinline__ bool attn_finish(const Ctx& c, int b, int g, int ci, int tix, int nc, int G,
                                           const float* sw) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  constexpr int DP = D + 4;
  const int tid = threadIdx.x;
  float* o = o_of(a, c.l) + (size_t)b * dm.Hq * D + (size_t)g * G * D;
  float* part = a.attn_merge_o ? mpart_of(a, c.l) + (((size_t)b * dm.Hkv + g) * kMergeChunks + ci) * G * DP
                               : a.ws.part + (((size_t)b * dm.Hkv + g) * dm.max_chunks + ci) * G * DP;
  const auto orr = rsrc(o), prr = rsrc(part);
  for (int t = tid; t < G * D / 4; t += kBlock) {
    const int h = t / (D / 4), e0 = (t - h * (D / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sw[(w * G + h) * DP + D]);
    float Ls = 0.f;
    f4v A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* sp = sw + (w * G + h) * DP;
      const float f = (sp[D] == -INFINITY) ? 0.f : exp2f(sp[D] - M);
      Ls += sp[D + 1] * f;
      A += *reinterpret_cast<const f4v*>(sp + e0) * f;
    }
    if (nc == 1 && !a.attn_merge_o && !a.per_op) {
      stc4(orr, (h * D + e0) * 4, A / Ls);
    } else {
      stc4(prr, (h * DP + e0) * 4, A);
      if (e0 == 0) stc4(prr, (h * DP + D) * 4, f4v{M, Ls, 0.f, 0.f});
    }
  }
  if (tid == 0) c.s.tclk[5] = (uint32_t)now_ticks();   // outputs issued
  // the event of (block of b, group g): flat, counts the chunk tasks that
  // notify (the O-projection, or the per-op merge, merges the partials) or
  // one notify per request
  int* aev = c.nev;
  if (a.attn_merge_o || a.per_op || nc == 1) {
    wg_notify(aev, -1);
    return true;
  }
  // the last chunk task of (b, g) to finish merges the partials
  vm_drain();
  __syncthreads();
  if (tid == 0) {
    int* mc = a.ws.mctr + (((size_t)c.l * dm.max_batch + b) * dm.Hkv + g) * kCtr;
    *c.s.flag = (atomic_add_relaxed(mc, -1) == 1);
  }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(*c.s.flag)) {
    const auto pbr = rsrc(a.ws.part + ((size_t)b * dm.Hkv + g) * dm.max_chunks * G * DP);
    for (int t = tid; t < G * D / 4; t += kBlock) {
      const int h = t / (D / 4), e0 = (t - h * (D / 4)) * 4;
      float M = -INFINITY, Ls = 0.f;
      f4v A = {0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < nc; c0 += 16) {   // 16 chunks' loads in flight at once
        f4v ms[16], as[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int cc = min(c0 + u, nc - 1);
          const int ro = ((cc * G + h) * DP) * 4;
          as[u] = ldc4(pbr, ro + e0 * 4);
          ms[u] = ldc4(pbr, ro + D * 4);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (c0 + u < nc) {
            const float mn = fmaxf(M, ms[u].x);
            const float fo = (M == -INFINITY) ? 0.f : exp2f(M - mn), fc = exp2f(ms[u].x - mn);
            Ls = Ls * fo + ms[u].y * fc;
            A = A * fo + as[u] * fc;
            M = mn;
          }
        }
      }
      stc4(orr, (h * D + e0) * 4, A / Ls);
    }
    wg_notify(aev, -1);
  }
  __syncthreads();
  return true;
}

template <typename KT, int HB, int ITS>
__device__ __forceinline__ bool task_attn(const Ctx& c, int b, int g, int ci, int tix, const int* wev, int wsubs) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  constexpr int EPL = 16 / (int)sizeof(KT);   // elements per lane (16 B)
  constexpr int D = 16 * EPL;                 // head_dim: 128 (bf16) or 64 (f32)
  constexpr int DP = D + 4;                   // partial record: acc[D], max, sum, pad
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), rs = lane >> 4, li = lane & 15;
  const int G = dm.Hq / dm.Hkv;               // query heads of the group, a multiple of HB
  const int ck = ITS * 32;
  const int qkv_dim = (dm.Hq + 2 * dm.Hkv) * D;
  const int S = ldku(a.seq_lens + b), n = S + 1;
  const int p0 = ci * ck, p1 = min(n, p0 + ck);
  const int nc = (n + ck - 1) / ck;

  const KT* Kb = reinterpret_cast<const KT*>(a.kv) + kv_off(dm, c.l, 0, b, g, 0) + li * EPL;
  const KT* Vb = reinterpret_cast<const KT*>(a.kv) + kv_off(dm, c.l, 1, b, g, 0) + li * EPL;
  uint4 kr[ITS], vr[ITS];
  const int pmax = S > 0 ? S - 1 : 0;
#pragma unroll
  for (int it = 0; it < ITS; ++it) {
    const int p = min(p0 + it * 32 + wave * 4 + rs, pmax);   // cached slots only (others replaced or unused)
    kr[it] = ldg16(Kb + (size_t)p * D);
    vr[it] = ldg16(Vb + (size_t)p * D);
  }
  if (!ctx_wait(c, wev, wsubs)) return false;   // flat counters: QKV[block][group] (all groups: per stage)

  float* sw = reinterpret_cast<float*>(c.s.xs);     // [kWaves][G][DP] per-wave partials
  float* qs = sw + kWaves * 8 * DP;                  // [G][D] this group's rotated queries
  const float* qrow = qkv_of(a, c.l) + (size_t)b * qkv_dim + (size_t)g * G * D;
  for (int t = tid; t < G * D / 4; t += kBlock) *reinterpret_cast<f4v*>(qs + 4 * t) = ldk4(rsrc(qrow), 16 * t);
  uint4 kn = make_uint4(0, 0, 0, 0), vn = kn;
  if (S >= p0 && S < p1) {
    const auto qr = rsrc(qkv_of(a, c.l) + (size_t)b * qkv_dim);
    kn = pack_row<KT>(qr, ((dm.Hq + g) * D + li * EPL) * 4);
    vn = pack_row<KT>(qr, ((dm.Hq + dm.Hkv + g) * D + li * EPL) * 4);
  }
  __syncthreads();
  if (tid == 0) c.s.tclk[2] = (uint32_t)now_ticks();
  const float qscale = 1.4426950408889634f / sqrtf((float)D);   // 1/sqrt(d), in log2 units

  for (int h0 = 0; h0 < G; h0 += HB) {
    // keep the KV rows packed across head groups (unpacking them once for all
    // groups would hold 16 floats per row live and spill)
#pragma unroll
    for (int it = 0; it < ITS; ++it) {
      __asm__ volatile("" : "+v"(kr[it].x), "+v"(kr[it].y), "+v"(kr[it].z), "+v"(kr[it].w));
      __asm__ volatile("" : "+v"(vr[it].x), "+v"(vr[it].y), "+v"(vr[it].z), "+v"(vr[it].w));
    }
    float q[HB][EPL], m[HB], ls[HB], acc[HB][EPL];
#pragma unroll
    for (int h = 0; h < HB; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[h][e] = qs[(h0 + h) * D + li * EPL + e] * qscale;
      m[h] = -INFINITY;
      ls[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }
#pragma unroll
    for (int it = 0; it < ITS; ++it) {
      const int p = p0 + it * 32 + wave * 4 + rs;
      if (p < p1) {
        float kf[EPL], vf[EPL];
        unpack_row<KT>(p == S ? kn : kr[it], kf);
        unpack_row<KT>(p == S ? vn : vr[it], vf);
#pragma unroll
        for (int h = 0; h < HB; ++h) {
          float sc = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) sc += q[h][e] * kf[e];
          sc = sum16(sc);
          const float mn = fmaxf(m[h], sc);
          const float al = exp2f(m[h] - mn), pe = exp2f(sc - mn);
          ls[h] = ls[h] * al + pe;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * al + pe * vf[e];
          m[h] = mn;
        }
      }
    }
    // combine the 4 position slots of the wave into this wave's LDS record
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      const float M = xrow_max(m[h]);
      const float sc = (M == -INFINITY) ? 0.f : exp2f(m[h] - M);
      const float lw = xrow_sum(ls[h] * sc);
      float* dst = sw + (wave * G + h0 + h) * DP;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float v = xrow_sum(acc[h][e] * sc);
        if (rs == 0) dst[li * EPL + e] = v;
      }
      if (lane == 0) { dst[D] = M; dst[D + 1] = lw; }
    }
  }
  if (tid == 0) c.s.tclk[3] = (uint32_t)now_ticks();   // wave 0's positions done
  __syncthreads();
  if (tid == 0) c.s.tclk[4] = (uint32_t)now_ticks();   // every wave's
  return attn_finish<D>(c, b, g, ci, tix, nc, G, sw);
}

// Split-K GQA decode attention with bfloat16 KV and head_dim 128, at most 8
// query heads per KV head (same task as task_attn, other engine). Each wave
// takes 16-position tiles (TW of them: tile t covers positions
// p0 + (wave + 8 t) * 16 ..). Scores come from the matrix cores: the G query
// heads (rows, padded to 16) times the tile's K rows (columns), the rows
// loaded as 16-row x 64-byte MFMA fragments exactly like GEMV weights, the
// queries as hi + lo bfloat16 pairs (float32-level products). The softmax of
// a wave's positions is plain (no running rescale): row max and sum are DPP
// reductions over the tile's 16 lanes. P V runs on the vector ALUs with each
// lane owning two head_dim elements over all of the wave's positions, the
// probabilities broadcast through LDS, so no cross-lane reduction is needed.
// GP: query heads rounded up to 4 or 8.
template <int TW, int GP>
__device__ __forceinline__ bool task_attn_mm(const Ctx& c, int b, int g, int ci, int tix, const int* wev, int wsubs) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  typedef MM<uint16_t> T;
  constexpr int D = 128, DP = D + 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), j = lane & 15, r = lane >> 4;
  const int G = dm.Hq / dm.Hkv;
  const int ck = a.attn_chunk;
  const int qkv_dim = (dm.Hq + 2 * dm.Hkv) * D;
  const int S = ldku(a.seq_lens + b), n = S + 1;
  const int p0 = ci * ck, p1 = min(n, p0 + ck);
  const int nc = (n + ck - 1) / ck;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.kv) + kv_off(dm, c.l, 0, b, g, 0);
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.kv) + kv_off(dm, c.l, 1, b, g, 0);
  const int pmax = S > 0 ? S - 1 : 0;   // cached slots only (slot S is this step's)
  // the cached rows, before the QKV event: K as MFMA fragments (lane (j, r):
  // row tb + j, elements 32 s + 8 r ..), V as one element pair per lane per row
  uint4 kr[TW][4];
  uint32_t vr[TW][16];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int tb = p0 + (wave + kWaves * t) * 16;
    const uint16_t* kp = Kb + (size_t)min(tb + j, pmax) * D + r * 8;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) kr[t][s4] = ldg16(kp + s4 * 32);
#pragma unroll
    for (int i = 0; i < 16; ++i) vr[t][i] = ldg4_nt(Vb + (size_t)min(tb + i, pmax) * D + 2 * lane);
  }
  if (!ctx_wait(c, wev, wsubs)) return false;   // flat counters: QKV[block][group] (all groups: per stage)

  // A operand: query head j of the group (zero beyond G), q * log2(e) / sqrt(d) as hi + lo
  const auto qr = rsrc_n(qkv_of(a, c.l) + (size_t)b * qkv_dim, qkv_dim * 4);
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  uint4 qh[4], ql[4];
  {
    const int qo = j < G ? ((g * G + j) * D + r * 8) * 4 : kNoRecord;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const f4v x0 = ldk4(qr, qo + s4 * 128) * qscale, x1 = ldk4(qr, qo + s4 * 128 + 16) * qscale;
      uint16_t hb[8], lb[8];
      const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hb[e] = f2bf(xv[e]);
        lb[e] = f2bf(xv[e] - __uint_as_float((uint32_t)hb[e] << 16));
      }
      qh[s4] = make_uint4(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16),
                          hb[4] | ((uint32_t)hb[5] << 16), hb[6] | ((uint32_t)hb[7] << 16));
      ql[s4] = make_uint4(lb[0] | ((uint32_t)lb[1] << 16), lb[2] | ((uint32_t)lb[3] << 16),
                          lb[4] | ((uint32_t)lb[5] << 16), lb[6] | ((uint32_t)lb[7] << 16));
    }
  }
  // position S takes this step's rotated k and v, rounded as the KV append stores them
  if (S >= p0 && S < p1) {
    const int tt = (S - p0) >> 4, jj = (S - p0) & 15;
    if (tt % kWaves == wave) {
      const int ts = tt / kWaves;
      const int ko = j == jj ? ((dm.Hq + g) * D + r * 8) * 4 : kNoRecord;
      const float2 vv = ldk2(qr, ((dm.Hq + dm.Hkv + g) * D + 2 * lane) * 4);
      const uint32_t vn = (uint32_t)f2bf(vv.x) | ((uint32_t)f2bf(vv.y) << 16);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const f4v x0 = ldk4(qr, ko + s4 * 128), x1 = ldk4(qr, ko + s4 * 128 + 16);
        const uint4 kn = make_uint4((uint32_t)f2bf(x0.x) | ((uint32_t)f2bf(x0.y) << 16),
                                    (uint32_t)f2bf(x0.z) | ((uint32_t)f2bf(x0.w) << 16),
                                    (uint32_t)f2bf(x1.x) | ((uint32_t)f2bf(x1.y) << 16),
                                    (uint32_t)f2bf(x1.z) | ((uint32_t)f2bf(x1.w) << 16));
#pragma unroll
        for (int t = 0; t < TW; ++t)
          if (t == ts && j == jj) kr[t][s4] = kn;
      }
#pragma unroll
      for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t == ts && i == jj) vr[t][i] = vn;
    }
  }
  if (tid == 0) c.s.tclk[2] = (uint32_t)now_ticks();

  // scores: lane (j + 16 rr), element e holds head 4 rr + e at position tb + j
  f4v sc[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    sc[t] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      sc[t] = T::mac(qh[s4], kr[t][s4], sc[t]);
      sc[t] = T::mac(ql[s4], kr[t][s4], sc[t]);
    }
  }
  bool valid[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) valid[t] = p0 + (wave + kWaves * t) * 16 + j < p1;
  float mx[4], ls[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < TW; ++t) m = fmaxf(m, valid[t] ? sc[t][e] : -INFINITY);
    mx[e] = max16(m);
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const float pe = valid[t] ? exp2f(sc[t][e] - mx[e]) : 0.f;
      sc[t][e] = pe;
      l += pe;
    }
    ls[e] = sum16(l);
  }
  // probabilities to LDS, [t][position][head], for the broadcast reads of P V
  float* sw = reinterpret_cast<float*>(c.s.xs);                         // [kWaves][G][DP] wave partials
  float* pb = sw + kWaves * 8 * DP + wave * (TW * 16 * GP);             // this wave's [TW][16][GP]
  if (r < GP / 4) {
#pragma unroll
    for (int t = 0; t < TW; ++t) *reinterpret_cast<f4v*>(pb + (t * 16 + j) * GP + 4 * r) = sc[t];
  }
  float acc[GP][2];
#pragma unroll
  for (int h = 0; h < GP; ++h) acc[h][0] = acc[h][1] = 0.f;
#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v0 = bf_lo(vr[t][i]), v1 = bf_hi(vr[t][i]);
#pragma unroll
      for (int h4 = 0; h4 < GP / 4; ++h4) {
        const f4v pp = *reinterpret_cast<const f4v*>(pb + (t * 16 + i) * GP + 4 * h4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[4 * h4 + e][0] += pp[e] * v0;
          acc[4 * h4 + e][1] += pp[e] * v1;
        }
      }
      // one position at a time: left alone, the compiler sinks every
      // accumulation to the final store and holds all TW * 16 * GP
      // probabilities and V pairs live until then
#pragma unroll
      for (int h = 0; h < GP; ++h) __asm__ volatile("" : "+v"(acc[h][0]), "+v"(acc[h][1]));
    }
  }
  // this wave's partial per head: acc (2 elements per lane), max and sum (uniform)
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    if (h < G) {
      float* dst = sw + (wave * G + h) * DP;
      *reinterpret_cast<float2*>(dst + 2 * lane) = make_float2(acc[h][0], acc[h][1]);
      const int M = __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx[h & 3]), 16 * (h >> 2));
      const int L = __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls[h & 3]), 16 * (h >> 2));
      if (lane == 0) { dst[D] = __builtin_bit_cast(float, M); dst[D + 1] = __builtin_bit_cast(float, L); }
    }
  }
  if (tid == 0) c.s.tclk[3] = (uint32_t)now_ticks();   // wave 0's positions done
  __syncthreads();
  if (tid == 0) c.s.tclk[4] = (uint32_t)now_ticks();   // every wave's
  return attn_finish<D>(c, b, g, ci, tix, nc, G, sw);
}

// Streamed split-K attention for bfloat16 KV with head_dim 128 and at most 8
// query heads per KV head: positions [p0, p1) of request b, KV head g, the
// piece `piece` of the npieces the (b, g) positions were cut into. The piece
// is cut into 16-position tiles dealt to the waves in turn; a wave streams
// its tiles through two register buffers (the next tile's K and V rows load
// while the current one is computed) with an online softmax: a running max
// and sum per head, the accumulators rescaled when the max grows. Scores come
// from the matrix cores as in task_attn_mm (query hi + lo pairs against the
// tile's K rows), P V from the vector ALUs with the probabilities broadcast
// through LDS.
struct AttnTile {
  uint4 k[4];        // lane (j, r): K row j of the tile, elements 32 s + 8 r ..
  uint32_t v[16];    // V rows 0..15 of the tile: this lane's element pair
};

template <int GP>
__device__ __forceinline__ bool task_attn_stream(const Ctx& c, int b, int g, int p0, int p1, int piece, int npieces,
                                                 const int* wev, int wsubs) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  typedef MM<uint16_t> T;
  constexpr int D = 128, DP = D + 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), j = lane & 15, r = lane >> 4;
  const int G = dm.Hq / dm.Hkv;
  const int qkv_dim = (dm.Hq + 2 * dm.Hkv) * D;
  const int S = ldku(a.seq_lens + b);
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.kv) + kv_off(dm, c.l, 0, b, g, 0);
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.kv) + kv_off(dm, c.l, 1, b, g, 0);
  const int pmax = S > 0 ? S - 1 : 0;   // cached slots only (slot S is this step's)
  const int nt = (p1 - p0 + 15) >> 4;   // tiles of the piece
  const int ntw = nt > wave ? (nt - wave + kWaves - 1) / kWaves : 0;   // this wave's: wave, wave + 8, ...
  auto load = [&](AttnTile& t, int i) {
    const int tb = p0 + (wave + kWaves * i) * 16;
    const uint16_t* kp = Kb + (size_t)min(tb + j, pmax) * D + r * 8;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) t.k[s4] = ldg16(kp + s4 * 32);
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) t.v[ii] = ldg4_nt(Vb + (size_t)min(tb + ii, pmax) * D + 2 * lane);
  };
  AttnTile t0, t1;
  if (ntw > 0) load(t0, 0);
  if (ntw > 1) load(t1, 1);
  if (!ctx_wait(c, wev, wsubs)) return false;   // flat counters: QKV[block][group] (all groups: per stage)

  // A operand: query head j of the group (zero beyond G), q * log2(e) / sqrt(d) as hi + lo
  const auto qr = rsrc_n(qkv_of(a, c.l) + (size_t)b * qkv_dim, qkv_dim * 4);
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  uint4 qh[4], ql[4];
  {
    const int qo = j < G ? ((g * G + j) * D + r * 8) * 4 : kNoRecord;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const f4v x0 = ldk4(qr, qo + s4 * 128) * qscale, x1 = ldk4(qr, qo + s4 * 128 + 16) * qscale;
      const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t h0 = f2bf(xv[2 * e]), h1 = f2bf(xv[2 * e + 1]);
        const uint16_t l0 = f2bf(xv[2 * e] - __uint_as_float((uint32_t)h0 << 16));
        const uint16_t l1 = f2bf(xv[2 * e + 1] - __uint_as_float((uint32_t)h1 << 16));
        hw[e] = h0 | ((uint32_t)h1 << 16);
        lw[e] = l0 | ((uint32_t)l1 << 16);
      }
      qh[s4] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      ql[s4] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }
  // position S takes this step's rotated k and v (rounded as the KV append
  // stores them): row jj of this wave's tile iS, if the piece holds S
  int iS = -1, jj = 0;
  uint4 kn[4];
  uint32_t vn = 0;
  if (S >= p0 && S < p1 && ((S - p0) >> 4) % kWaves == wave) {
    iS = ((S - p0) >> 4) / kWaves;
    jj = (S - p0) & 15;
    const int ko = j == jj ? ((dm.Hq + g) * D + r * 8) * 4 : kNoRecord;
    const float2 vv = ldk2(qr, ((dm.Hq + dm.Hkv + g) * D + 2 * lane) * 4);
    vn = (uint32_t)f2bf(vv.x) | ((uint32_t)f2bf(vv.y) << 16);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const f4v x0 = ldk4(qr, ko + s4 * 128), x1 = ldk4(qr, ko + s4 * 128 + 16);
      kn[s4] = make_uint4((uint32_t)f2bf(x0.x) | ((uint32_t)f2bf(x0.y) << 16),
                          (uint32_t)f2bf(x0.z) | ((uint32_t)f2bf(x0.w) << 16),
                          (uint32_t)f2bf(x1.x) | ((uint32_t)f2bf(x1.y) << 16),
                          (uint32_t)f2bf(x1.z) | ((uint32_t)f2bf(x1.w) << 16));
    }
  }
  if (tid == 0) c.s.tclk[2] = (uint32_t)now_ticks();

  float* sw = reinterpret_cast<float*>(c.s.xs);                // [kWaves][G][DP] wave partials
  float* pb = sw + kWaves * 8 * DP + wave * (16 * GP);         // this wave's [16][GP] probabilities
  // running max and sum of head 4 rr + e in row rr's lanes, element e
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, ls[4] = {0.f, 0.f, 0.f, 0.f};
  float acc[GP][2];
#pragma unroll
  for (int h = 0; h < GP; ++h) acc[h][0] = acc[h][1] = 0.f;
  auto process = [&](AttnTile& t, int i) {
    if (i == iS) {   // uniform
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        if (j == jj) t.k[s4] = kn[s4];
#pragma unroll
      for (int ii = 0; ii < 16; ++ii)
        if (ii == jj) t.v[ii] = vn;
    }
    f4v sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      sc = T::mac(qh[s4], t.k[s4], sc);
      sc = T::mac(ql[s4], t.k[s4], sc);
    }
    const bool valid = p0 + (wave + kWaves * i) * 16 + j < p1;
    float scale[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float mn = fmaxf(mx[e], max16(valid ? sc[e] : -INFINITY));
      scale[e] = mx[e] == -INFINITY ? 0.f : exp2f(mx[e] - mn);
      const float pe = valid ? exp2f(sc[e] - mn) : 0.f;
      ls[e] = ls[e] * scale[e] + sum16(pe);
      mx[e] = mn;
      sc[e] = pe;
    }
    if (r < GP / 4) *reinterpret_cast<f4v*>(pb + j * GP + 4 * r) = sc;
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float f = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, scale[h & 3]),
                                                                          16 * (h >> 2)));
      acc[h][0] *= f;
      acc[h][1] *= f;
    }
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      const float v0 = bf_lo(t.v[ii]), v1 = bf_hi(t.v[ii]);
#pragma unroll
      for (int h4 = 0; h4 < GP / 4; ++h4) {
        const f4v pp = *reinterpret_cast<const f4v*>(pb + ii * GP + 4 * h4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[4 * h4 + e][0] += pp[e] * v0;
          acc[4 * h4 + e][1] += pp[e] * v1;
        }
      }
      // one position at a time (left alone, the compiler sinks the
      // accumulations and holds every probability and V pair live)
#pragma unroll
      for (int h = 0; h < GP; ++h) __asm__ volatile("" : "+v"(acc[h][0]), "+v"(acc[h][1]));
    }
  };
  // two buffers: while one tile is computed the next one's rows load; the
  // main loop is branch-free so its waits stay exact, the tail handles the
  // last one to three tiles
  int i = 0;
  for (; i + 3 < ntw; i += 2) {
    process(t0, i);
    load(t0, i + 2);
    process(t1, i + 1);
    load(t1, i + 3);
  }
  if (i < ntw) {
    process(t0, i);
    if (i + 2 < ntw) load(t0, i + 2);
  }
  if (i + 1 < ntw) process(t1, i + 1);
  if (i + 2 < ntw) process(t0, i + 2);

  // this wave's partial per head: acc (2 elements per lane), max and sum
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    if (h < G) {
      float* dst = sw + (wave * G + h) * DP;
      *reinterpret_cast<float2*>(dst + 2 * lane) = make_float2(acc[h][0], acc[h][1]);
      const int M = __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx[h & 3]), 16 * (h >> 2));
      const int L = __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls[h & 3]), 16 * (h >> 2));
      if (lane == 0) { dst[D] = __builtin_bit_cast(float, M); dst[D + 1] = __builtin_bit_cast(float, L); }
    }
  }
  if (tid == 0) c.s.tclk[3] = (uint32_t)now_ticks();   // wave 0's positions done
  __syncthreads();
  if (tid == 0) c.s.tclk[4] = (uint32_t)now_ticks();   // every wave's
  return attn_finish<D>(c, b, g, piece, 0, npieces, G, sw);
}

template <typename KT, int HB>
__device__ __forceinline__ bool attn_its(const Ctx& c, int b, int g, int ci, int tix, int ck, const int* wev, int wsubs) {
  if (ck <= 64) return task_attn<KT, HB, 2>(c, b, g, ci, tix, wev, wsubs);
  if (ck <= 128) return task_attn<KT, HB, 4>(c, b, g, ci, tix, wev, wsubs);
  // 256-position chunks hold 16 KV rows per lane: two query heads at a time keep them in registers
  return task_attn<KT, (HB > 2 ? 2 : HB), 8>(c, b, g, ci, tix, wev, wsubs);
}

template <typename KT>
__device__ __forceinline__ bool attn_dispatch(const Ctx& c, int b, int g, int ci, int tix, const int* wev, int wsubs) {
  const int G = c.a.dm.Hq / c.a.dm.Hkv, ck = c.a.attn_chunk;
  if constexpr (sizeof(KT) == 2) {
    // bfloat16 caches: decode_layer_init admits head_dim 128 with at most 8
    // query heads per KV head only, all on the matrix cores
    if (G <= 4)
      return ck > 128 ? task_attn_mm<2, 4>(c, b, g, ci, tix, wev, wsubs) : task_attn_mm<1, 4>(c, b, g, ci, tix, wev, wsubs);
    return ck > 128 ? task_attn_mm<2, 8>(c, b, g, ci, tix, wev, wsubs) : task_attn_mm<1, 8>(c, b, g, ci, tix, wev, wsubs);
  } else {
    if (G >= 4) return attn_its<KT, 4>(c, b, g, ci, tix, ck, wev, wsubs);
    if (G == 2) return attn_its<KT, 2>(c, b, g, ci, tix, ck, wev, wsubs);
    return attn_its<KT, 1>(c, b, g, ci, tix, ck, wev, wsubs);
  }
}

// ---------------------------------------------------------------------------
// MoE routing and combine
// ---------------------------------------------------------------------------

// Wave-wide inclusive prefix sum.
__device__ __forceinline__ int wave_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Top-k, gates and expert grouping for all tokens (one workgroup).
//   topk:     per token, the k largest float32 logits ordered by (logit desc,
//             index asc): ties go to the lower expert index;
//   gates:    softmax over the k selected logits;
//   grouping: exp_indptr = prefix sum of per-expert routed rows (last = T k),
//             tile_indptr = prefix sum of ceil(count / kMoeBM), sorted_tok /
//             sorted_slot = routed (token, slot) ordered by expert then token;
//   arming:   the counter of expert e starts at e's number of gate/up tasks
//             (its row tiles x gate/up slices) -- the data-dependent event.
// A logit as an unsigned key whose order is the float order (-0 taken as +0).
__device__ __forceinline__ uint32_t ord_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// Largest (hi, lo) pair over each row of 16 lanes, every lane of the row gets it.
template <int CTRL> __device__ __forceinline__ void key_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t oh = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, CTRL, 0xF, 0xF, false);
  const uint32_t ol = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, CTRL, 0xF, 0xF, false);
  const bool take = oh > hi || (oh == hi && ol > lo);
  hi = take ? oh : hi;
  lo = take ? ol : lo;
}
// Over groups of GS = 16 lanes (a row) or 64 (the wave).
template <int GS> __device__ __forceinline__ void key_max(uint32_t& hi, uint32_t& lo) {
  key_step<0xB1>(hi, lo);
  key_step<0x4E>(hi, lo);
  key_step<0x141>(hi, lo);
  key_step<0x140>(hi, lo);
  if constexpr (GS == 64) {
    auto cross = [&](auto swap) {
      float ah = __uint_as_float(hi), bh = ah, al = __uint_as_float(lo), bl = al;
      swap(ah, bh);
      swap(al, bl);
      const uint32_t h0 = __float_as_uint(ah), l0 = __float_as_uint(al);
      const uint32_t h1 = __float_as_uint(bh), l1 = __float_as_uint(bl);
      const bool take = h1 > h0 || (h1 == h0 && l1 > l0);
      hi = take ? h1 : h0;
      lo = take ? l1 : l0;
    };
    cross([](float& x, float& y) { swap16(x, y); });
    cross([](float& x, float& y) { swap32(x, y); });
  }
}

// GS lanes per token (16 while the experts fit 8 per lane, else the wave).
template <int GS>
__device__ __forceinline__ bool task_route(const Ctx& c, const int* wev) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  if (!ctx_wait(c, wev)) return false;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int T = a.batch, E = dm.E, k = dm.k, Tk = T * k, G = dm.grid, TW = (T + 31) >> 5;
  int* sidx = reinterpret_cast<int*>(c.s.xs);   // [T k]
  int* cnt = sidx + dm.max_batch * kMaxTopK;     // [E]
  int* ptr = cnt + kMaxExperts;                  // [E + 1]
  int* tptr = ptr + kMaxExperts + 1;             // [E + 1]
  // [TW][E]: bit t % 32 of word (t / 32, e) is set when token t selected e
  // (expert-fastest, so that lanes on different experts read different banks)
  uint32_t* sel = reinterpret_cast<uint32_t*>(tptr + kMaxExperts + 1);
  for (int i = tid; i < E * TW; i += kBlock) sel[i] = 0;
  __syncthreads();
  // top-k: a token per group of GS lanes, lane r of the group holding experts
  // r, r + GS, ...; k rounds of a group-wide maximum of (logit, -index) keys.
  // The next tokens' logits are loaded while these are selected.
  constexpr int EPG = 8, TPW = 64 / GS;   // experts per lane, tokens per wave
  const int row = lane / GS, rl = lane % GS, ng = (E + GS - 1) / GS;
  // branch-free, so that a round's loads are all in flight together: a token
  // past T, or an expert past E, reads past the descriptor's range (zeros)
  const auto lr = rsrc_n(a.ws.logits, T * E * 4);
  auto load = [&](int t, float (&z)[EPG]) {
#pragma unroll
    for (int i = 0; i < EPG; ++i) {
      const int e = rl + GS * i;
      z[i] = ldc1(lr, (i < ng && e < E) ? (t * E + e) * 4 : kNoRecord);
    }
  };
  float z[EPG];
  load(wave * TPW + row, z);
  for (int t0 = wave * TPW; t0 < T; t0 += kWaves * TPW) {
    const int t = t0 + row;
    float zn[EPG];
    load(t + kWaves * TPW, zn);
    // each lane's candidates as 64-bit (logit order, ~index) keys, 0 (below
    // every valid key) for none; a selected key is cleared by its lane. No
    // branch per candidate: with one, the selection was ~350 instructions per
    // selected expert, and the rounds ran at ~7 us per 32 tokens.
    uint64_t key[EPG];
#pragma unroll
    for (int i = 0; i < EPG; ++i) {
      const int e = rl + GS * i;
      key[i] = (i < ng && e < E) ? ((uint64_t)ord_key(z[i]) << 32) | (uint32_t)~(uint32_t)e : 0ull;
    }
    float zsel[kMaxTopK];
    int isel[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      zsel[j] = 0.f;
      isel[j] = 0;
      if (j >= k) continue;
      uint64_t b = key[0];
#pragma unroll
      for (int i = 1; i < EPG; ++i) b = key[i] > b ? key[i] : b;
      uint32_t bh = (uint32_t)(b >> 32), bl = (uint32_t)b;
      key_max<GS>(bh, bl);
      const uint64_t win = ((uint64_t)bh << 32) | bl;
#pragma unroll
      for (int i = 0; i < EPG; ++i) key[i] = key[i] == win ? 0ull : key[i];
      zsel[j] = key_value(bh);
      isel[j] = (int)~bl;
    }
    if (t < T) {
      if (rl == 0) {
        float w[kMaxTopK], sum = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
          w[j] = j < k ? __expf(zsel[j] - zsel[0]) : 0.f;
          sum += w[j];
        }
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
          if (j < k) {
            sidx[t * k + j] = isel[j];
            stc(a.ws.topk_w + t * k + j, w[j] / sum);
          }
        }
      }
      int mine = 0;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) mine = rl == j ? isel[j] : mine;
      if (rl < k) atomicOr(&sel[(t >> 5) * E + mine], 1u << (t & 31));
    }
#pragma unroll
    for (int i = 0; i < EPG; ++i) z[i] = zn[i];
  }
  __syncthreads();
  for (int e = tid; e < E; e += kBlock) {
    int n = 0;
    for (int w = 0; w < TW; ++w) n += __popc(sel[w * E + e]);
    cnt[e] = n;
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0, tcarry = 0;
    if (lane == 0) { ptr[0] = 0; tptr[0] = 0; }
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int v = e < E ? cnt[e] : 0, tv = (v + kMoeBM - 1) / kMoeBM;
      const int s = wave_scan(v) + carry, ts = wave_scan(tv) + tcarry;
      if (e < E) { ptr[e + 1] = s; tptr[e + 1] = ts; }
      carry = __shfl(s, 63, 64);
      tcarry = __shfl(ts, 63, 64);
    }
  }
  __syncthreads();
  const int ntiles = tptr[E];
  // gate/up slices of Fe and down slices of H per row tile: about two tasks
  // per workgroup, each slice at least 16 rows and at most what the LDS holds
  // of a pass's outputs for 16 token rows beside the rows it stages (a pass's
  // outputs follow its staged rows: make_pass). Where the row tiles hold fewer
  // than 4 tokens on average, the passes are weight streams like a small
  // dense batch, and slices of at most 2048 outputs (more, smaller tasks)
  // spread the weights more evenly over the workgroups (measured: 16 tokens
  // 4 % faster; 128 and 1024 tokens 5 % slower than with the LDS bound).
  auto out_floats = [&](int K) {
    const int rowb = ((K + dm.kstep - 1) / dm.kstep * dm.kstep + dm.xpad) * 4;
    const int room = (kXyBytes - (kMaxNb * rowb + 15) / 16 * 16) / 4;
    return Tk >= 4 * ntiles ? room : min(room, kYsFloats);
  };
  const int target = (2 * G + ntiles - 1) / ntiles;
  const int rows_g = out_floats(dm.H) / (2 * kMaxNb), rows_d = out_floats(dm.Fe) / kMaxNb;   // per slice at most
  const int sg = min(max(target, (dm.Fe + rows_g - 1) / rows_g), max(dm.Fe / 16, 1));
  const int sd = min(max(target, (dm.H + rows_d - 1) / rows_d), max(dm.H / 16, 1));
  // scatter in (expert, token) order: (t, j) goes after the tokens below t
  // that selected the same expert (a token selects an expert at most once)
  for (int i = tid; i < Tk; i += kBlock) {
    const int t = i / k, e = sidx[i];
    int rank = __popc(sel[(t >> 5) * E + e] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(sel[w * E + e]);
    const int pos = ptr[e] + rank;
    stci(a.ws.sorted_tok + pos, t);
    stci(a.ws.sorted_slot + pos, i - t * k);
    stci(a.ws.pos_of + i, pos);
  }
  for (int e = tid; e < E; e += kBlock) {
    for (int tt = tptr[e]; tt < tptr[e + 1]; ++tt) {
      stci(a.ws.tile_info + 2 * tt, e);
      stci(a.ws.tile_info + 2 * tt + 1, ptr[e] + (tt - tptr[e]) * kMoeBM);
    }
    stci(a.ws.ectr + ((size_t)c.l * E + e) * kCtr, (tptr[e + 1] - tptr[e]) * sg);
    stci(a.ws.exp_indptr + e + 1, ptr[e + 1]);
    stci(a.ws.tile_ptr + e + 1, tptr[e + 1]);
  }
  if (a.moe_dyn) {   // this layer's task queue: empty, nothing popped or pushed yet
    for (int i = tid; i < ntiles * sd; i += kBlock) stci(a.ws.rq + (size_t)c.l * dm.max_down + i, 0);
    if (tid < kMq) stci(a.ws.mq + ((size_t)c.l * kMq + tid) * kCtr, 0);
  }
  for (int i = tid; i < Tk; i += kBlock) stci(a.ws.topk_idx + i, sidx[i]);
  if (tid == 0) {
    stci(a.ws.exp_indptr, 0);
    stci(a.ws.tile_ptr, 0);
    stci(a.ws.moe_info + 0, ntiles * sg);
    stci(a.ws.moe_info + 1, ntiles * sd);
    stci(a.ws.moe_info + 2, sg);
    stci(a.ws.moe_info + 3, sd);
    stci(a.ws.moe_info + 4, ntiles);
  }
  // routing outputs of the last layer for the caller
  if (c.l == dm.L - 1) {
    const pmk_routing& r = a.rout;
    for (int i = tid; i < Tk; i += kBlock) {
      if (r.topk_idx) *gp(r.topk_idx + i) = sidx[i];
      if (r.topk_w) *gp(r.topk_w + i) = ldc(a.ws.topk_w + i);
    }
    if (r.router_logits)
      for (int i = tid; i < T * E; i += kBlock) *gp(r.router_logits + i) = ldc(a.ws.logits + i);
    for (int e = tid; e <= E; e += kBlock) {
      if (r.exp_indptr) *gp(r.exp_indptr + e) = ptr[e];
      if (r.tile_indptr) *gp(r.tile_indptr + e) = tptr[e];
    }
  }
  // the scattered order is read back once the stores above have landed
  vm_drain();
  __syncthreads();
  if (c.l == dm.L - 1 && (a.rout.sorted_tok || a.rout.sorted_slot)) {
    for (int i = tid; i < Tk; i += kBlock) {
      if (a.rout.sorted_tok) *gp(a.rout.sorted_tok + i) = ldci(a.ws.sorted_tok + i);
      if (a.rout.sorted_slot) *gp(a.rout.sorted_slot + i) = ldci(a.ws.sorted_slot + i);
    }
  }
  wg_notify(c.nev, -1);
  return true;
}

// Per-token combine: x'_t = h1_t + sum_j w_tj * Y[pos(t, j)], slots in order j = 0..k-1.
__device__ __forceinline__ bool task_combine(const Ctx& c, const int* wev) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  if (!ctx_wait(c, wev)) return false;
  const auto mo = rsrc(a.ws.mout);   // routed rows: T k H floats, < 2 GiB
  for (int t = c.wg; t < a.batch; t += dm.grid) {
    for (int i = threadIdx.x; i < dm.H / 4; i += kBlock) {
      f4v x = ldk4(rsrc(h1_of(a, c.l) + (size_t)t * dm.H), i * 16);
      for (int j = 0; j < dm.k; ++j) {
        const float w = ldc(a.ws.topk_w + t * dm.k + j);
        const int p = ldci(a.ws.pos_of + t * dm.k + j);
        x += ldc4(mo, (p * dm.H) * 4 + i * 16) * w;
      }
      stc4(rsrc(hid_out(a, c.l) + (size_t)t * dm.H), i * 16, x);
    }
  }
  return true;
}

// ---------------------------------------------------------------------------
// The per-op schedule's separate operators. Each runs in a launch of its own
// (the kernel boundary orders it after the previous op), and every workgroup
// takes a grid-stride share of the op's elements. They compute what the fused
// tasks fold into the projections: the RMSNorms, RoPE, the K/V append and the
// merge of the attention partials.
// ---------------------------------------------------------------------------
// u = x g / sqrt(mean(x^2) + eps) for every request row (x: the layer input,
// or h1 for the second norm); one row per workgroup at a time.
__device__ __forceinline__ bool task_norm(const Ctx& c, bool ffn) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const float* x = ffn ? h1_of(a, c.l) : hid_in(a, c.l);
  const float* g = ffn ? ldp(&a.layers[c.l].ffn_norm) : ldp(&a.layers[c.l].attn_norm);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  __syncthreads();
  for (int b = c.wg; b < a.batch; b += dm.grid) {
    const float* xr = x + (size_t)b * dm.H;
    float ss = 0.f;
    for (int i = tid; i < dm.H; i += kBlock) {
      const float v = ldc(xr + i);
      ss += v * v;
    }
    ss = wave_sum(ss);
    if (lane == 0) c.s.red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < kWaves; ++w) tot += c.s.red[w];
    const float r = 1.0f / sqrtf(tot / (float)dm.H + dm.eps);
    for (int i = tid; i < dm.H; i += kBlock) stc(a.ws.u + (size_t)b * dm.H + i, ldc(xr + i) * r * g[i]);
    __syncthreads();
  }
  return true;
}

// RoPE in place on the projected q and k heads: pair (i, i + d/2) of head h of
// request b turned by the angle of position seq_lens[b] (the host-built table).
__device__ __forceinline__ bool task_rope(const Ctx& c) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const int half = dm.d >> 1, nh = dm.Hq + dm.Hkv, qkv_dim = (dm.Hq + 2 * dm.Hkv) * dm.d;
  const long n = (long)a.batch * nh * half;
  float* q = qkv_of(a, c.l);
  for (long t = (long)c.wg * kBlock + threadIdx.x; t < n; t += (long)dm.grid * kBlock) {
    const int b = (int)(t / (nh * half)), r = (int)(t - (long)b * nh * half), h = r / half, i = r - h * half;
    const int pos = *gp(a.seq_lens + b);
    const float2 cs = a.ws.rope[(size_t)pos * half + i];
    float* z = q + (size_t)b * qkv_dim + h * dm.d + i;
    const float y1 = ldc(z), y2 = ldc(z + half);
    stc(z, y1 * cs.x - y2 * cs.y);
    stc(z + half, y2 * cs.x + y1 * cs.y);
  }
  return true;
}

// The new K and V rows of every request into its cache slot seq_lens[b],
// rounded to the cache dtype (nearest even).
template <typename KT>
__device__ __forceinline__ bool task_append(const Ctx& c) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const int qkv_dim = (dm.Hq + 2 * dm.Hkv) * dm.d;
  const long n = (long)a.batch * 2 * dm.Hkv * dm.d;
  const float* q = qkv_of(a, c.l);
  for (long t = (long)c.wg * kBlock + threadIdx.x; t < n; t += (long)dm.grid * kBlock) {
    const int b = (int)(t / (2 * dm.Hkv * dm.d)), r = (int)(t - (long)b * 2 * dm.Hkv * dm.d);
    const int kvh = r / dm.d, e = r - kvh * dm.d, which = kvh / dm.Hkv, g = kvh - which * dm.Hkv;
    const int pos = *gp(a.seq_lens + b);
    const float v = ldc(q + (size_t)b * qkv_dim + (dm.Hq + kvh) * dm.d + e);
    Elem<KT>::put(reinterpret_cast<KT*>(a.kv) + kv_off(dm, c.l, which, b, g, pos) + e, v);
  }
  return true;
}

// o of every (request, KV head): the log-sum-exp merge of the chunk partials
// (acc, max, sum per query head, log2 units) the attention op left in part.
__device__ __forceinline__ bool task_merge(const Ctx& c) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const int D = dm.d, DP = D + 4, G = dm.Hq / dm.Hkv, ck = a.attn_chunk;
  for (int bg = c.wg; bg < a.batch * dm.Hkv; bg += dm.grid) {
    const int b = bg / dm.Hkv, g = bg - b * dm.Hkv;
    const int nc = (*gp(a.seq_lens + b) + ck) / ck;
    const float* part = a.ws.part + ((size_t)b * dm.Hkv + g) * dm.max_chunks * G * DP;
    float* o = o_of(a, c.l) + (size_t)b * dm.Hq * D + (size_t)g * G * D;
    for (int t = threadIdx.x; t < G * D; t += kBlock) {
      const int h = t / D, e = t - h * D;
      float M = -INFINITY;
      for (int cc = 0; cc < nc; ++cc) M = fmaxf(M, ldc(part + (cc * G + h) * DP + D));
      float L = 0.f, A = 0.f;
      for (int cc = 0; cc < nc; ++cc) {
        const float* p = part + (cc * G + h) * DP;
        const float f = exp2f(ldc(p + D) - M);
        L += ldc(p + D + 1) * f;
        A += ldc(p + e) * f;
      }
      stc(o + t, A / L);
    }
  }
  return true;
}

// ---------------------------------------------------------------------------
// The persistent kernel
// ---------------------------------------------------------------------------
// Task types that run as GEMV passes.
__device__ __forceinline__ bool gemv_task(int type) {
  return type == T_QKV || type == T_O || type == T_GU || type == T_DOWN || type == T_ROUTER || type == T_MGU ||
         type == T_MDOWN;
}
// Stage of a task type within its layer, in queue order.
__device__ __forceinline__ int stage_of(int type) {
  switch (type) {
    case T_QKV: return 0;
    case T_ATTN: case T_ATTS: return 1;
    case T_O: return 2;
    case T_GU: case T_ROUTER: return 3;
    case T_DOWN: case T_ROUTE: return 4;
    case T_MGU: return 5;
    case T_MDOWN: return 6;
    default: return 7;
  }
}

// kPart: a launch of an ablation schedule, which runs the layers and task
// types `rs` names, with a grid-wide barrier after every stage if rs.barrier;
// the fused launch (kPart false) runs everything, chained by events alone.
// Copy a device error into the host mirror (system scope: the host reads it
// without synchronising). Called by one thread.
__device__ __forceinline__ void mirror_error(const StepArgs& a, int e) {
  if (e != 0 && a.ws.err_host)
    __hip_atomic_store(a.ws.err_host, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <typename WT, bool kPart, int KP>
__device__ __forceinline__ void main_body(const StepArgs& a, RunSpec rs, char* lds_raw);

template <typename WT, bool kPart, int KP>
__global__ void __launch_bounds__(kBlock, 1) pmk_main(const StepArgs* __restrict__ pa, RunSpec rs) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  main_body<WT, kPart, KP>(*pa, rs, lds_raw);
  // every exit path ends here: a workgroup that leaves with the error word set
  // (a watchdog expiry anywhere in the grid) copies it to the host mirror
  if (threadIdx.x == 0) mirror_error(*pa, ldci(pa->ws.err));
}

template <typename WT, bool kPart, int KP>
__device__ __forceinline__ void main_body(const StepArgs& a, RunSpec rs, char* lds_raw) {
  const Dims& dm = a.dm;
  const int wg = blockIdx.x, wave = wave_id();
  const Lds s = lds_layout(lds_raw);
  if (threadIdx.x == 0) *s.flag = (ldci(a.ws.err) == 0);
  if (threadIdx.x < 8) s.seen[threadIdx.x] = 0;
  if (threadIdx.x < 3) s.rope_key[threadIdx.x] = 0;
  if (threadIdx.x < kMaxNb) s.rope_pos[threadIdx.x] = 0;
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(*s.flag)) return;
  const int n = ldku(a.ws.qlen + wg);
  const int4* q = a.ws.queue + (size_t)wg * dm.max_queue;
  const int4* qe = a.ws.qev + (size_t)wg * dm.max_queue;
  uint32_t* tr = a.trace ? a.trace + (size_t)wg * a.trace_cap * 8 : nullptr;
  // records accumulate over the launches of a step (the prologue zeroes the counts)
  int tn = tr ? ldu(reinterpret_cast<const int*>(tr)) + 1 : 1;
  const int l_end = kPart ? rs.l1 : dm.L;
  auto mine = [&](int type) { return !kPart || ((rs.types >> type) & 1u); };
  int l = kPart ? rs.l0 : 0, t = 0;
  // barrier schedule: barrier i = l * ns + stage is passed once every
  // workgroup has finished its tasks of that stage; `arrived` counts the
  // barriers this workgroup has arrived at (it arrives at every one, waits on
  // the last before its first task of a later stage, and arrives at the rest
  // when its queue ends)
  const bool bars = kPart && rs.barrier;
  const int ns = dm.moe ? kMaxStages : 5;
  int arrived = 0;
  auto barrier_to = [&](int bi) -> bool {
    if (arrived >= bi) return true;
    for (; arrived < bi; ++arrived) wg_notify(a.ws.bar + (size_t)arrived * kEvInts, wg & (kSubs - 1));
    return ctx_wait(Ctx{a, l, wg, s}, a.ws.bar + (size_t)(bi - 1) * kEvInts, kSubs);
  };
  // The events this workgroup has seen fired, one per wait kind (s.seen[k] =
  // key of the last event waited on, key = offset / kCtr + 1 + (counters - 1)
  // << 24: event offsets are multiples of kCtr below 2^27, waits span at most
  // kMaxHkv counters),
  // so a later task that waits on the same event does not poll it again.
  // Every wave records the key after its task's wait and reads it before the
  // next task, so all waves agree.
  enum : int { W_QKV = 0, W_ATTN, W_O, W_GU, W_DOWN, W_ROUTER, W_ROUTE, W_MDOWN };
  auto key_of = [](long off, int subs) { return (int)(off / kCtr) + 1 + (subs << 24); };
  int pend_kind = -1, pend_key = 0;   // the wait the current task performs (recorded once it has)
  // the event (offset `off`, counters off .. off + subs kCtr) a task waits on,
  // or nullptr when this workgroup has already seen it fired
  auto need = [&](int kind, long off, int subs) -> const int* {
    const int key = key_of(off, subs);
    if (s.seen[kind] == key) return nullptr;
    pend_kind = kind;
    pend_key = key;
    return a.ws.ev + off;
  };
  auto seen_done = [&]() {
    if (pend_kind >= 0) s.seen[pend_kind] = pend_key;
    pend_kind = -1;
  };
  // whether this workgroup has seen event `off` fired
  auto seen = [&](int kind, long off, int subs) -> bool { return s.seen[kind] == key_of(off, subs); };
  // the wait of a task as its queue entry gives it (pmk_sched.h:
  // task_events): the event pointer of this layer and its extra counters,
  // nullptr when there is none or this workgroup has already seen it fired
  const long LI = ev_layer_ints(dm);
  auto wait_of = [&](const int4& te, int type, int& subs) -> const int* {
    subs = kSubs;
    if (te.y < 0 || (l == 0 && type == T_QKV)) return nullptr;
    subs = te.y & 0xffff;
    return need(te.y >> 16, te.x + l * LI, subs);
  };
  auto notify_ev = [&](const int4& te) -> int* { return te.z >= 0 ? a.ws.ev + te.z + l * LI : nullptr; };
  auto advance = [&]() {
    if (++t == n) {
      t = 0;
      ++l;
    }
  };
  auto record = [&](int type, uint32_t t_begin) {
    if (tr && threadIdx.x == 0 && tn < a.trace_cap) {
      const uint32_t t_end = (uint32_t)now_ticks();
      __attribute__((address_space(1))) uint32_t* e = gp(tr + (size_t)tn * 8);
      e[0] = (uint32_t)type | ((uint32_t)l << 8) | ((uint32_t)(ldku4(q + t).y & 0xffff) << 16);
      e[1] = t_begin;
#pragma unroll
      for (int i = 1; i < 6; ++i) e[1 + i] = s.tclk[i];
      e[7] = t_end;
      ++tn;
    }
  };
  auto begin = [&]() -> uint32_t {
    const uint32_t t0 = (uint32_t)now_ticks();
    if (tr && threadIdx.x == 0)
      for (int i = 1; i < 7; ++i) s.tclk[i] = t0;
    return t0;
  };
  if (n > 0) {
    while (l < l_end) {
      int4 task = ldku4(q + t);
      int4 te = ldku4(qe + t);
      const int tix = task.x >> 8;   // attention tasks: the task's index within the stage
      task.x &= 0xff;
      if (!mine(task.x)) {   // not this launch's (a per-stage schedule)
        advance();
        continue;
      }
      if (bars && !barrier_to(l * ns + stage_of(task.x))) return;
      if (!gemv_task(task.x)) {
        const Ctx c{a, l, wg, s, notify_ev(te)};
        const uint32_t t_begin = begin();
        bool ok = true;
        switch (task.x) {
          case T_ATTN: {   // (b, g): waits on the QKV tiles of its block and group alone
            int subs;
            const int* wev = wait_of(te, T_ATTN, subs);
            ok = attn_dispatch<WT>(c, task.y, task.z, task.w, tix, wev, subs);
            break;
          }
          case T_ATTS: {   // x: piece << 8 | pieces << 20, y: b | g << 16, z/w: positions [z, w)
            const int b = task.y & 0xffff, g = task.y >> 16, piece = tix & 0xfff, np = tix >> 12;
            int subs;
            const int* wev = wait_of(te, T_ATTS, subs);
            if constexpr (sizeof(WT) == 2) {
              ok = dm.Hq / dm.Hkv <= 4 ? task_attn_stream<4>(c, b, g, task.z, task.w, piece, np, wev, subs)
                                       : task_attn_stream<8>(c, b, g, task.z, task.w, piece, np, wev, subs);
            }
            break;
          }
          case T_ROUTE:
            if constexpr ((KP & 3) != KP_DENSE) {
              int subs;
              const int* wev = wait_of(te, T_ROUTE, subs);
              ok = dm.E <= 128 ? task_route<16>(c, wev) : task_route<64>(c, wev);
            }
            break;
          case T_COMBINE:
            if constexpr ((KP & 3) != KP_DENSE) {
              int subs;
              ok = task_combine(c, wait_of(te, T_COMBINE, subs));
              if (ok) wg_notify(c.nev, -1);
            }
            break;
          case T_NORM1: case T_NORM2: case T_ROPE: case T_APPEND: case T_MERGE:
            if constexpr (kPart && (KP & 3) == KP_ALL) {
              switch (task.x) {
                case T_NORM1: ok = task_norm(c, false); break;
                case T_NORM2: ok = task_norm(c, true); break;
                case T_ROPE: ok = task_rope(c); break;
                case T_APPEND: ok = task_append<WT>(c); break;
                default: ok = task_merge(c); break;
              }
              __syncthreads();
            }
            break;
          default: break;
        }
        if (!ok) return;
        seen_done();
        record(task.x, t_begin);
        advance();
        continue;
      }
      // a run of consecutive GEMV tasks (across layers too)
      for (;;) {
        const Ctx c{a, l, wg, s, notify_ev(te)};
        const uint32_t t_begin = begin();
        bool ok = true;
        const int* wev = nullptr;
        int wsubs = kSubs;
        // dense tasks: y = row tile, z = K slice, w = batch block; their block's events
        const int eb = (task.x == T_QKV || task.x == T_O || task.x == T_GU || task.x == T_DOWN)
                           ? (ldku(&a.nblk) > 1 ? task.w : 0) : 0;
        // its wait (the queue entry's: pmk_sched.h, task_events)
        if (task.x == T_MGU) {   // the share's size is known once routing is done
          ok = ctx_wait(c, wait_of(te, T_MGU, wsubs), kSubs);
        } else if (task.x != T_MDOWN) {
          wev = wait_of(te, task.x, wsubs);
        }
        bool done = true;   // this task finished its row tile (not so for a split-K slice that was not the last)
        bool split_last = false;   // it finished a split tile as its last slice task (a split task has one pass)
        for (int p = 0; ok; ++p) {
          Pass ps;
          if (!make_pass<WT, KP>(c, task, p, wev, ps)) break;
          if (ps.wev == wev) ps.wsubs = wsubs;
          // the residual of O (the layer input) / down (h1) is final once this
          // workgroup has seen the event that produced it, or one that fires
          // only after it (every QKV tile waits for the previous layer's down
          // stage): load it before waiting
          float resid[kResid];
          // (block eb of layer l's input: its down event of layer l - 1, or a QKV
          // event of its block, whose tiles waited on that down event)
          auto qkv_seen = [&]() {
            const long k = (long)(s.seen[W_QKV] - 1) * kCtr;
            return k >= ev_off(dm, l, EV_QKV, eb, 0) && k < ev_off(dm, l, EV_QKV, eb, dm.Hkv);
          };
          const bool early = ps.R * ps.nb <= kYsFloats &&
                             ((ps.epi == E_O && (l == 0 || seen(W_DOWN, ev_off(dm, l - 1, EV_DOWN, eb), kSubs) ||
                                                 qkv_seen())) ||
                              (ps.epi == E_DOWN && seen(W_O, ev_off(dm, l, EV_O, eb), kSubs)));
          if (early) load_resid(a, ps, resid);
          ok = gemv_any<WT, (KP & KP_TILES) != 0>(c, ps.rw, ps.R, ps.K, ps.in, ps.nb, ps.wev, ps.wsubs, ps.ys);
          if (!ok) break;
          seen_done();
          if (ps.ks > 1 && !reduce_slices(c, ps)) {
            done = false;
            break;
          }
          split_last = ps.ks > 1;
          if (early) add_resid(ps, resid);
          // a split tile's last slice task is its stage's critical path: every
          // wave stores the outputs and the workgroup notifies together,
          // before any wave issues the next task's weight loads (those would
          // hold the stores back in the compute unit's memory queue)
          if (split_last || wave == 0) {
            const int t0 = split_last ? (int)threadIdx.x : (int)(threadIdx.x & 63);
            epilogue<WT, KP>(c, ps, early, t0, split_last ? kBlock : 64);
          }
          if (threadIdx.x == 0) s.tclk[5] = (uint32_t)now_ticks();
        }
        if (!ok) return;
        // dense stages notify per row tile (by the last slice of a split tile),
        // the others per workgroup: the counter(s) of the queue entry (a QKV
        // tile, the flat counter of each KV group its units cover)
        if (done && c.nev && (split_last || wave == 0)) {
          if (split_last) {
            vm_drain();
            __syncthreads();
          } else {
            vm_drain();
          }
          if ((threadIdx.x & (split_last ? kBlock - 1 : 63)) == 0)
            for (int i = 0; i < te.w; ++i) (void)atomic_add_relaxed(c.nev + i * kCtr, -1);
        }
        record(task.x, t_begin);
        advance();
        if (l >= l_end || bars) break;
        task = ldku4(q + t);
        te = ldku4(qe + t);
        task.x &= 0xff;
        if (!gemv_task(task.x) || !mine(task.x)) break;
      }
    }
  }
  if (bars)   // the last barrier has no waiter
    for (; arrived < dm.L * ns - 1; ++arrived) wg_notify(a.ws.bar + (size_t)arrived * kEvInts, wg & (kSubs - 1));
  if (tr && threadIdx.x == 0) *gp(tr) = (uint32_t)(tn - 1);
}

// ---------------------------------------------------------------------------
// The per-step prologue: validate lengths, build queues, arm events.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) pmk_prologue(StepArgs a) {
  const Dims& dm = a.dm;
  const int tid = threadIdx.x, B = a.batch, G = dm.grid;
  __shared__ int bad;
  __shared__ Plan plan;
  __shared__ int gtiles[kMaxHkv];   // QKV row tiles meeting each KV group
  __shared__ int cb[kMaxBatchAll + 1];
  __shared__ int sl[kMaxBatchAll];   // the requests' lengths, read once
  StepArgs* copy = reinterpret_cast<StepArgs*>(a.ws.args);
  if (tid == 0) {
    // the persistent kernel reads this step's arguments from here, on every
    // path (it first checks the error word through it)
    *copy = a;
    bad = (ldci(a.ws.err) != 0) ? 1 : 0;
  }
  __syncthreads();
  for (int b = tid; b < B; b += blockDim.x) {
    const int s = a.seq_lens[b];
    sl[b] = s;
    if (s < 0 || s >= dm.max_seq) atomicOr(&bad, 2);
  }
  __syncthreads();
  if (bad) {
    if (tid == 0) {
      int expected = 0;
      if (bad & 2)
        __hip_atomic_compare_exchange_strong(a.ws.err, &expected, (int)PMK_ERR_SEQ, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      mirror_error(a, ldci(a.ws.err));
    }
    for (int w = tid; w < G; w += blockDim.x) a.ws.qlen[w] = 0;
    return;
  }
  // The step's split: pmk_sched.h's plan_step. Up to 32 requests, on one
  // thread. Beyond, its parts in parallel (one thread over every request took
  // up to ~190 us at 1024 requests): the lengths' aggregates by wave
  // reductions, the attention plan on one thread, cb as a prefix sum over the
  // workgroup (a request per thread), and each dense stage's split on a
  // thread of its own (at one request the reductions and barriers cost more
  // than they save).
  __shared__ unsigned long long agg_sum[kChunkSizes + 1];   // tasks per chunk size, then positions
  __shared__ int agg_max[kChunkSizes];
  __shared__ int wave_tot[32];
  if (B <= 32) {
    if (tid == 0) {
      a.ws.err[16] = 0;   // abort flag
      plan = plan_step(dm, B, sl, cb, a.per_op, a.ev_mode);
    }
  } else {
    if (tid < kChunkSizes + 1) agg_sum[tid] = 0;
    if (tid < kChunkSizes) agg_max[tid] = 0;
    __syncthreads();
    {
      PlanAgg g{};
      for (int b = tid; b < B; b += blockDim.x) plan_agg_add(g, sl[b]);
      for (int i = 0; i <= kChunkSizes; ++i) {
        long long t = i < kChunkSizes ? g.tasks[i] : g.positions;
        int m = i < kChunkSizes ? g.max_nc[i] : 0;
        for (int o = 32; o > 0; o >>= 1) {
          t += __shfl_xor(t, o, 64);
          m = max(m, __shfl_xor(m, o, 64));
        }
        if ((tid & 63) == 0) {
          atomicAdd(&agg_sum[i], (unsigned long long)t);
          if (i < kChunkSizes) atomicMax(&agg_max[i], m);
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      a.ws.err[16] = 0;   // abort flag
      PlanAgg g{};
      for (int i = 0; i < kChunkSizes; ++i) {
        g.tasks[i] = (long)agg_sum[i];
        g.max_nc[i] = agg_max[i];
      }
      g.positions = (long)agg_sum[kChunkSizes];
      plan = plan_attention(dm, B, g, a.per_op, a.ev_mode);
    }
    __syncthreads();
    {
      static_assert(kMaxBatchAll <= 1024, "one request per prologue thread");
      const int v = tid < B ? plan_cb_term(plan, sl[tid]) : 0, inc = wave_scan(v), wv = tid >> 6;
      if ((tid & 63) == 63) wave_tot[wv] = inc;
      __syncthreads();
      int off = 0;
      for (int i = 0; i < wv; ++i) off += wave_tot[i];
      if (tid < B) cb[tid] = off + inc - v;
      if (tid == B - 1) cb[B] = off + inc;
    }
    if (tid < 4) plan.geo[tid] = plan_geo(dm, plan, tid);
    __syncthreads();
    if (tid == 0) plan.nblk = plan_nblk(dm, plan);
  }
  if (tid == 0) {
    copy->attn_merge_o = plan.merge;
    copy->attn_chunk = plan.ck;
    for (int st = 0; st < 4; ++st) copy->geo[st] = plan.geo[st];
    copy->qkv_tiles = plan.geo[0].tiles;
    copy->nblk = plan.nblk;
  }
  for (int g = tid; g < dm.Hkv; g += blockDim.x) gtiles[g] = 0;
  __syncthreads();
  for (int t = tid; t < plan.geo[0].tiles; t += blockDim.x) {
    const int2 gr = qkv_tile_groups(dm, plan.geo[0].tiles, t);
    for (int g = gr.x; g <= gr.y; ++g) atomicAdd(&gtiles[g], 1);
  }
  // every workgroup's queue (pmk_sched.h: build_queue)
  for (int w = tid; w < G; w += blockDim.x) {
    int4* q = a.ws.queue + (size_t)w * dm.max_queue;
    int4* qe = a.ws.qev + (size_t)w * dm.max_queue;
    int n = 0;
    build_queue(dm, plan, cb, w, [&](int4 v) {
      if (n < dm.max_queue) {
        q[n] = v;
        qe[n] = task_events(dm, plan, v, w);   // its wait and notify counters
      }
      ++n;
    });
    a.ws.qlen[w] = n <= dm.max_queue ? n : 0;
    if (n > dm.max_queue) atomicOr(&bad, 4);
  }
  __syncthreads();
  // every counter of every layer armed with its count (pmk_sched.h: ev_count).
  // Per layer: QKV and ATTN flat counters of the blocks in use, the O, GU and
  // DOWN events of those blocks, and ROUTER, ROUTE, MDOWN.
  const int nb = plan.nblk, H = dm.Hkv, per_layer = 2 * nb * H + (3 * nb + 3) * (1 + kSubs);
  for (int idx = tid; idx < dm.L * per_layer; idx += blockDim.x) {
    const int l = idx / per_layer;
    int r = idx - l * per_layer;
    int kind, blk = 0, g = 0, sub = 0;
    if (r < 2 * nb * H) {
      kind = r < nb * H ? EV_QKV : EV_ATTN;
      r %= nb * H;
      blk = r / H;
      g = r - blk * H;
    } else {
      r -= 2 * nb * H;
      const int e = r / (1 + kSubs);
      sub = r - e * (1 + kSubs);
      if (e < 3 * nb) {
        kind = e < nb ? EV_O : e < 2 * nb ? EV_GU : EV_DOWN;
        blk = e % nb;
      } else {
        kind = e == 3 * nb ? EV_ROUTER : e == 3 * nb + 1 ? EV_ROUTE : EV_MDOWN;
      }
    }
    a.ws.ev[ev_off(dm, l, kind, blk, g) + sub * kCtr] = ev_count(dm, plan, cb, kind, blk, g, sub, gtiles);
  }
  for (int idx = tid; idx < 4 * G * ((B + kMaxNb - 1) / kMaxNb); idx += blockDim.x) {
    const int used = G * ((B + kMaxNb - 1) / kMaxNb), st = idx / used;   // (block, tile) records of each stage
    a.ws.tctr[((size_t)st * dm.tctr_stride + idx - st * used) * kCtr] = 0;
  }
  if (a.barrier)   // every workgroup arrives at every stage barrier
    for (int idx = tid; idx < dm.L * kMaxStages; idx += blockDim.x) {
      int* ev = a.ws.bar + (size_t)idx * kEvInts;
      ev[0] = 0;
      for (int x = 0; x < kSubs; ++x) ev[(1 + x) * kCtr] = sub_tiles(G, G, x);
    }
  if (a.trace)
    for (int w = tid; w < G; w += blockDim.x) a.trace[(size_t)w * a.trace_cap * 8] = 0;
  // attention merge counters: the pieces (streamed) or chunks of each (request, KV head)
  for (int idx = tid; idx < dm.L * B * dm.Hkv; idx += blockDim.x) {
    const int l = idx / (B * dm.Hkv), rem = idx - l * B * dm.Hkv, b = rem / dm.Hkv, g = rem - b * dm.Hkv;
    a.ws.mctr[(((size_t)l * dm.max_batch + b) * dm.Hkv + g) * kCtr] = attn_pieces(dm, plan, cb, b, g);
  }
  __syncthreads();
  if (tid == 0 && (bad & 4)) {
    int expected = 0;
    __hip_atomic_compare_exchange_strong(a.ws.err, &expected, (int)PMK_ERR_ARG, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    mirror_error(a, ldci(a.ws.err));
  }
}

// ---------------------------------------------------------------------------
// Launch wrappers
// ---------------------------------------------------------------------------
static const void* main_fn(int dtype, bool part, bool moe, bool tiles) {
  if (dtype == PMK_BF16 && tiles) {
    if (part) return (const void*)pmk_main<uint16_t, true, KP_ALL | KP_TILES>;
    return moe ? (const void*)pmk_main<uint16_t, false, KP_MOE | KP_TILES>
               : (const void*)pmk_main<uint16_t, false, KP_DENSE | KP_TILES>;
  }
  if (dtype == PMK_BF16) {
    if (part) return (const void*)pmk_main<uint16_t, true, KP_ALL>;
    return moe ? (const void*)pmk_main<uint16_t, false, KP_MOE> : (const void*)pmk_main<uint16_t, false, KP_DENSE>;
  }
  return part ? (const void*)pmk_main<float, true, KP_ALL> : (const void*)pmk_main<float, false, KP_ALL>;
}

hipError_t prepare_main(int dtype, int wtiles) {
  for (bool part : {false, true})
    for (bool moe : {false, true}) {
      const hipError_t e = hipFuncSetAttribute(main_fn(dtype, part, moe, wtiles != 0),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

// Writes a bfloat16 [rows][cols] matrix (rows % 16 == 0, cols % 32 == 0) in
// the tile layout: 16 x 32 tiles in row-group-major order, each row-major, so
// 16-byte piece q = (rg (cols / 32) + s) 64 + 4 r + g holds row 16 rg + r,
// columns 32 s + 8 g .. + 7. One thread per piece; the writes are contiguous,
// the reads 64-byte runs.
__global__ void __launch_bounds__(256) pmk_pack(const uint4* __restrict__ src, uint4* __restrict__ dst, long rows,
                                                long cols) {
  const long n = rows * cols / 8, nks = cols / 32;
  for (long q = blockIdx.x * 256L + threadIdx.x; q < n; q += (long)gridDim.x * 256) {
    const long lp = q & 63, t = q >> 6, rg = t / nks, st = t - rg * nks;
    const long row = rg * 16 + (lp >> 2), col = st * 32 + (lp & 3) * 8;
    dst[q] = src[(row * cols + col) >> 3];
  }
}

hipError_t launch_pack(const void* src, void* dst, long rows, long cols, hipStream_t s) {
  const long n = rows * cols / 8;
  const long need = (n + 255) / 256, blocks = need < 65536 ? need : 65536;
  hipLaunchKernelGGL(pmk_pack, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const uint4*>(src),
                     reinterpret_cast<uint4*>(dst), rows, cols);
  return hipGetLastError();
}

hipError_t launch_prologue(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(pmk_prologue, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_main(const StepArgs& a, int dtype, hipStream_t s, RunSpec rs) {
  const StepArgs* pa = reinterpret_cast<const StepArgs*>(a.ws.args);
  void* args[] = {&pa, &rs};
  const bool part = rs.l0 != 0 || rs.l1 != a.dm.L || rs.types != kAllTypes || rs.barrier;
  return hipLaunchCooperativeKernel(main_fn(dtype, part, a.dm.moe != 0, a.dm.wtiles != 0), dim3(a.dm.grid),
                                    dim3(kBlock), args,
                                    kLdsBytes, s);
}

}  // namespace pmk
