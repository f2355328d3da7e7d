// pmk_kernels.hip -- the per-step prologue and the persistent decode kernel.
//
// One decode step = two launches on the caller's stream:
//  1. pmk_prologue (one workgroup): reads (batch, seq_lens) on the device,
//     checks every length, derives the attention chunk count of each request,
//     writes each persistent workgroup's task queue for one layer, and arms
//     every event counter of every layer. This is the runtime instantiation of
//     a dependency template whose batch and length dimensions are symbolic
//     (Event Tensor summary, Core method, two kinds of dynamism: shape
//     dynamism), so a new batch size or new lengths need no recompilation.
//  2. pmk_main (one workgroup per compute unit, cooperative launch so that all
//     are co-resident): every workgroup replays its queue for layer 0, 1, ...,
//     waiting on the events its tasks consume and notifying the events they
//     produce (same page, Core method, Event Tensor abstraction and ETC
//     compiler and scheduling: static scheduling with per-SM queues and a
//     persistent main loop).
//
// Deadlock freedom: each queue lists its tasks in stage order (QKV, attention,
// O, FFN stages) and every task only waits on events produced by earlier
// stages of the same layer or by the previous layer. All workgroups are
// resident, so by induction on (layer, stage) the earliest unfinished stage
// always has all its producers done. Every wait is bounded by a watchdog; on
// expiry the step is abandoned (error word + abort flag), so every wave exits.
#include "pmk_device.h"

namespace pmk {

// LDS layout (floats): [xs: GEMV inputs | ys: GEMV outputs | misc]
constexpr int MISC_RSTD = 0;    // 8 floats: per-row 1/rms of the staged batch block
constexpr int MISC_RED = 16;    // kWaves * 8 floats: block reduction scratch
constexpr int MISC_FLAG = 96;   // int: broadcast flag
constexpr int MISC_OK = 100;    // int: wait result
constexpr int MISC_ROUTE = 128; // MoE routing scratch (ints)

__device__ __forceinline__ int* ev_ptr(const StepArgs& a, int layer, int e) {
  return a.ws.ev + ((size_t)layer * EV_COUNT + e) * kEvInts;
}

__device__ __forceinline__ size_t kv_off(const Dims& dm, int l, int which, int b, int g, int pos) {
  return (((((size_t)l * 2 + which) * dm.max_batch + b) * dm.Hkv + g) * (size_t)dm.max_seq + pos) * dm.d;
}

// ---------------------------------------------------------------------------
// Staging of a GEMV input block: xs[b][k] = src[b][k] * gain[k] for b < nb,
// zero rows for nb <= b < BB. With `norm`, misc[MISC_RSTD + b] = 1/sqrt(mean
// src[b]^2 + eps) (RMSNorm folded into the GEMV: the dot product uses x*gain
// and the epilogue multiplies by rstd). src is device-coherent data.
// ---------------------------------------------------------------------------
template <int BB>
__device__ void stage_x(const float* src, int ld, int nb, int K, const float* gain, bool norm, float eps,
                        float* xs, float* misc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float ss[BB];
#pragma unroll
  for (int b = 0; b < BB; ++b) ss[b] = 0.f;
  const int k4 = K >> 2;
#pragma unroll
  for (int b = 0; b < BB; ++b) {
    float* xr = xs + b * K;
    if (b < nb) {
      const auto r = rsrc(src + (size_t)b * ld);
      for (int i = tid; i < k4; i += kBlock) {
        f4v v = ldc4(r, i * 16);
        ss[b] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        if (gain) {
          const float4 gg = reinterpret_cast<const float4*>(gain)[i];
          v.x *= gg.x; v.y *= gg.y; v.z *= gg.z; v.w *= gg.w;
        }
        reinterpret_cast<f4v*>(xr)[i] = v;
      }
    } else {
      for (int i = tid; i < k4; i += kBlock) reinterpret_cast<f4v*>(xr)[i] = f4v{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (norm) {
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      float s = wave_sum(ss[b]);
      if (lane == 0) misc[MISC_RED + wave * 8 + b] = s;
    }
    __syncthreads();
    if (tid < BB) {
      float s = 0.f;
      for (int w = 0; w < kWaves; ++w) s += misc[MISC_RED + w * 8 + tid];
      misc[MISC_RSTD + tid] = 1.0f / sqrtf(s / (float)K + eps);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// GEMV core: ys[j][b] = sum_k W[row(j)][k] xs[b][k] for j < R, b < BB.
// Wave w takes rows w, w+8, ...; each lane streams 16 B of a row per load
// (a wave reads 1 KiB contiguous per instruction), U loads in flight per wave.
// ---------------------------------------------------------------------------
struct RowsContig {
  int r0;
  __device__ __forceinline__ int operator()(int j) const { return r0 + j; }
};
// QKV tiles are in rotation pairs: local row 2u is (h, i), 2u+1 is (h, i + d/2).
struct RowsQkv {
  int u0, d;
  __device__ __forceinline__ int operator()(int j) const {
    const int half = d >> 1, unit = u0 + (j >> 1);
    return (unit / half) * d + (unit % half) + (j & 1) * half;
  }
};

template <typename WT, int BB, typename RowMap>
__device__ void gemv(const WT* __restrict__ W, int K, int R, RowMap rm, const float* xs, float* ys) {
  constexpr int U = sizeof(WT) == 2 ? 8 : 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = (K + 511) >> 9;
  for (int j = wave; j < R; j += kWaves) {
    const WT* wr = W + (size_t)rm(j) * K;
    float acc[BB];
#pragma unroll
    for (int b = 0; b < BB; ++b) acc[b] = 0.f;
    for (int c0 = 0; c0 < nch; c0 += U) {
      Raw8<WT> raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = ((c0 + u) << 9) + (lane << 3);
        if (c0 + u < nch && k < K) raw[u].load(wr + k); else raw[u].zero();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = ((c0 + u) << 9) + (lane << 3);
        if (c0 + u < nch && k < K) {
          float w[8];
          raw[u].to(w);
#pragma unroll
          for (int b = 0; b < BB; ++b) {
            const float4 x0 = *reinterpret_cast<const float4*>(xs + b * K + k);
            const float4 x1 = *reinterpret_cast<const float4*>(xs + b * K + k + 4);
            acc[b] += w[0] * x0.x + w[1] * x0.y + w[2] * x0.z + w[3] * x0.w +
                      w[4] * x1.x + w[5] * x1.y + w[6] * x1.z + w[7] * x1.w;
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      const float s = wave_sum(acc[b]);
      if (lane == 0) ys[j * BB + b] = s;
    }
  }
}

// Largest batch block (1, 2, 4 or 8) that fits the LDS staging for a GEMV of
// depth K producing R rows, and is not wider than the batch needs.
__device__ __forceinline__ int pick_bb(int batch, int K, int R) {
  int lim = kXsFloats / K;
  if (kYsFloats / R < lim) lim = kYsFloats / R;
  int bb = 8;
  while (bb > 1 && (bb > lim || (bb >> 1) >= batch)) bb >>= 1;
  return bb;
}

// ---------------------------------------------------------------------------
// Task bodies
// ---------------------------------------------------------------------------
struct Ctx {
  const StepArgs& a;
  int l, wg;
  float* xs;
  float* ys;
  float* misc;
};

// RMSNorm1 + QKV rows of one tile + RoPE + KV append.
template <typename WT, int BB>
__device__ __noinline__ void task_qkv(const Ctx c, int tile) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const LayerPtrs& L = a.layers[c.l];
  const int half = dm.d >> 1, qkv_dim = (dm.Hq + 2 * dm.Hkv) * dm.d;
  const int u0 = (int)((long)tile * dm.qkv_units / dm.qkv_tiles);
  const int u1 = (int)((long)(tile + 1) * dm.qkv_units / dm.qkv_tiles);
  const int nu = u1 - u0;
  for (int b0 = 0; b0 < a.batch; b0 += BB) {
    const int nb = min(BB, a.batch - b0);
    stage_x<BB>(a.hidden + (size_t)b0 * dm.H, dm.H, nb, dm.H, L.attn_norm, true, dm.eps, c.xs, c.misc);
    gemv<WT, BB>(reinterpret_cast<const WT*>(L.w_qkv), dm.H, 2 * nu, RowsQkv{u0, dm.d}, c.xs, c.ys);
    __syncthreads();
    for (int idx = threadIdx.x; idx < nu * nb; idx += kBlock) {
      const int ju = idx / nb, b = idx - ju * nb;
      const int unit = u0 + ju, h = unit / half, i = unit - h * half;
      const float r = c.misc[MISC_RSTD + b];
      float y1 = c.ys[(2 * ju) * BB + b] * r, y2 = c.ys[(2 * ju + 1) * BB + b] * r;
      const int bb = b0 + b, pos = a.seq_lens[bb];
      if (h < dm.Hq + dm.Hkv) {
        const float2 cs = a.ws.rope[(size_t)pos * half + i];
        const float t1 = y1 * cs.x - y2 * cs.y, t2 = y2 * cs.x + y1 * cs.y;
        y1 = t1;
        y2 = t2;
      }
      float* dst = a.ws.qkv + (size_t)bb * qkv_dim + h * dm.d + i;
      stc(dst, y1);
      stc(dst + half, y2);
      if (h >= dm.Hq) {
        const int kvh = h - dm.Hq, which = kvh / dm.Hkv, g = kvh - which * dm.Hkv;
        WT* cp = reinterpret_cast<WT*>(a.kv) + kv_off(dm, c.l, which, bb, g, pos);
        Elem<WT>::put(cp + i, y1);
        Elem<WT>::put(cp + i + half, y2);
      }
    }
    __syncthreads();
  }
}

// A KV row slice of 16 bytes (8 bfloat16 or 4 float) as raw bits.
template <typename KT> __device__ __forceinline__ void unpack_row(const uint4 r, float (&f)[16 / sizeof(KT)]);
template <> __device__ __forceinline__ void unpack_row<uint16_t>(const uint4 r, float (&f)[8]) {
  f[0] = bf_lo(r.x); f[1] = bf_hi(r.x); f[2] = bf_lo(r.y); f[3] = bf_hi(r.y);
  f[4] = bf_lo(r.z); f[5] = bf_hi(r.z); f[6] = bf_lo(r.w); f[7] = bf_hi(r.w);
}
template <> __device__ __forceinline__ void unpack_row<float>(const uint4 r, float (&f)[4]) {
  f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y); f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
}
// Device-coherent float row slice -> cache-dtype bits (rounded like the KV append).
template <typename KT> __device__ __forceinline__ uint4 pack_row(const float* p);
template <> __device__ __forceinline__ uint4 pack_row<uint16_t>(const float* p) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(ldc(p + 2 * i)) | ((uint32_t)f2bf(ldc(p + 2 * i + 1)) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
template <> __device__ __forceinline__ uint4 pack_row<float>(const float* p) {
  return make_uint4(__float_as_uint(ldc(p)), __float_as_uint(ldc(p + 1)), __float_as_uint(ldc(p + 2)),
                    __float_as_uint(ldc(p + 3)));
}

// Split-K GQA decode attention for (request b, KV head g, chunk ci): the G
// query heads of group g against positions [ci*CK, min((ci+1)*CK, S+1)).
// Writes the chunk's (acc, max, sum) partial; the workgroup that completes the
// last chunk of (b, g) merges all partials by log-sum-exp and notifies.
template <typename KT, int G>
__device__ __noinline__ void task_attn(const Ctx c, int b, int g, int ci) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  constexpr int EPL = 16 / (int)sizeof(KT);   // elements per lane (16 B)
  constexpr int D = 16 * EPL;                 // head_dim: 128 (bf16) or 64 (f32)
  constexpr int ITS = kAttnChunk / (kWaves * 4);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, rs = lane >> 4, li = lane & 15;
  const int qkv_dim = (dm.Hq + 2 * dm.Hkv) * D;
  const int S = a.seq_lens[b], n = S + 1;
  const int p0 = ci * kAttnChunk, p1 = min(n, p0 + kAttnChunk);
  const float qscale = 1.4426950408889634f / sqrtf((float)D);   // 1/sqrt(d), in log2 units

  const float* qrow = a.ws.qkv + (size_t)b * qkv_dim + (size_t)g * G * D;
  float q[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[h][e] = ldc(qrow + h * D + li * EPL + e) * qscale;

  const KT* Kb = reinterpret_cast<const KT*>(a.kv) + kv_off(dm, c.l, 0, b, g, 0);
  const KT* Vb = reinterpret_cast<const KT*>(a.kv) + kv_off(dm, c.l, 1, b, g, 0);
  const float* knew = a.ws.qkv + (size_t)b * qkv_dim + (size_t)(dm.Hq + g) * D;
  const float* vnew = a.ws.qkv + (size_t)b * qkv_dim + (size_t)(dm.Hq + dm.Hkv + g) * D;

  float m[G], ls[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  // KV rows in flight per lane group, kept as raw 16-byte vectors until use:
  // all ITS iterations for small groups, two at a time for G = 8
  constexpr int ITB = G >= 8 ? 2 : ITS;
#pragma unroll
  for (int it0 = 0; it0 < ITS; it0 += ITB) {
    uint4 kr[ITB], vr[ITB];
#pragma unroll
    for (int ib = 0; ib < ITB; ++ib) {
      const int p = p0 + (it0 + ib) * (kWaves * 4) + wave * 4 + rs;
      if (p < p1 && p != S) {
        kr[ib] = *reinterpret_cast<const uint4*>(Kb + (size_t)p * D + li * EPL);
        vr[ib] = *reinterpret_cast<const uint4*>(Vb + (size_t)p * D + li * EPL);
      } else if (p == S) {
        // the new token: this step's rotated k and v, rounded exactly as they
        // were stored into the cache
        kr[ib] = pack_row<KT>(knew + li * EPL);
        vr[ib] = pack_row<KT>(vnew + li * EPL);
      }
    }
#pragma unroll
    for (int ib = 0; ib < ITB; ++ib) {
      const int p = p0 + (it0 + ib) * (kWaves * 4) + wave * 4 + rs;
      if (p < p1) {
        float kf[EPL], vf[EPL];
        unpack_row<KT>(kr[ib], kf);
        unpack_row<KT>(vr[ib], vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) s += q[h][e] * kf[e];
          s = sum16(s);
          const float mn = fmaxf(m[h], s);
          const float al = exp2f(m[h] - mn), pe = exp2f(s - mn);
          ls[h] = ls[h] * al + pe;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * al + pe * vf[e];
          m[h] = mn;
        }
      }
    }
  }
  // combine the 4 row slots of the wave
  float* sw = c.xs;   // [kWaves][G][D + 2]
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = fmaxf(m[h], __shfl_xor(m[h], 16, 64));
    M = fmaxf(M, __shfl_xor(M, 32, 64));
    const float sc = (M == -INFINITY) ? 0.f : exp2f(m[h] - M);
    float lw = ls[h] * sc;
    lw += __shfl_xor(lw, 16, 64);
    lw += __shfl_xor(lw, 32, 64);
    float* dst = sw + (wave * G + h) * (D + 2);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[h][e] * sc;
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (rs == 0) dst[li * EPL + e] = v;
    }
    if (lane == 0) { dst[D] = M; dst[D + 1] = lw; }
  }
  __syncthreads();
  // combine waves, write this chunk's partial
  float* part = a.ws.part + (((size_t)b * dm.Hkv + g) * dm.max_chunks + ci) * G * (D + 2);
  for (int t = tid; t < G * D; t += kBlock) {
    const int h = t / D, e = t - h * D;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sw[(w * G + h) * (D + 2) + D]);
    float Ls = 0.f, A = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float* s = sw + (w * G + h) * (D + 2);
      const float f = (s[D] == -INFINITY) ? 0.f : exp2f(s[D] - M);
      Ls += s[D + 1] * f;
      A += s[e] * f;
    }
    stc(part + h * (D + 2) + e, A);
    if (e == 0) { stc(part + h * (D + 2) + D, M); stc(part + h * (D + 2) + D + 1, Ls); }
  }
  // the last chunk task of (b, g) to finish merges the partials
  vm_drain();
  __syncthreads();
  int* flag = reinterpret_cast<int*>(c.misc + MISC_FLAG);
  if (tid == 0) {
    int* mc = a.ws.mctr + (((size_t)c.l * dm.max_batch + b) * dm.Hkv + g) * kCtr;
    *flag = (atomic_add_relaxed(mc, -1) == 1);
  }
  __syncthreads();
  if (*flag) {
    const int nc = (n + kAttnChunk - 1) / kAttnChunk;
    const float* pb = a.ws.part + ((size_t)b * dm.Hkv + g) * dm.max_chunks * G * (D + 2);
    float* o = a.ws.o + (size_t)b * dm.Hq * D + (size_t)g * G * D;
    for (int t = tid; t < G * D; t += kBlock) {
      const int h = t / D, e = t - h * D;
      float M = -INFINITY;
      for (int cc = 0; cc < nc; ++cc) M = fmaxf(M, ldc(pb + ((size_t)cc * G + h) * (D + 2) + D));
      float Ls = 0.f, A = 0.f;
      for (int cc = 0; cc < nc; ++cc) {
        const float* s = pb + ((size_t)cc * G + h) * (D + 2);
        const float f = exp2f(ldc(s + D) - M);
        Ls += ldc(s + D + 1) * f;
        A += ldc(s + e) * f;
      }
      stc(o + h * D + e, A / Ls);
    }
    wg_notify(ev_ptr(a, c.l, EV_ATTN), -1);
  }
  __syncthreads();
}

// O-projection rows [r0, r1) of a tile + residual: h1 = x + W_o o.
template <typename WT, int BB>
__device__ __noinline__ void task_o(const Ctx c, int tile) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const LayerPtrs& L = a.layers[c.l];
  const int K = dm.Hq * dm.d;
  const int r0 = (int)((long)tile * dm.H / dm.o_tiles), r1 = (int)((long)(tile + 1) * dm.H / dm.o_tiles);
  const int R = r1 - r0;
  for (int b0 = 0; b0 < a.batch; b0 += BB) {
    const int nb = min(BB, a.batch - b0);
    stage_x<BB>(a.ws.o + (size_t)b0 * K, K, nb, K, nullptr, false, 0.f, c.xs, c.misc);
    gemv<WT, BB>(reinterpret_cast<const WT*>(L.w_o), K, R, RowsContig{r0}, c.xs, c.ys);
    __syncthreads();
    for (int idx = threadIdx.x; idx < R * nb; idx += kBlock) {
      const int j = idx / nb, b = idx - j * nb;
      const size_t off = (size_t)(b0 + b) * dm.H + r0 + j;
      stc(a.ws.h1 + off, ldc(a.hidden + off) + c.ys[j * BB + b]);
    }
    __syncthreads();
  }
}

// RMSNorm2 + gate and up rows [r0, r1) + SwiGLU: act = silu(gate) * up.
template <typename WT, int BB>
__device__ __noinline__ void task_gu(const Ctx c, int tile) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const LayerPtrs& L = a.layers[c.l];
  const int r0 = (int)((long)tile * dm.F / dm.gu_tiles), r1 = (int)((long)(tile + 1) * dm.F / dm.gu_tiles);
  const int R = r1 - r0;
  for (int b0 = 0; b0 < a.batch; b0 += BB) {
    const int nb = min(BB, a.batch - b0);
    stage_x<BB>(a.ws.h1 + (size_t)b0 * dm.H, dm.H, nb, dm.H, L.ffn_norm, true, dm.eps, c.xs, c.misc);
    gemv<WT, BB>(reinterpret_cast<const WT*>(L.w_gate), dm.H, R, RowsContig{r0}, c.xs, c.ys);
    gemv<WT, BB>(reinterpret_cast<const WT*>(L.w_up), dm.H, R, RowsContig{r0}, c.xs, c.ys + R * BB);
    __syncthreads();
    for (int idx = threadIdx.x; idx < R * nb; idx += kBlock) {
      const int j = idx / nb, b = idx - j * nb;
      const float r = c.misc[MISC_RSTD + b];
      const float gt = c.ys[j * BB + b] * r, up = c.ys[(R + j) * BB + b] * r;
      stc(a.ws.act + (size_t)(b0 + b) * dm.F + r0 + j, gt / (1.0f + __expf(-gt)) * up);
    }
    __syncthreads();
  }
}

// Down-projection rows [r0, r1) + residual: x' = h1 + W_down act (written to hidden).
template <typename WT, int BB>
__device__ __noinline__ void task_down(const Ctx c, int tile) {
  const StepArgs& a = c.a;
  const Dims& dm = a.dm;
  const LayerPtrs& L = a.layers[c.l];
  const int r0 = (int)((long)tile * dm.H / dm.down_tiles), r1 = (int)((long)(tile + 1) * dm.H / dm.down_tiles);
  const int R = r1 - r0;
  for (int b0 = 0; b0 < a.batch; b0 += BB) {
    const int nb = min(BB, a.batch - b0);
    stage_x<BB>(a.ws.act + (size_t)b0 * dm.F, dm.F, nb, dm.F, nullptr, false, 0.f, c.xs, c.misc);
    gemv<WT, BB>(reinterpret_cast<const WT*>(L.w_down), dm.F, R, RowsContig{r0}, c.xs, c.ys);
    __syncthreads();
    for (int idx = threadIdx.x; idx < R * nb; idx += kBlock) {
      const int j = idx / nb, b = idx - j * nb;
      const size_t off = (size_t)(b0 + b) * dm.H + r0 + j;
      stc(a.hidden + off, ldc(a.ws.h1 + off) + c.ys[j * BB + b]);
    }
    __syncthreads();
  }
}

#define PMK_BB_DISPATCH(FN, WT, bb, ...)          \
  switch (bb) {                                   \
    case 8: FN<WT, 8>(__VA_ARGS__); break;        \
    case 4: FN<WT, 4>(__VA_ARGS__); break;        \
    case 2: FN<WT, 2>(__VA_ARGS__); break;        \
    default: FN<WT, 1>(__VA_ARGS__); break;       \
  }

// ---------------------------------------------------------------------------
// The persistent kernel
// ---------------------------------------------------------------------------
template <typename WT>
__global__ void __launch_bounds__(kBlock, 1) pmk_main(const StepArgs* __restrict__ pa) {
  extern __shared__ float lds[];
  const StepArgs& a = *pa;
  const Dims& dm = a.dm;
  const int wg = blockIdx.x;
  float* misc = lds + kXsFloats + kYsFloats;
  int* okp = reinterpret_cast<int*>(misc + MISC_OK);
  if (threadIdx.x == 0) *okp = (ldci(a.ws.err) == 0);
  __syncthreads();
  if (!*okp) return;
  const int n = a.ws.qlen[wg];
  const int4* q = a.ws.queue + (size_t)wg * dm.max_queue;
  const int G = dm.Hq / dm.Hkv;
  uint32_t* tr = a.trace ? a.trace + (size_t)wg * a.trace_cap * 4 : nullptr;
  int tn = 1;
  for (int l = 0; l < dm.L; ++l) {
    Ctx c{a, l, wg, lds, lds + kXsFloats, misc};
    unsigned passed = 0;
    for (int t = 0; t < n; ++t) {
      const int4 task = q[t];
      const uint32_t t_begin = (uint32_t)now_ticks();
      int need = -1, need_l = l;
      switch (task.x) {
        case T_QKV: if (l > 0) { need = EV_DOWN; need_l = l - 1; } break;
        case T_ATTN: need = EV_QKV; break;
        case T_O: need = EV_ATTN; break;
        case T_GU: need = EV_O; break;
        case T_DOWN: need = EV_GU; break;
        default: break;
      }
      if (need >= 0) {
        const unsigned bit = 1u << (need + (need_l != l ? 16 : 0));
        if (!(passed & bit)) {
          if (threadIdx.x == 0) *okp = spin_zero(ev_ptr(a, need_l, need), a.ws.err, a.watchdog_ticks);
          __syncthreads();
          if (!*okp) return;
          passed |= bit;
        }
      }
      const uint32_t t_waited = (uint32_t)now_ticks();
      switch (task.x) {
        case T_QKV: {
          const int nu = (int)((long)(task.y + 1) * dm.qkv_units / dm.qkv_tiles) -
                         (int)((long)task.y * dm.qkv_units / dm.qkv_tiles);
          PMK_BB_DISPATCH(task_qkv, WT, pick_bb(a.batch, dm.H, 2 * nu), c, task.y);
          wg_notify(ev_ptr(a, l, EV_QKV), wg & (kSubs - 1));
          break;
        }
        case T_ATTN:
          if (G == 8) task_attn<WT, 8>(c, task.y, task.z, task.w);
          else if (G == 4) task_attn<WT, 4>(c, task.y, task.z, task.w);
          else if (G == 2) task_attn<WT, 2>(c, task.y, task.z, task.w);
          else task_attn<WT, 1>(c, task.y, task.z, task.w);
          break;
        case T_O: {
          const int R = (int)((long)(task.y + 1) * dm.H / dm.o_tiles) - (int)((long)task.y * dm.H / dm.o_tiles);
          PMK_BB_DISPATCH(task_o, WT, pick_bb(a.batch, dm.Hq * dm.d, R), c, task.y);
          wg_notify(ev_ptr(a, l, EV_O), wg & (kSubs - 1));
          break;
        }
        case T_GU: {
          const int R = (int)((long)(task.y + 1) * dm.F / dm.gu_tiles) - (int)((long)task.y * dm.F / dm.gu_tiles);
          PMK_BB_DISPATCH(task_gu, WT, pick_bb(a.batch, dm.H, 2 * R), c, task.y);
          wg_notify(ev_ptr(a, l, EV_GU), wg & (kSubs - 1));
          break;
        }
        case T_DOWN: {
          const int R = (int)((long)(task.y + 1) * dm.H / dm.down_tiles) - (int)((long)task.y * dm.H / dm.down_tiles);
          PMK_BB_DISPATCH(task_down, WT, pick_bb(a.batch, dm.F, R), c, task.y);
          wg_notify(ev_ptr(a, l, EV_DOWN), wg & (kSubs - 1));
          break;
        }
        default: break;
      }
      if (tr && threadIdx.x == 0 && tn < a.trace_cap) {
        const uint32_t t_end = (uint32_t)now_ticks();
        uint32_t* e = tr + (size_t)tn * 4;
        e[0] = (uint32_t)task.x | ((uint32_t)l << 8) | ((uint32_t)(task.y & 0xffff) << 16);
        e[1] = t_begin;
        e[2] = t_waited;
        e[3] = t_end;
        ++tn;
      }
    }
  }
  if (tr && threadIdx.x == 0) tr[0] = (uint32_t)(tn - 1);
}

// ---------------------------------------------------------------------------
// The per-step prologue: validate lengths, build queues, arm events.
// ---------------------------------------------------------------------------
// Number of the first `tiles` tasks of a stage (task t runs on workgroup
// t % grid and notifies sub-counter (t % grid) & (kSubs - 1)) that notify
// sub-counter x.
__device__ __forceinline__ int sub_count(int tiles, int grid, int x) {
  auto below = [x](int n) { return n > x ? (n - x + kSubs - 1) / kSubs : 0; };   // w < n with w % kSubs == x
  return (tiles / grid) * below(grid) + below(tiles % grid);
}

__global__ void __launch_bounds__(1024) pmk_prologue(StepArgs a) {
  const Dims& dm = a.dm;
  const int tid = threadIdx.x, B = a.batch, G = dm.grid;
  if (tid == 0) *reinterpret_cast<StepArgs*>(a.ws.args) = a;
  __shared__ int bad;
  __shared__ int total_attn;
  if (tid == 0) bad = (ldci(a.ws.err) != 0) ? 1 : 0;
  __syncthreads();
  for (int b = tid; b < B; b += blockDim.x) {
    const int s = a.seq_lens[b];
    if (s < 0 || s >= dm.max_seq) atomicOr(&bad, 2);
  }
  __syncthreads();
  if (bad) {
    if ((bad & 2) && tid == 0) {
      int expected = 0;
      __hip_atomic_compare_exchange_strong(a.ws.err, &expected, (int)PMK_ERR_SEQ, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int w = tid; w < G; w += blockDim.x) a.ws.qlen[w] = 0;
    return;
  }
  if (tid == 0) {
    a.ws.err[16] = 0;   // abort flag
    int acc = 0;
    for (int b = 0; b < B; ++b) {
      a.ws.chunk_base[b] = acc;
      acc += (a.seq_lens[b] + kAttnChunk) / kAttnChunk;   // ceil((S + 1) / CK)
    }
    a.ws.chunk_base[B] = acc;
    total_attn = acc * dm.Hkv;
  }
  __syncthreads();
  const int* cb = a.ws.chunk_base;
  // queues: stage order QKV, attention, O, gate/up, down
  for (int w = tid; w < G; w += blockDim.x) {
    int4* q = a.ws.queue + (size_t)w * dm.max_queue;
    int n = 0;
    for (int t = w; t < dm.qkv_tiles; t += G) { if (n < dm.max_queue) q[n] = make_int4(T_QKV, t, 0, 0); ++n; }
    for (int i = w; i < total_attn; i += G) {
      int lo = 0, hi = B;   // find b: Hkv*cb[b] <= i < Hkv*cb[b+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (dm.Hkv * cb[mid] <= i) lo = mid; else hi = mid;
      }
      const int r = i - dm.Hkv * cb[lo], nc = cb[lo + 1] - cb[lo];
      if (n < dm.max_queue) q[n] = make_int4(T_ATTN, lo, r / nc, r % nc);
      ++n;
    }
    for (int t = w; t < dm.o_tiles; t += G) { if (n < dm.max_queue) q[n] = make_int4(T_O, t, 0, 0); ++n; }
    for (int t = w; t < dm.gu_tiles; t += G) { if (n < dm.max_queue) q[n] = make_int4(T_GU, t, 0, 0); ++n; }
    for (int t = w; t < dm.down_tiles; t += G) { if (n < dm.max_queue) q[n] = make_int4(T_DOWN, t, 0, 0); ++n; }
    a.ws.qlen[w] = n <= dm.max_queue ? n : 0;
    if (n > dm.max_queue) atomicOr(&bad, 4);
  }
  // events of every layer
  for (int idx = tid; idx < dm.L * EV_COUNT; idx += blockDim.x) {
    const int e = idx % EV_COUNT;
    int* ev = a.ws.ev + (size_t)idx * kEvInts;
    int tiles = 0;
    if (e == EV_QKV) tiles = dm.qkv_tiles;
    else if (e == EV_O) tiles = dm.o_tiles;
    else if (e == EV_GU) tiles = dm.gu_tiles;
    else if (e == EV_DOWN) tiles = dm.down_tiles;
    if (tiles > 0) {
      int top = 0;
      for (int x = 0; x < kSubs; ++x) {
        const int cnt = sub_count(tiles, G, x);
        ev[(1 + x) * kCtr] = cnt;
        top += cnt > 0;
      }
      ev[0] = top;
    } else if (e == EV_ATTN) {
      ev[0] = B * dm.Hkv;
    } else {
      ev[0] = 0;
    }
  }
  for (int idx = tid; idx < dm.L * B * dm.Hkv; idx += blockDim.x) {
    const int l = idx / (B * dm.Hkv), rem = idx - l * B * dm.Hkv, b = rem / dm.Hkv, g = rem - b * dm.Hkv;
    a.ws.mctr[(((size_t)l * dm.max_batch + b) * dm.Hkv + g) * kCtr] = cb[b + 1] - cb[b];
  }
  __syncthreads();
  if (tid == 0 && (bad & 4)) {
    int expected = 0;
    __hip_atomic_compare_exchange_strong(a.ws.err, &expected, (int)PMK_ERR_ARG, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Launch wrappers
// ---------------------------------------------------------------------------
hipError_t prepare_main(int dtype) {
  const void* f = dtype == PMK_BF16 ? (const void*)pmk_main<uint16_t> : (const void*)pmk_main<float>;
  return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
}

hipError_t launch_prologue(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(pmk_prologue, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_main(const StepArgs& a, int dtype, hipStream_t s) {
  const StepArgs* pa = reinterpret_cast<const StepArgs*>(a.ws.args);
  void* args[] = {&pa};
  const void* f = dtype == PMK_BF16 ? (const void*)pmk_main<uint16_t> : (const void*)pmk_main<float>;
  return hipLaunchCooperativeKernel(f, dim3(a.dm.grid), dim3(kBlock), args, kLdsBytes, s);
}

}  // namespace pmk
