// pmk_device.h -- device-side building blocks of the persistent decode kernel:
// device-coherent loads/stores, event notify/wait, wave reductions, bfloat16
// conversion. gfx950 (CDNA4) only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmk_internal.h"

namespace pmk {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Cross-workgroup data: every intermediate that one workgroup writes and
// another reads within a step is stored and loaded with device-coherent (sc1)
// accesses, which go through to the coherence point shared by all XCDs instead
// of stopping in a per-XCD L2. Together with `s_waitcnt vmcnt(0)` before a
// counter update, that is what lets a relaxed agent-scope counter carry the
// data dependency without a full L2 write-back on notify or an L2 invalidate
// on wait. Weights and already-cached KV entries are immutable during a step
// and use ordinary cached loads.
// ---------------------------------------------------------------------------
//
// Every access here goes through the global address space: through a generic
// pointer it would compile to a FLAT instruction, which also counts against
// the LDS wait counter, so each later LDS wait would wait for it as well (a
// store: until the coherence point acknowledges it).
template <typename T> __device__ __forceinline__ const __attribute__((address_space(1))) T* gp(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}
template <typename T> __device__ __forceinline__ __attribute__((address_space(1))) T* gp(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}
// A pointer that is the same for the whole wave, kept in scalar registers.
template <typename T> __device__ __forceinline__ T* uptr(T* p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (T*)(((unsigned long long)hi << 32) | lo);
}
// Loads of data that nothing writes while the persistent kernel runs (the
// queues, the step's split, layer pointers, request lengths: written by the
// host or by the prologue kernel before it) at a wave-uniform address, through
// the constant address space: scalar loads via the scalar cache, which do not
// wait behind the wave's vector loads in flight. Kept scalar.
typedef const __attribute__((address_space(4))) int* kptr_i;
__device__ __forceinline__ int ldku(const int* p) { return __builtin_amdgcn_readfirstlane(*(kptr_i)(p)); }
__device__ __forceinline__ int4 ldku4(const int4* p) {
  typedef int i4v __attribute__((ext_vector_type(4)));
  const i4v v = *(const __attribute__((address_space(4))) i4v*)(p);
  return make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                   __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
}
// A pointer field of an immutable struct (the same for the whole wave).
template <typename T> __device__ __forceinline__ T* ldp(T* const* field) {
  return uptr(*(T* const __attribute__((address_space(4)))*)(field));
}
__device__ __forceinline__ float ldc(const float* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float* p, float v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ldci(const int* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stci(int* p, int v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-coherent load of a value that is the same for the whole wave (one
// address), kept in a scalar register: the compiler cannot tell that an
// atomic load's result is uniform, and addresses built from it would need a
// loop over lanes.
__device__ __forceinline__ int ldsu(const int* p) { return __builtin_amdgcn_readfirstlane(ldci(p)); }
// Plain load of a wave-uniform int through a generic pointer, kept scalar.
__device__ __forceinline__ int ldu(const int* p) { return __builtin_amdgcn_readfirstlane(*gp(p)); }
__device__ __forceinline__ int4 ldu4(const int4* p) {
  typedef int i4v __attribute__((ext_vector_type(4)));
  const i4v v = *gp(reinterpret_cast<const i4v*>(p));
  return make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                   __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
}
__device__ __forceinline__ int atomic_add_relaxed(int* p, int v) {
  return __hip_atomic_fetch_add(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Buffer resource for device-coherent 16-byte accesses. `base` must be
// wave-uniform (per-lane differences go into the byte offset): a varying base
// compiles to a loop over the distinct values that also waits for every
// memory operation in flight.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
// Buffer resource covering exactly `bytes` (< kNoRecord): a load at a byte
// offset at or past the range returns zeros without touching memory (the
// descriptor's range check), so kNoRecord + a small offset is a safe "no
// data" address for it.
constexpr int kNoRecord = 1 << 30;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_n(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16-byte device-coherent load/store at byte offset `off` from a wave-uniform base.
__device__ __forceinline__ f4v ldc4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}
// The same loads through the caches, for per-layer activations (written once
// per step before any workgroup reads them).
__device__ __forceinline__ f4v ldk4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
typedef unsigned u2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 ldk2(__amdgpu_buffer_rsrc_t r, int off) {
  const u2v v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
}
__device__ __forceinline__ float2 ldc2(__amdgpu_buffer_rsrc_t r, int off) {
  const u2v v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 16);
  return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
}
__device__ __forceinline__ float ldc1(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 16));
}
__device__ __forceinline__ void stc4(__amdgpu_buffer_rsrc_t r, int off, f4v v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4v, v), r, off, 0, 16);
}
// Device-coherent 16-byte load straight into LDS (no registers): lane i's 16
// bytes land at dst + 16 i, dst being wave-uniform (it goes to M0). A lane
// whose offset is past the descriptor's range writes zeros there. The data is
// in LDS once this wave's vector-memory counter has drained (vm_drain).
__device__ __forceinline__ void ldc4_lds(__amdgpu_buffer_rsrc_t r, int off, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 16);
}

// 16-byte load of immutable data (weights, cached KV) through the global
// address space: a generic pointer would compile to a flat load, which also
// counts against the LDS wait counter, so every LDS wait would stall on all
// weight loads in flight.
typedef const __attribute__((address_space(1))) u4v* gptr_u4;
__device__ __forceinline__ uint4 ldg16(const void* p) {
  const u4v v = *(gptr_u4)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The same as a streaming (non-temporal) load: for weights read once per step
// whose wave-wide loads cover whole 1 KiB blocks.
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  const u4v v = __builtin_nontemporal_load((gptr_u4)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef const __attribute__((address_space(1))) uint32_t* gptr_u32;
__device__ __forceinline__ uint32_t ldg4(const void* p) { return *(gptr_u32)(p); }
// The same as a streaming (non-temporal) load: for cached KV rows read once per
// step, whose wave-wide loads cover whole 128-byte lines.
__device__ __forceinline__ uint32_t ldg4_nt(const void* p) { return __builtin_nontemporal_load((gptr_u32)(p)); }

// Wait until every vector memory operation of this wave has completed
// (stores acknowledged by the coherence point).
__device__ __forceinline__ void vm_drain() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// This thread's wave within the workgroup, as a wave-uniform (scalar) value:
// derived from threadIdx.x the compiler would treat it as varying per lane,
// and every address built from it would be too.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// ---------------------------------------------------------------------------
// Events (Event Tensor summary, Core method: notify = atomic decrement,
// wait = spin until zero). An event is kEvInts ints holding 1 + kSubs
// counters 64 bytes apart: [0] and sub-counters [1 + x], x < kSubs. The event
// has fired when all of them are zero. Notifiers decrement one of them (a
// stage with many notifying tasks spreads them over the sub-counters, so no
// single address takes every decrement) with an atomic whose result is not
// awaited; the waiting wave reads all of them at once and votes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int* ev_slot(int* ev, int sub) { return sub >= 0 ? ev + (1 + sub) * kCtr : ev; }

// Whole workgroup: publish this workgroup's completed stores, then notify
// (sub < 0: counter [0]).
__device__ __forceinline__ void wg_notify(int* ev, int sub) {
  vm_drain();
  __syncthreads();
  if (threadIdx.x == 0) (void)atomic_add_relaxed(ev_slot(ev, sub), -1);
}

// One wave: publish this wave's completed stores, then notify. Used where that
// wave alone stored what the event covers; the other waves of the workgroup
// keep their own loads in flight.
__device__ __forceinline__ void wave_notify(int* ev, int sub) {
  vm_drain();
  if ((threadIdx.x & 63) == 0)
    (void)atomic_add_relaxed(ev_slot(ev, sub), -1);
}

// Wave 0 only: spin until the event's counters are all zero (`subs` = number
// of sub-counters to read besides [0]; 0 for a bare counter; a run of flat
// counters may hold up to kMaxHkv). Returns false on abort or watchdog expiry
// (then the error word holds PMK_ERR_TIMEOUT and the abort flag is set, so
// every other waiting workgroup also leaves its loop).
__device__ __forceinline__ bool spin_fail(int* err) {
  if ((threadIdx.x & 63) == 0) {
    int expected = 0;
    __hip_atomic_compare_exchange_strong(gp(err), &expected, (int)PMK_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stci(err + 16, 1);
  }
  return false;
}
// More than 64 counters (a wait on the flat counters of more than 64 KV
// groups): two reads per lane.
__device__ __forceinline__ bool spin_zero_wide(const int* ev, int subs, int* err, unsigned long long ticks) {
  const int lane = threadIdx.x & 63;
  const int* m0 = ev + (lane <= subs ? lane : 0) * kCtr;
  const int* m1 = ev + (lane + 64 <= subs ? lane + 64 : 0) * kCtr;
  const unsigned long long t0 = now_ticks();
  for (int it = 0;; ++it) {
    const int x0 = ldci(m0), x1 = ldci(m1);
    if (__all(x0 == 0 && x1 == 0)) return true;
    __builtin_amdgcn_s_sleep(1);
    if ((it & 15) == 15) {
      if (ldci(err + 16) != 0) return false;
      if (now_ticks() - t0 > ticks) return spin_fail(err);
    }
  }
}
// Up to 64 counters: one read per lane.
__device__ __forceinline__ bool spin_zero(const int* ev, int subs, int* err, unsigned long long ticks) {
  if (subs >= 64) return spin_zero_wide(ev, subs, err, ticks);
  const int lane = threadIdx.x & 63;
  const int* mine = ev + (lane <= subs ? lane : 0) * kCtr;
  if (__all(ldci(mine) == 0)) return true;
  const unsigned long long t0 = now_ticks();
  for (int it = 0;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    if (__all(ldci(mine) == 0)) return true;
    if ((it & 15) == 15) {
      if (ldci(err + 16) != 0) return false;
      if (now_ticks() - t0 > ticks) return spin_fail(err);
    }
  }
}

// Wave 0 only: spin until *p is nonzero and return it; 0 on abort or
// watchdog expiry (which sets the error word and the abort flag as above).
__device__ __forceinline__ int spin_nonzero(const int* p, int* err, unsigned long long ticks) {
  int v = ldci(p);
  if (v != 0) return v;
  const unsigned long long t0 = now_ticks();
  for (int it = 0;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    v = ldci(p);
    if (v != 0) return v;
    if ((it & 15) == 15) {
      if (ldci(err + 16) != 0) return 0;
      if (now_ticks() - t0 > ticks) {
        if ((threadIdx.x & 63) == 0) {
          int expected = 0;
          __hip_atomic_compare_exchange_strong(gp(err), &expected, (int)PMK_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          stci(err + 16, 1);
        }
        return 0;
      }
    }
  }
}

// Whole workgroup: wait until the event has fired (wave 0 spins, the others
// park at the barrier). `flag` is an LDS int. Returns false if the step was
// abandoned.
__device__ __forceinline__ bool wg_wait(const int* ev, int subs, int* err, unsigned long long ticks, int* flag) {
  if (!ev) return true;
  if (threadIdx.x < 64) {
    const bool ok = spin_zero(ev, subs, err, ticks);
    if (threadIdx.x == 0) *flag = ok ? 1 : 0;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*flag) != 0;   // same for every lane: keep it scalar
}

// ---------------------------------------------------------------------------
// Wave reductions (wave64) without the LDS crossbar: DPP moves within a row of
// 16 lanes (quad permutes, half-row and row mirrors) and the gfx950 permlane
// swaps between rows (16: rows 0<->1 and 2<->3; 32: rows 0,1 <-> 2,3).
// ---------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over each row of 16 lanes (every lane of the row gets it).
__device__ __forceinline__ float sum16(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  v += dpp<0x140>(v);   // row_mirror
  return v;
}
// Max over each row of 16 lanes (every lane of the row gets it).
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return v;
}
// Row exchange between two registers holding the same value: afterwards one
// holds rows (0, 0, 2, 2) and the other (1, 1, 3, 3) for the 16-lane swap, or
// (lo, lo) and (hi, hi) for the 32-lane swap. Written as inline assembly (two
// read-write register operands, with the hazard padding the swap needs): the
// compiler's lowering of the builtin here returns one register for both halves.
__device__ __forceinline__ void swap16(float& a, float& b) {
  __asm__ volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// Sum / max over the 4 rows, lane by lane (lane i gets the value of lanes i, i^16, i^32, i^48).
__device__ __forceinline__ float xrow_sum(float v) {
  float a = v, b = v;
  swap16(a, b);
  float c = a + b, d = c;
  swap32(c, d);
  return c + d;
}
__device__ __forceinline__ float xrow_max(float v) {
  float a = v, b = v;
  swap16(a, b);
  float c = fmaxf(a, b), d = c;
  swap32(c, d);
  return fmaxf(c, d);
}
__device__ __forceinline__ float wave_sum(float v) { return xrow_sum(sum16(v)); }
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return xrow_max(v);
}

// ---------------------------------------------------------------------------
// bfloat16 <-> float
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// float -> bfloat16 bits, round to nearest even (the hardware conversion,
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two floats -> packed bfloat16 pair (a in the low half), one conversion
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), b2));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float rnd(float f) { return f; }
  static __device__ __forceinline__ void put(float* p, float f) { *gp(p) = f; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float rnd(float f) { return __uint_as_float((uint32_t)f2bf(f) << 16); }
  static __device__ __forceinline__ void put(uint16_t* p, float f) { *gp(p) = f2bf(f); }
};

// 8 consecutive elements (16 B of bfloat16, or 32 B of float) -> float[8].
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void to(float (&f)[8]) const {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = make_float4(0, 0, 0, 0); b = a; }
  __device__ __forceinline__ void to(float (&f)[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// ---------------------------------------------------------------------------
// Matrix-core step of the weight-streaming GEMV. One "chunk" is one 16-byte
// load per lane: lane l holds 16 bytes of weight row (l & 15) of a 16-row group
// at k-slot group (l >> 4), and the matching 16 bytes of the staged input row
// (l & 15). One chunk covers KSTEP consecutive k of 16 rows.
//  bfloat16: one v_mfma_f32_16x16x32_bf16 (8 k per lane group);
//  float:    four v_mfma_f32_16x16x4_f32 (4 k per lane group, one per MFMA).
// The 16x16 result D[m][j] (input row m, weight row j) sits in lane
// j + 16 * (m / 4), element m % 4.
// ---------------------------------------------------------------------------
template <typename WT> struct MM;
template <> struct MM<uint16_t> {
  static constexpr int EPL = 8;     // elements per 16-byte load
  static constexpr int KSTEP = 32;
  static constexpr int XPAD = 8;    // LDS row padding (elements)
  typedef uint16_t XT;
  static __device__ __forceinline__ f4v mac(uint4 x, uint4 w, f4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, x), __builtin_bit_cast(bf8v, w), c, 0, 0, 0);
  }
  // four consecutive inputs -> LDS (8 bytes)
  static __device__ __forceinline__ void put4(XT* p, f4v v) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pk_bf16(v.x, v.y), pk_bf16(v.z, v.w));
  }
  // two-term split x = hi + lo, both bfloat16 (hi nearest to x, lo nearest to
  // the remainder): products with bfloat16 weights are exact in the MFMA's
  // float32 accumulation, so the pair carries x to about 2^-16 relative
  static __device__ __forceinline__ void put4_split(XT* hi, XT* lo, f4v v) {
    const uint32_t h01 = pk_bf16(v.x, v.y), h23 = pk_bf16(v.z, v.w);
    const f4v h = {bf_lo(h01), bf_hi(h01), bf_lo(h23), bf_hi(h23)};
    *reinterpret_cast<uint2*>(hi) = make_uint2(h01, h23);
    put4(lo, v - h);
  }
};
template <> struct MM<float> {
  static constexpr int EPL = 4;
  static constexpr int KSTEP = 16;
  static constexpr int XPAD = 4;
  typedef float XT;
  static __device__ __forceinline__ f4v mac(uint4 x, uint4 w, f4v c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.x), __uint_as_float(w.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.y), __uint_as_float(w.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.z), __uint_as_float(w.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.w), __uint_as_float(w.w), c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ void put4(XT* p, f4v v) { *reinterpret_cast<f4v*>(p) = v; }
  static __device__ __forceinline__ void put4_split(XT* hi, XT* lo, f4v v) {
    put4(hi, v);
    put4(lo, f4v{0.f, 0.f, 0.f, 0.f});
  }
};

}  // namespace pmk
