// pmk_probe.hip -- two diagnostics beside the decode library:
//  * a plain streaming-read kernel: the bandwidth a kernel that does nothing
//    but read HBM reaches on this device, with the two weight access patterns
//    of the decode step's GEMV engine, as the reference point next to the
//    8 TB/s nominal peak for the decode kernel's roofline figures;
//  * a cross-XCD message-passing litmus of the persistent kernel's
//    synchronisation scheme, built from the same device primitives.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmk_device.h"
#include "pmk_internal.h"

namespace pmk {

typedef unsigned pu4v __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) pu4v* pgp;

// Each wave streams 16 KiB blocks, 16 loads of 16 bytes per lane in flight
// (the GEMV engine's ring depth). Block b of the buffer:
//  pattern 0 (tile layout): 16 contiguous 1 KiB pieces; load d of lane l
//    reads piece d at byte 16 l, non-temporally;
//  pattern 1 (row-major weights): the buffer as rows of 8 KiB; block b is row
//    group b / 8 (16 rows), k-slice b % 8 (1 KiB of each row); load d of lane
//    l reads row l % 16 at byte 64 d + 16 (l / 16) of the slice (16 rows x
//    64 bytes per instruction), through the caches.
// Blocks are dealt to waves round-robin over the grid. Every load stays
// inside [0, nblocks * 16 KiB).
template <int P>
__global__ void __launch_bounds__(kBlock, 1) pmk_stream(const char* __restrict__ src, long nblocks, int* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long nw = (long)gridDim.x * kWaves;
  auto addr = [&](long b, int d) -> long {
    if (P == 0) return b * 16384 + d * 1024 + lane * 16;
    const long rg = b >> 3, ks = b & 7;
    return rg * 16 * 8192 + (lane & 15) * 8192 + ks * 1024 + d * 64 + (lane >> 4) * 16;
  };
  auto ld = [&](long off) -> pu4v {
    if (P == 0) return __builtin_nontemporal_load((pgp)(src + off));
    return *(pgp)(src + off);
  };
  pu4v acc = {0u, 0u, 0u, 0u};
  long b = blockIdx.x * (long)kWaves + wave;
  if (b >= nblocks) return;
  pu4v ring[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) ring[d] = ld(addr(b, d));
  for (;;) {
    const long bn = b + nw;
    const bool more = bn < nblocks;
    const long br = more ? bn : b;   // past the end: re-read this block (in bounds), not used
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      acc ^= ring[d];
      ring[d] = ld(addr(br, d));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!more) break;
    b = bn;
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) atomicAdd(sink, 1);   // keeps the loads
}


// ---------------------------------------------------------------------------
// Cross-XCD litmus. Round r: workgroup p = r mod grid writes a fresh 4 KiB
// block (its own address, written once: as the step's activations) and a
// reused 4 KiB block (the same address every round: as the split-K records)
// with device-coherent 16-byte stores, drains its stores and decrements the
// round's counter with a relaxed agent-scope atomic (wg_notify). Its next
// eight workgroups -- on the eight XCDs, workgroups being dealt to XCDs round
// robin -- wait for the counter with the kernel's watchdog-bounded spin, read
// the fresh block through the caches (ldk4, as activations are staged) and
// the reused block device-coherently (ldc4, as split-K records are), check
// every element, and acknowledge; the next round's writer waits for the
// acknowledgements before it rewrites the reused block. The first stale
// value stops the run. Also counted, not checked: the reused block read
// through the caches, the access the kernels avoid.
//   result[0] first stale round (-1: none), [1] element, [2] value read,
//   [3] value expected, [4] block (0 fresh, cached; 1 reused, coherent),
//   [5] 1 if a wait timed out, [6] rounds checked by the consumers, [7] stale
//   values of the reused block read through the caches.
// ---------------------------------------------------------------------------
constexpr int kLitConsumers = 8;
constexpr int kLitInts = 1024;   // 4 KiB per block: 256 threads x 16 bytes

__global__ void pmk_litmus_init(int* flag, int* ack, int* err, int rounds, int* result) {
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < rounds; r += gridDim.x * blockDim.x) {
    flag[(size_t)r * kCtr] = 1;
    ack[(size_t)r * kCtr] = kLitConsumers;
  }
  if (blockIdx.x == 0 && threadIdx.x < 64) err[threadIdx.x] = 0;
  if (blockIdx.x == 0 && threadIdx.x < 8) result[threadIdx.x] = threadIdx.x == 0 ? -1 : 0;
}

__global__ void __launch_bounds__(256, 1) pmk_litmus(int* fresh, int* reuse, int* flag, int* ack, int* err,
                                                     int rounds, int* result, unsigned long long ticks) {
  __shared__ int ok;
  const int G = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const auto rr = rsrc(reuse);
  for (int r = 0; r < rounds; ++r) {
    const int p = r % G, k = (wg - p - 1 + G) % G;
    if (wg == p) {   // writer
      if (r > 0 && !wg_wait(ack + (size_t)(r - 1) * kCtr, 0, err, ticks, &ok)) break;
      const auto fr = rsrc(fresh + (size_t)r * kLitInts);
      const int v = r * kLitInts + 4 * tid;
      const f4v x = {__int_as_float(v), __int_as_float(v + 1), __int_as_float(v + 2), __int_as_float(v + 3)};
      stc4(fr, 16 * tid, x);
      stc4(rr, 16 * tid, x);
      wg_notify(flag + (size_t)r * kCtr, -1);
    }
    if (k < kLitConsumers) {   // reader
      if (!wg_wait(flag + (size_t)r * kCtr, 0, err, ticks, &ok)) break;
      const auto fr = rsrc(fresh + (size_t)r * kLitInts);
      const f4v a = ldk4(fr, 16 * tid), b = ldc4(rr, 16 * tid), c = ldk4(rr, 16 * tid);
      int bad = -1, got = 0, blk = 0, stale_c = 0;
      for (int j = 0; j < 4; ++j) {
        const int want = r * kLitInts + 4 * tid + j;
        const int ga = __float_as_int(a[j]), gb = __float_as_int(b[j]);
        if (bad < 0 && ga != want) { bad = 4 * tid + j; got = ga; blk = 0; }
        if (bad < 0 && gb != want) { bad = 4 * tid + j; got = gb; blk = 1; }
        stale_c += __float_as_int(c[j]) != want;
      }
      if (stale_c) atomicAdd(result + 7, stale_c);
      if (bad >= 0 && atomicCAS(result, -1, r) == -1) {
        result[1] = bad;
        result[2] = got;
        result[3] = r * kLitInts + bad;
        result[4] = blk;
        stci(err + 16, 1);   // every workgroup leaves its loop
      }
      __syncthreads();
      if (tid == 0) {
        atomicAdd(result + 6, 1);
        (void)atomic_add_relaxed(ack + (size_t)r * kCtr, -1);
      }
      if (ldsu(err + 16) != 0) break;
    }
  }
  if (tid == 0 && ldci(err) == PMK_ERR_TIMEOUT) result[5] = 1;
}

}  // namespace pmk

using namespace pmk;

extern "C" int pmk_stream_probe(const void* buf, int64_t bytes, int32_t pattern, int32_t reps, int* sink,
                                void* stream, double* ms_out) {
  if (!buf || !sink || !ms_out || bytes <= 0 || bytes % (1 << 20) || reps < 1 || (pattern != 0 && pattern != 1))
    return PMK_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(buf) & 255) return PMK_ERR_ARG;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return PMK_ERR_DEVICE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const long nblocks = bytes / 16384;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return PMK_ERR_DEVICE;
  if (hipEventCreate(&e1) != hipSuccess) { (void)hipEventDestroy(e0); return PMK_ERR_DEVICE; }
  int rc = PMK_OK;
  double best = 1e30;
  for (int r = 0; r < reps && rc == PMK_OK; ++r) {
    if (hipEventRecord(e0, s) != hipSuccess) { rc = PMK_ERR_DEVICE; break; }
    if (pattern == 0)
      hipLaunchKernelGGL(pmk_stream<0>, dim3(prop.multiProcessorCount), dim3(kBlock), 0, s,
                         static_cast<const char*>(buf), nblocks, sink);
    else
      hipLaunchKernelGGL(pmk_stream<1>, dim3(prop.multiProcessorCount), dim3(kBlock), 0, s,
                         static_cast<const char*>(buf), nblocks, sink);
    if (hipGetLastError() != hipSuccess || hipEventRecord(e1, s) != hipSuccess ||
        hipEventSynchronize(e1) != hipSuccess) { rc = PMK_ERR_DEVICE; break; }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) { rc = PMK_ERR_DEVICE; break; }
    if (ms < best) best = ms;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc == PMK_OK) *ms_out = best;
  return rc;
}

extern "C" int pmk_event_litmus(void* work, int64_t bytes, int32_t rounds, int32_t* result, void* stream) {
  if (!work || !result || rounds < 1 || rounds > (1 << 20)) return PMK_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(work) & 255) return PMK_ERR_ARG;
  const int64_t need = (int64_t)rounds * (kLitInts * 4 + 2 * kCtr * 4) + kLitInts * 4 + 256;
  if (bytes < need) return PMK_ERR_ARG;
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < kLitConsumers + 1)
    return PMK_ERR_DEVICE;
  char* base = static_cast<char*>(work);
  int* fresh = reinterpret_cast<int*>(base);
  int* reuse = fresh + (size_t)rounds * kLitInts;
  int* flag = reuse + kLitInts;
  int* ack = flag + (size_t)rounds * kCtr;
  int* err = ack + (size_t)rounds * kCtr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(pmk_litmus_init, dim3(64), dim3(256), 0, s, flag, ack, err, (int)rounds, (int*)result);
  if (hipGetLastError() != hipSuccess) return PMK_ERR_DEVICE;
  unsigned long long ticks = 200000000ull;   // 2 s of the 100 MHz clock per wait
  int nr = rounds;
  void* args[] = {&fresh, &reuse, &flag, &ack, &err, &nr, &result, &ticks};
  if (hipLaunchCooperativeKernel((const void*)pmk_litmus, dim3(cu), dim3(256), args, 0, s) != hipSuccess)
    return PMK_ERR_DEVICE;
  return PMK_OK;
}
