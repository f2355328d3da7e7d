// pmk_probe.hip -- a plain streaming-read kernel: the bandwidth a kernel that
// does nothing but read HBM reaches on this device, with the two weight access
// patterns of the decode step's GEMV engine, as the reference point next to the
// 8 TB/s nominal peak for the decode kernel's roofline figures.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
