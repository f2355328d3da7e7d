// Checks the dense stages' work split (stage_geo in pmk_internal.h) on the
// host: for every depth, row count, batch and grid share used by the decode
// shapes, the split it returns covers the depth with whole ring-length
// slices, fits the LDS, keeps the tile count within the grid, and splits
// nothing at batch 1. For a split, the slice record (a tile's sums, then its
// rows' sums of squares) has a stride of whole 16-byte units that covers it,
// and the last slice task's landing area for the other slices' records (1 KiB
// blocks per slice) fits below the pass outputs in LDS, so the records are
// pulled in one round trip. Prints "ok <cases>" or the first failing case.
#include <cstdio>

#include "../../persistent_megakernel_04_amd/csrc/pmk_internal.h"

using namespace pmk;

int main() {
  const int Ks[] = {256, 512, 688, 2048, 4096, 5120, 8192, 14336, 28672};
  const int units[] = {64, 128, 344, 688, 2048, 3072, 4096, 5120, 8192, 14336, 28672};
  const int urows[] = {1, 2};
  const int avails[] = {192, 256};   // the grid (256 CUs) and its share without the attention workgroups
  const int steps[][2] = {{32, 8}, {16, 4}};   // bfloat16 and float: k per load step, LDS row padding
  long cases = 0;
  for (auto& st : steps)
    for (int K : Ks)
      for (int U : units)
        for (int R : urows)
          for (int nb = 1; nb <= kMaxNb; ++nb)
            for (int avail : avails) {
              ++cases;
              const StageGeo g = stage_geo(K, U, R, nb, avail, st[0], st[1]);
              const int grain = kRingK * st[0];
              auto fail = [&](const char* why) {
                std::printf("FAIL %s: K %d units %d urows %d nb %d avail %d kstep %d -> ks %d tiles %d kr %d\n", why, K,
                            U, R, nb, avail, st[0], g.ks, g.tiles, g.kr);
                return 1;
              };
              if (g.blk != 1) return fail("blk");
              if (g.ks == 0) {   // no split within kMaxKs slices: the caller makes passes instead
                const int kr8 = ((K + kMaxKs - 1) / kMaxKs + grain - 1) / grain * grain, t8 = avail / kMaxKs;
                const long rows8 = (long)(U + t8 - 1) / t8 * R;
                if (nb * (kr8 + st[1]) * 4L + rows8 * nb * 4 + 16 <= kXyBytes) return fail("gave up on a split that fits");
                continue;
              }
              if (g.ks < 1 || g.ks > kMaxKs) return fail("slice count");
              if (g.tiles < 1 || g.tiles > U || (g.tiles > avail && g.tiles > 1)) return fail("tile count");
              if ((long)(g.ks - 1) * g.kr >= K || (long)g.ks * g.kr < K) return fail("slices do not cover K");
              if (g.kr != K && g.kr % grain != 0) return fail("slice not whole ring lengths");
              const long rows = (long)(U + g.tiles - 1) / g.tiles * R;
              const long xs = (long)nb * ((g.kr + st[0] - 1) / st[0] * st[0] + st[1]) * 4;
              if ((xs + 15) / 16 * 16 + rows * nb * 4 > kXyBytes && g.kr > grain) return fail("does not fit the LDS");
              if (nb == 1 && K <= 28672 && g.ks != 1) return fail("split at batch 1");
              if (g.ks > 1) {
                // the kernel's record stride (rows of the stage's largest tile) and a normed record's length
                const long rs = ((long)(U + g.tiles - 1) / g.tiles * R * nb + 16 + 3) & ~3L;
                const long nrec = rows * nb + nb, units4 = (nrec + 3) / 4;
                if (rs % 4 != 0 || 4 * units4 > rs) return fail("record stride");
              }
            }
  // Batches beyond 16 (stage_split): blocks of 16 rows over row tiles sized
  // for fewer tasks than one set per block. Every split with more than one
  // tile set per workgroup's share must fit the LDS outright; the whole-share
  // split keeps stage_geo's rule; slices cover K; blocks match the batch.
  {
    struct BShape { int H, Hq, Hkv, d, F, kstep, xpad; };
    const BShape bshapes[] = {{4096, 32, 8, 128, 14336, 32, 8}, {2048, 32, 4, 128, 0, 32, 8},
                              {8192, 64, 8, 128, 28672, 32, 8}, {256, 4, 2, 64, 688, 16, 4},
                              {4096, 4, 2, 64, 256, 16, 4}};
    const int bavails[] = {192, 240, 256, 304, 80};
    for (const BShape& sh : bshapes)
      for (int st = 0; st < 4; ++st) {
        if (st >= 2 && sh.F == 0) continue;
        const int K4[4] = {sh.H, sh.Hq * sh.d, sh.H, sh.F};
        const int U4[4] = {(sh.Hq + 2 * sh.Hkv) * sh.d / 2, sh.H, sh.F, sh.H};
        const int R4[4] = {2, 1, 2, 1};
        const int grain = kRingK * sh.kstep;
        for (int B = 17; B <= 1024; B += (B < 64 ? 1 : 16))
          for (int avail : bavails) {
            ++cases;
            const StageGeo g = stage_split(K4[st], U4[st], R4[st], B, avail, sh.kstep, sh.xpad);
            const StageGeo whole = stage_geo(K4[st], U4[st], R4[st], kMaxNb, avail, sh.kstep, sh.xpad);
            auto fail = [&](const char* why) {
              std::printf("FAIL %s: H %d stage %d B %d avail %d -> ks %d tiles %d kr %d blk %d\n", why, sh.H, st, B,
                          avail, g.ks, g.tiles, g.kr, g.blk);
              return 1;
            };
            if (whole.ks == 0) {   // passes over the batch, as before
              if (g.blk != 1 || g.ks != 1) return fail("no split fits, yet blocks");
              continue;
            }
            if (g.blk != (B + kMaxNb - 1) / kMaxNb) return fail("block count");
            if (g.ks < 1 || g.ks > kMaxKs) return fail("slice count");
            if ((long)(g.ks - 1) * g.kr >= K4[st] || (long)g.ks * g.kr < K4[st]) return fail("slices do not cover K");
            if (g.tiles < 1 || g.tiles > U4[st] || g.tiles > whole.tiles) return fail("tile count");
            const bool is_whole = g.tiles == whole.tiles && g.ks == whole.ks && g.kr == whole.kr;
            if (!is_whole && !stage_fits(g, U4[st], R4[st], kMaxNb, sh.kstep, sh.xpad)) return fail("does not fit the LDS");
            if (is_whole && !stage_fits(g, U4[st], R4[st], kMaxNb, sh.kstep, sh.xpad) && g.kr > grain)
              return fail("whole-share split does not fit the LDS");
            // fewer tasks per workgroup than one set of tiles per block, where the blocks outnumber one
            if ((long)g.tiles * g.ks * g.blk > (long)whole.tiles * whole.ks * g.blk) return fail("more tasks");
          }
      }
  }
  // The decode workloads' own splits pull the other slices' records into LDS
  // in one round trip (the kernel falls back to register loads otherwise,
  // e.g. for the 70B-shaped gate/up tiles at 10 to 16 rows).
  struct Shape { int H, Hq, Hkv, d, F, nb_lo, nb_hi; };
  const Shape shapes[] = {{4096, 32, 8, 128, 14336, 2, 16},   // 8B-shaped stack, batch 2..16 (and 16-row blocks)
                          {2048, 32, 4, 128, 0, 2, 16},       // MoE layer's attention projections
                          {8192, 64, 8, 128, 28672, 8, 8}};   // 70B-shaped stack, batch 8
  for (const Shape& sh : shapes)
    for (int st = 0; st < 4; ++st) {
      if (st >= 2 && sh.F == 0) continue;
      const int K4[4] = {sh.H, sh.Hq * sh.d, sh.H, sh.F};
      const int U4[4] = {(sh.Hq + 2 * sh.Hkv) * sh.d / 2, sh.H, sh.F, sh.H};
      const int R4[4] = {2, 1, 2, 1};
      for (int nb = sh.nb_lo; nb <= sh.nb_hi; ++nb)
        for (int avail : avails) {
          ++cases;
          const StageGeo g = stage_geo(K4[st], U4[st], R4[st], nb, avail, 32, 8);
          if (g.ks <= 1) continue;
          const long rows = (long)(U4[st] + g.tiles - 1) / g.tiles * R4[st];
          const long xs = (long)nb * ((g.kr + 31) / 32 * 32 + 8) * 4;
          const long units4 = (rows * nb + nb + 3) / 4;
          const long land = (long)(g.ks - 1) * ((units4 + 63) / 64) * 1024;
          if (land > (xs + 15) / 16 * 16) {
            std::printf("FAIL slice records do not fit below the outputs: H %d stage %d nb %d avail %d ks %d\n", sh.H,
                        st, nb, avail, g.ks);
            return 1;
          }
        }
    }
  // Split-K record extent against the allocation. For every batch the
  // prologue may see and every share it may give QKV and O (a quarter of the
  // grid at most goes to attention workgroups of their own), the records the
  // kernel writes -- task (tile t, slice s, block k) at record
  // ((k tiles + t) ks + s), each `rs` floats holding the tile's rows x nb sums
  // and nb sums of squares -- must lie inside the workspace's kpart region,
  // sized by kpart_need. rs is written out here from the kernel's addressing.
  struct KShape { int H, Hq, Hkv, d, F, kstep, xpad, max_batch; };
  const KShape kshapes[] = {
      {4096, 32, 8, 128, 14336, 32, 8, 128},   // 8B-shaped
      {8192, 64, 8, 128, 28672, 32, 8, 16},    // 70B-shaped
      {2048, 32, 4, 128, 0, 32, 8, 128},       // MoE layer's attention projections
      {8192, 8, 1, 128, 3584, 32, 8, 16},      // a tensor-parallel share of the 70B shape
      {4096, 4, 2, 64, 256, 16, 4, 16},        // float32, small QKV: the shares change the split's record size
      {1024, 8, 2, 64, 4096, 16, 4, 16},
      {256, 4, 2, 64, 688, 16, 4, 4}};
  const int grids[] = {256, 304, 240, 80};
  for (const KShape& sh : kshapes)
    for (int G : grids)
      for (int st = 0; st < 4; ++st) {
        if (st >= 2 && sh.F == 0) continue;
        const int K4[4] = {sh.H, sh.Hq * sh.d, sh.H, sh.F};
        const int U4[4] = {(sh.Hq + 2 * sh.Hkv) * sh.d / 2, sh.H, sh.F, sh.H};
        const int R4[4] = {2, 1, 2, 1};
        const long alloc = kpart_need(K4[st], U4[st], R4[st], sh.max_batch, G, st <= 1, sh.kstep, sh.xpad);
        for (int B = 1; B <= sh.max_batch; ++B)
          for (int own = 0; own <= (st <= 1 ? G / 4 : 0); ++own) {
            ++cases;
            const int nb = B < kMaxNb ? B : kMaxNb;
            StageGeo g = stage_split(K4[st], U4[st], R4[st], B, G - own, sh.kstep, sh.xpad);
            if (g.ks <= 1) continue;   // no records (or passes over the batch)
            const long blk = g.blk;
            const long rows = (long)(U4[st] + g.tiles - 1) / g.tiles * R4[st];
            const long rs = (rows * (blk > 1 ? kMaxNb : nb) + 16 + 3) & ~3L;
            const long used = rows * nb + nb;   // sums, then sums of squares
            const long extent = (blk * g.tiles * g.ks - 1) * rs + used;
            if (rs % 4 || used > rs || extent > alloc) {
              std::printf("FAIL split-K records past the allocation: H %d Hq %d Hkv %d d %d F %d grid %d stage %d "
                          "batch %d own %d: ks %d tiles %d rs %ld extent %ld alloc %ld\n",
                          sh.H, sh.Hq, sh.Hkv, sh.d, sh.F, G, st, B, own, g.ks, g.tiles, rs, extent, alloc);
              return 1;
            }
          }
      }
  std::printf("ok %ld\n", cases);
  return 0;
}
