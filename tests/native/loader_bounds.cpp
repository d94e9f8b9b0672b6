// Host-side check of the forward kernel's tile-copy maps (fb_tile_map.h), for every
// 16-bit kernel shape that the library instantiates: every byte a direct load reads lies
// inside its source row (K and V rows of D elements, phi_k rows of R elements), and every
// chunk slot of the K, phi_k and V regions is written by exactly one lane of one load.
// Prints one line per shape and exits non-zero on the first violation.
#include <cstdio>
#include <vector>

#include "fb_tile_map.h"

using namespace fb::attn;

static int check(int D, int RP, int R, bool loader) {
  const int CE = 8;                       // 16-bit elements per 16-byte chunk
  const int KCH = D / CE;
  const int PCH = RP / CE;
  const int DP = D < 32 ? 32 : D;
  const int VCH = DP / CE;
  const int npch = R / CE;                // phi_k chunks with data (R a multiple of a chunk)
  const int NDMA = KCH + PCH + VCH;
  std::vector<int> seen[3];
  const int cprs[3] = {KCH, PCH, VCH};
  for (int r = 0; r < 3; ++r) seen[r].assign(64 * (cprs[r] > 0 ? cprs[r] : 1), 0);
  for (int n = 0; n < NDMA; ++n) {
    for (int lane = 0; lane < 64; ++lane) {
      const TileSlot d = tile_slot(n, lane, KCH, PCH, VCH);
      if (d.row < 0 || d.row >= 64 || d.c < 0 || d.c >= d.cpr) {
        std::printf("D=%d RP=%d R=%d: load %d lane %d maps to row %d chunk %d of %d\n", D, RP, R, n, lane, d.row,
                    d.c, d.cpr);
        return 1;
      }
      seen[d.region][d.row * d.cpr + d.c] += 1;
      const int row_bytes = d.region == 1 ? 2 * R : 2 * D;
      const bool data = slot_has_data(d, KCH, npch);
      const int byte = loader ? loader_src_byte(d, KCH, npch) : d.c * 16;
      if ((loader || data) && byte + 16 > row_bytes) {
        std::printf("D=%d RP=%d R=%d %s: load %d lane %d (region %d, chunk %d) reads bytes [%d, %d) of a %d-byte row\n",
                    D, RP, R, loader ? "loader" : "compute", n, lane, d.region, d.c, byte, byte + 16, row_bytes);
        return 1;
      }
    }
  }
  for (int r = 0; r < 3; ++r) {
    if (cprs[r] == 0) continue;
    for (size_t i = 0; i < seen[r].size(); ++i) {
      if (seen[r][i] != 1) {
        std::printf("D=%d RP=%d: region %d slot %zu written %d times\n", D, RP, r, i, seen[r][i]);
        return 1;
      }
    }
  }
  std::printf("ok D=%d RP=%d R=%d %s: %d loads x 64 lanes in bounds, every slot once\n", D, RP, R,
              loader ? "loader" : "compute", NDMA);
  return 0;
}

// The resident kernel copies every tile of one (b, h): load g of the workgroup is load
// g mod NDMA of tile g / NDMA, written at tile * (tile bytes) + 1024 (load within the region)
// + 16 lane.  With the most tiles that fit (the host admits N <= res_max_keys), every write
// must land inside the K' and V arrays and both must fit the workgroup's LDS.
static int check_resident(int D, int RP) {
  const int CE = 8;
  const int KCH = D / CE, PCH = RP / CE, VCH = (D < 32 ? 32 : D) / CE;
  const int NDMA = KCH + PCH + VCH;
  const int SKB = 1024 * (KCH + PCH), SVB = 1024 * VCH;
  const int T = res_max_tiles(D, RP);
  if (T < 1 || T * (SKB + SVB) > kResLdsBytes || SKB + SVB != res_tile_bytes(D, RP)) {
    std::printf("resident D=%d RP=%d: %d tiles of %d bytes do not fit %d\n", D, RP, T, SKB + SVB, kResLdsBytes);
    return 1;
  }
  for (int g = 0; g < T * NDMA; ++g) {
    const int t = g / NDMA, n = g % NDMA;
    for (int lane = 0; lane < 64; ++lane) {
      const bool isv = n >= KCH + PCH;
      const int off = isv ? t * SVB + (n - KCH - PCH) * 1024 + 16 * lane : t * SKB + n * 1024 + 16 * lane;
      if (off < 0 || off + 16 > (isv ? T * SVB : T * SKB)) {
        std::printf("resident D=%d RP=%d: load %d lane %d writes bytes [%d, %d)\n", D, RP, g, lane, off, off + 16);
        return 1;
      }
    }
  }
  std::printf("ok resident D=%d RP=%d: %d tiles (%d keys), %d bytes of LDS\n", D, RP, T, res_max_keys(D, RP),
              T * (SKB + SVB));
  return 0;
}

int main() {
  int bad = 0;
  for (int D : {16, 32, 64})
    for (int RP : {0, 16, 32}) bad |= check_resident(D, RP);
  const int Ds[] = {16, 32, 64, 128};
  const int RPs[] = {0, 16, 32, 64, 128};
  for (int D : Ds)
    for (int RP : RPs) {
      // R values whose phi_k rows go by direct loads: multiples of a chunk in (RP - 16, RP]
      for (int R = RP > 0 ? RP - 8 : 0; R <= RP; R += 8) {
        if (RP > 0 && R <= 0) continue;
        const bool loader = D <= 64 && RP <= 64;   // the kernels that run loader wavefronts
        bad |= check(D, RP, R, false);
        if (loader) bad |= check(D, RP, R, true);
      }
    }
  return bad;
}
