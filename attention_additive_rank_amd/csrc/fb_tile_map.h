// Index maps of the fused attention kernels' LDS tiles: plain integer functions, usable
// on the host (the CPU bounds test compiles this header with g++) and on the device.
//
// A tile holds 64 keys.  Its K' part is two row-major regions, K (64 rows x KCH chunks of
// 16 bytes) then phi_k (64 x PCH chunks), and its V part one region of 64 x VCH chunks.
// Chunk c of row r is stored at position c ^ swz(r) inside its row, which keeps every
// row's chunks in the row while spreading the rows over the LDS banks.
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define FB_HD __host__ __device__
#else
#define FB_HD
#endif

namespace fb {
namespace attn {

// Position inside a 32-row MFMA block that holds logical index k (key or head dim):
// MFMA row m = 8a + 4h + c carries index 16h + 4a + c, so that output register r
// of lane half h corresponds to index 16h + r.
FB_HD constexpr int perm_row(int k) {
  return (k & ~31) | (((k & 15) >> 2) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}
// The inverse: the logical index held by MFMA row r.
FB_HD constexpr int inv_perm_row(int r) {
  return (r & ~31) | (((r >> 2) & 1) << 4) | (((r & 31) >> 3) << 2) | (r & 3);
}

// Swizzles of a region with cpr chunks per row (cpr a power of two).  The LDS serves a
// 128-bit read in passes of 16 lanes over 64 four-byte banks (256 bytes), so the lanes of
// a pass must touch 16 different 16-byte bank groups, i.e. distinct (row * cpr + position)
// mod 16:
//   swz_rows: 16 consecutive rows read at one chunk (the score MFMA operands);
//   swz_quad: four consecutive rows read at four adjacent chunks (the 64-bit transpose
//             reads of V, 32 lanes of 8 bytes per pass).
FB_HD constexpr int swz_rows(int cpr, int r) {
  return cpr >= 16 ? (r & 15) : cpr == 8 ? ((r >> 1) & 7) : cpr == 4 ? ((r >> 2) & 3) : cpr == 2 ? ((r >> 2) & 1) : 0;
}
FB_HD constexpr int swz_quad(int cpr, int r) {
  return cpr >= 8 ? 2 * (r & 3) : cpr == 4 ? 2 * ((r >> 1) & 1) : 0;
}
// K and phi_k rows are stored in key order but read by the score MFMA in the order of
// perm_row (lane ln of a 32-key block reads key inv_perm_row(ln)), so their swizzle follows
// the reading lane: eight lanes that read together still hit eight bank groups.
FB_HD constexpr int swz_key(int cpr, int key) { return swz_rows(cpr, perm_row(key)); }

// One 1 KB direct load of a tile fills 64 consecutive chunk slots of a region (whole rows).
// Load n covers K-region bytes [1024 n, 1024 (n+1)) for n < KCH, then the phi_k region,
// then V.  Lane l of load n writes chunk slot l of its 1 KB: row n' (64 / cpr) + l / cpr at
// position l % cpr, which holds logical chunk (l % cpr) ^ swz(row).
struct TileSlot {
  int region;   // 0 K, 1 phi_k, 2 V
  int cpr;      // chunks per row of the region
  int row;      // key row within the tile
  int c;        // logical chunk (16-byte column block) of that row
};
FB_HD constexpr TileSlot tile_slot(int n, int lane, int KCH, int PCH, int VCH) {
  TileSlot d{0, KCH, 0, 0};
  int nr = n;
  if (n < KCH) {
    d.region = 0;
    d.cpr = KCH;
  } else if (n < KCH + PCH) {
    d.region = 1;
    d.cpr = PCH;
    nr = n - KCH;
  } else {
    d.region = 2;
    d.cpr = VCH;
    nr = n - KCH - PCH;
  }
  d.row = nr * (64 / d.cpr) + lane / d.cpr;
  d.c = (lane % d.cpr) ^ (d.region == 2 ? swz_quad(d.cpr, d.row) : swz_key(d.cpr, d.row));
  return d;
}

// Whether a slot holds data of its source row: every K chunk; phi_k chunks below npch (the
// row's R columns in whole chunks); V chunks below KCH (a V row has D columns, KCH chunks,
// while the region may be wider: VCH > KCH when D < 32).
FB_HD constexpr bool slot_has_data(const TileSlot& d, int KCH, int npch) {
  return d.region == 0 || (d.region == 1 ? d.c < npch : d.c < KCH);
}

// Byte offset within its source row that a loader wavefront copies for a slot.  Loader
// wavefronts issue every load with all lanes active (their wait counts loads), so a slot
// without data copies a finite stand-in from inside the same row, chunk 0: for phi_k it
// meets zero phi_q columns, for V it only feeds head dims >= D, which are never stored.
FB_HD constexpr int loader_src_byte(const TileSlot& d, int KCH, int npch) {
  return slot_has_data(d, KCH, npch) ? d.c * 16 : 0;
}

// The resident-K'/V kernel (fb_attn_resident.h) holds every tile of one (b, h) in LDS: at most
// 80 KB per workgroup (two workgroups per compute unit).  Bytes of one 64-key tile (K rows, RP
// factor columns, V rows at least 32 wide), and the tiles / keys that fit.
constexpr int kResLdsBytes = 80 * 1024;
FB_HD constexpr int res_tile_bytes(int D, int RP) { return 64 * 2 * (D + RP + (D < 32 ? 32 : D)); }
FB_HD constexpr int res_max_tiles(int D, int RP) { return kResLdsBytes / res_tile_bytes(D, RP); }
FB_HD constexpr int res_max_keys(int D, int RP) { return 64 * res_max_tiles(D, RP); }

}  // namespace attn
}  // namespace fb
