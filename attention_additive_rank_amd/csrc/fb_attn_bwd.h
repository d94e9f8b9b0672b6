// Fused backward kernels of attention with an additive low-rank bias on gfx950.
//
// The forward computes O = softmax(S) V with S = Q' K'^T, Q' = [Q*s, phi_q], K' = [K, phi_k]
// (FlashBias rebuttal, answer to Reviewer UJUf, Q2).  With the row log-sum-exp L of the
// forward, P = exp(S - L), and Delta_i = sum_d dO_id O_id, the gradients are
//   dV = P^T dO,   dP = dO V^T,   dS = P .* (dP - Delta),
//   dQ' = dS K'  -> dQ = s dS K,  dphi_q = dS phi_k,
//   dK' = dS^T Q' -> dK = dS^T (Q s), dphi_k = dS^T phi_q,
// i.e. the factor gradients are the last R columns of dQ' / dK' (the pages train with
// these biases: rebuttal, answer to Reviewer UJUf, Q1, GPT-2 with Sandwich bias).
// Nothing N x N is stored: both kernels recompute S and P tile by tile from Q', K' and L.
//
//   attn_bwd_dkv_kernel: a workgroup owns 128 keys (32 per wavefront) and streams the
//     query tiles: S, dP, P, dS per 32-query block, then dV^T += dO^T P and
//     dK'^T += Q'^T dS, with the transposed operands read by 64-bit transpose reads;
//   attn_bwd_dq_kernel: a workgroup owns 128 queries (32 per wavefront, the forward's
//     orientation S^T = K' Q'^T) and streams the key tiles: S^T, dP^T = V dO^T, P^T,
//     dS^T, then dQ'^T += K'^T dS^T.
// Layout conventions are the forward's: the score MFMA reads rows in inv_perm_row order
// so that output register r of lane half h is row 16h + r; transposed A operands come
// from ds_read_b64_tr_b16 with k-slot j of half h in k-step u = row 16h + 8u + j, which
// matches the register order of P / dS used as B operands.  Tiles arrive by direct
// global->LDS loads (1 KB of consecutive rows per load) two tiles ahead, in three buffers.
#pragma once

#include "fb_attn_kernel.h"

namespace fb {


namespace attnb {
using namespace fb::attn;

constexpr int BW = 4;             // wavefronts per workgroup
constexpr int BTH = BW * 64;      // threads per workgroup
constexpr int TR = 64;            // rows per streamed tile
static_assert(32 * BW == kBwdRows, "backward block size");

// Streamed tile: region X (KCH chunks per row, 16-bit, the Q or K operand), region F
// (FCH chunks, the factor columns, at least four chunks so that a 32-column transposed
// read stays inside the row; columns at or beyond R hold finite stand-ins), region Y (KCH
// chunks: dO or V), and for the key-major kernel 512 bytes of L and Delta of the tile's
// queries.  Rows are stored in order; chunk c of row r sits at c ^ swzb(cpr, r).
template <int D, int RP, bool LD>
struct Tile {
  static constexpr int KCH = D / 8;
  static constexpr int FCH = RP == 0 ? 0 : (RP / 8 < 4 ? 4 : RP / 8);
  static constexpr int XOFF = 0;
  static constexpr int FOFF = TR * KCH * 16;
  static constexpr int YOFF = FOFF + TR * FCH * 16;
  static constexpr int LOFF = YOFF + TR * KCH * 16;
  static constexpr int BYTES = LOFF + (LD ? 512 : 0);
  static constexpr int NX = KCH, NF = FCH, NY = KCH;   // 1 KB loads per region
  static constexpr int NLOAD = NX + NF + NY;
};

// Chunk swizzle of the backward tiles, read both as rows (the score / dP A operands: the
// 16 lanes of a 128-bit pass read rows inv_perm_row(0..15) at one chunk) and transposed
// (64-bit transpose reads: a 32-lane pass reads four consecutive rows at four adjacent
// chunks).  It uses only row bits 1, 2 and 4, which makes both patterns conflict-free
// (distinct (row * cpr + position) mod 16 bank groups per pass) and keeps every read
// address a per-lane base plus an immediate: 8u and 32 rb change bits 3 and 5 only.
__host__ __device__ constexpr int swzb(int cpr, int r) {
  return cpr == 8 ? (4 * ((r >> 1) & 1) | 2 * ((r >> 2) & 1) | ((r >> 4) & 1))
       : cpr == 4 ? (2 * ((r >> 4) & 1) | ((r >> 2) & 1)) : 0;
}

// Byte offset of 16-bit element group (row, chunk c) in a region of cpr chunks per row.
__device__ __forceinline__ int toff(int cpr, int row, int c) { return row * cpr * 16 + 16 * (c ^ swzb(cpr, row)); }

// Per-lane read addresses of one region (cpr chunks per row):
//  row operand of k-step t (t < cpr / 2): row inv_perm_row(ln) (+ 32 rb), chunk 2 t + hf;
//  transposed operand of m-block mb, half q: lane 4 jj + a of 16-lane group g reads
//    columns 32 mb + 16 (g & 1) + 4 a .. + 3 of row 16 hf + 4 q + jj (+ 8 u + 32 rb); after
//    the two reads (q = 0, 1) lane (ln, hf) holds column 32 mb + ln of rows
//    32 rb + 16 hf + 8 u + 0..7 (k-slot j = row 16 hf + 8 u + j).
template <int CPR>
struct RegionAddr {
  static constexpr int NT = CPR / 2 > 0 ? CPR / 2 : 1, NM = CPR / 4 > 0 ? CPR / 4 : 1;
  int row[NT];
  int tr[2][NM];
  __device__ __forceinline__ void init(int lane) {
    const int ln = lane & 31, hf = lane >> 5;
    const int a = lane & 3, jj = (lane >> 2) & 3, gg = (lane >> 4) & 1;
    const int pr = inv_perm_row(ln);
#pragma unroll
    for (int t = 0; t < NT; ++t) row[t] = toff(CPR, pr, 2 * t + hf);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int mb = 0; mb < NM; ++mb) tr[q][mb] = toff(CPR, 16 * hf + 4 * q + jj, 4 * mb + 2 * gg + (a >> 1)) + 8 * (a & 1);
  }
  __device__ __forceinline__ u32x4 rowA(const unsigned char* reg, int rb, int t) const {
    return ld16(reg + row[t] + 32 * rb * CPR * 16);
  }
  __device__ __forceinline__ u32x4 trA(const unsigned char* reg, int rb, int u, int mb) const {
    const unsigned char* b = reg + (32 * rb + 8 * u) * CPR * 16;
    const s16x4 v[2] = {lds_read_tr16(b + tr[0][mb]), lds_read_tr16(b + tr[1][mb])};
    return __builtin_bit_cast(u32x4, v);
  }
};

// Eight fp32 values rounded (RNE) into one 16-byte B operand of type T.
template <typename T>
__device__ __forceinline__ u32x4 pack8(const float* x) {
  typedef T T8 __attribute__((ext_vector_type(8)));
  T8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (T)x[j];
  return __builtin_bit_cast(u32x4, r);
}

// Software pipelining of the backward blocks: the blocks are written as explicit
// instruction sequences (operand reads a fixed distance ahead of their MFMA, direct loads
// of a later tile one per MFMA), and a full scheduling fence after every step keeps the
// compiler from regrouping them.
constexpr int PD_ROW = 3;   // 128-bit operand reads in flight ahead of the score / dP MFMAs
constexpr int PD_TR = 2;    // gradient MFMAs whose transposed reads are in flight ahead
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup order: dispatch is round-robin over the 8 XCDs, so hardware id x runs on XCD
// x % 8; the logical id gives each XCD a contiguous range, which puts the blocks of one
// (b, h) on one XCD, where they share the streamed tiles in its L2.  Causal launches instead
// go longest-first over the whole grid, (b, h) fastest (each (b, h) stays on one XCD when
// B H is a multiple of 8).
__device__ __forceinline__ int xcd_order(int x, int G) {
  const int xcd = x & 7, idx = x >> 3, per = G >> 3, rem = G & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Direct global -> LDS loads of the backward tiles, written as inline asm: the compiler's
// own wait bookkeeping, which cannot tell the three tile buffers apart, would otherwise
// wait for every outstanding copy (vmcnt 0) and for every LDS read (lgkmcnt 0) before the
// next LDS read, serialising the prefetch.  Their completion is waited for explicitly
// (vmcnt) before the barrier that publishes a tile; the "memory" clobber keeps LDS
// accesses on their side of the asm.  lds: LDS byte address of lane 0's destination
// (the low half of a generic LDS pointer); lane l writes lds + 16 l (or 4 l).  The 16-byte
// form takes a scalar base and a 32-bit per-lane offset.  M0 carries
// the LDS address and is used by no compiler-generated instruction in these kernels.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ void dma16_async(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(off), "s"(base), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4_async(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(src), "s"(lds) : "memory");
}

// This wavefront's share of the direct loads of a tile: slot i copies load n = wave + BW i
// (regions X, F, Y in turn, 1 KB = 64 chunk slots each; every region is a multiple of BW
// loads, so slot i's region is a compile-time constant).  off[i] is the lane's source
// offset from the tile's first row (row * row stride + swizzled chunk; a factor chunk at
// or past R copies the row's first chunk).  Per tile, Bases holds each region's first-row
// address (scalar) and a clamp: rows past N read the last row's last chunk (finite
// stand-ins, masked by the caller), at the cost of one min per load.
// DV < D (head dim 16 in the D = 32 layout): chunks of regions X and Y at or past DV copy a
// chunk of the same row (finite stand-ins that meet zero register operands; the gradient
// columns they produce are not stored).
template <int D, int RP, bool LD, int DV = D>
struct DmaPlan {
  typedef Tile<D, RP, LD> T;
  static constexpr int VCH = DV / 8;   // chunks of a row that hold data (regions X, Y)
  static_assert(T::NX % BW == 0 && T::NF % BW == 0 && T::NY % BW == 0, "loads per region");
  static constexpr int NI = T::NLOAD / BW;
  static constexpr int region(int i) { return BW * i < T::NX ? 0 : BW * i < T::NX + T::NF ? 1 : 2; }
  static constexpr int first(int r) { return r == 0 ? 0 : r == 1 ? T::NX : T::NX + T::NF; }
  static constexpr int cpr(int r) { return r == 1 ? T::FCH : T::KCH; }
  static constexpr int doff(int r) { return r == 0 ? T::XOFF : r == 1 ? T::FOFF : T::YOFF; }
  uint32_t off[NI];
  const char* src[3];
  int stride2[3];                 // row strides in bytes
  int cmax[3];                    // last chunk a row may read
  struct Bases { const char* b[3]; uint32_t lim[3]; };
  __device__ __forceinline__ void init(int wave, int lane, const char* xb, int xs, const char* fb, int fs, int npch,
                                       const char* yb, int ys) {
    src[0] = xb; src[1] = fb; src[2] = yb;
    stride2[0] = 2 * xs; stride2[1] = 2 * fs; stride2[2] = 2 * ys;
    cmax[0] = VCH - 1; cmax[1] = npch - 1; cmax[2] = VCH - 1;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = region(i), c0 = cpr(r);
      const int nr = wave + BW * i - first(r);
      const int row = nr * (64 / c0) + lane / c0;
      int c = (lane % c0) ^ swzb(c0, row);
      if (r == 1 && c >= npch) c = 0;
      if (r != 1 && c >= VCH) c %= VCH;
      off[i] = (uint32_t)(row * stride2[r] + c * 16);
    }
  }
  // clamp row: the last row if it lies in the tile, else one past the tile's rows (no row
  // reaches it), so the 32-bit offsets stay within a tile
  __device__ __forceinline__ Bases bases(int r0, int N) const {
    Bases t;
    const int last = min(N - 1 - r0, TR - 1);
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      t.b[r] = src[r] + (int64_t)r0 * stride2[r];
      t.lim[r] = (uint32_t)(last * stride2[r] + cmax[r] * 16);
    }
    return t;
  }
  // slot i (a compile-time constant after unrolling) into the tile buffer dst
  __device__ __forceinline__ void issue(int i, const Bases& t, unsigned char* dst, int wave) const {
    const int r = region(i);
    const int nr = wave + BW * i - first(r);
    dma16_async(t.b[r], min(off[i], t.lim[r]), lds_addr(dst) + doff(r) + nr * 1024);
  }
};

// Wait until at most N direct loads of this wavefront are outstanding, then the workgroup
// barrier (the compiler barrier keeps LDS reads on their side of it).
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  static_assert(N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(N | 0x0F70);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------------
// dK, dV (and dphi_k): one workgroup per 128 keys of one (b, h).
// Two workgroups per compute unit up to D = 64; at D = 128 one (its B operands and
// accumulators take up to 256 VGPRs per wavefront).
// DV: head dims that hold data (DV = 16 runs in the D = 32 layout; see DmaPlan).  LOG2: phi_q
// in exp2 units (phi_q log2(e), as fb_attn_fwd_lowrank_log2 takes it): the scores are formed
// in exp2 units (K s log2(e) here, Q s log2(e) in the dQ kernel, L log2(e)), dS stays in
// natural units, and the factor gradients are those of the given factors (ln 2 dS phi).
template <typename QT, typename PT, int D, int RP, bool CAUSAL, int DV = D, bool LOG2 = false>
__global__ __launch_bounds__(BTH, D > 64 ? 1 : 2) void attn_bwd_dkv_kernel(BwdParams p) {
  typedef Tile<D, RP, true> T;
  constexpr int QST = D / 16, PST = RP / 16;
  constexpr int MBQ = D / 32, MBP = (RP + 31) / 32;
  static_assert(D % 32 == 0, "head dim multiple of 32");
  __shared__ __attribute__((aligned(16))) unsigned char s0[T::BYTES];   // three tile buffers
  __shared__ __attribute__((aligned(16))) unsigned char s1[T::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s2[T::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = xcd_order((int)blockIdx.x, (int)gridDim.x);
  int blk = L % p.nblk, bh = L / p.nblk;
  if (CAUSAL) {   // longest first over the grid: the first key blocks see the most query tiles
    const int BH = p.B * p.H;
    blk = (int)blockIdx.x / BH;
    bh = (int)blockIdx.x % BH;
  }
  const int hh = bh % p.H, bb = bh / p.H, N = p.N;
  const int kw0 = blk * kBwdRows + wave * 32;          // this wavefront's first key
  RegionAddr<T::KCH> ax, ay;
  RegionAddr<(T::FCH > 0 ? T::FCH : 4)> af;
  ax.init(lane);
  ay.init(lane);
  af.init(lane);
  const int key = kw0 + ln;
  const int keyc = min(key, N - 1);

  const QT* Qp = (const QT*)p.q + ((int64_t)bb * p.sq[0] + (int64_t)hh * p.sq[1]);
  const QT* Kp = (const QT*)p.k + ((int64_t)bb * p.sk[0] + (int64_t)hh * p.sk[1]);
  const QT* Vp = (const QT*)p.v + ((int64_t)bb * p.sv[0] + (int64_t)hh * p.sv[1]);
  const QT* Op = (const QT*)p.dout + ((int64_t)bb * p.sdo[0] + (int64_t)hh * p.sdo[1]);
  const float* Lp = p.lse + (int64_t)bh * N;
  const float* Dp = p.delta + (int64_t)bh * N;
  const PT* PQp = nullptr;
  const PT* PKp = nullptr;
  if constexpr (RP > 0) {
    PQp = (const PT*)p.phq + ((int64_t)bb * p.spq[0] + (int64_t)hh * p.spq[1]);
    PKp = (const PT*)p.phk + ((int64_t)bb * p.spk[0] + (int64_t)hh * p.spk[1]);
  }
  const int npch = RP > 0 ? p.R / 8 : 0;   // direct-load path needs R % 8 == 0 (host checks)

  // B operands of this wavefront's keys, negated: -K*s (scores; the tile holds Q unscaled,
  // so the scale goes to K here: identical products to the forward's (Q*s) K when s is a
  // power of two, one rounding apart otherwise), -phi_k (factor chain), -V (dP).  With the
  // chains started at L and Delta they end as L - S and Delta - dP: P = exp(-(L - S)) and
  // the block computes -dS = P (Delta - dP); the sign goes back at the dK / dphi_k stores.
  u32x4 kf[QST], vf[QST], pkf[PST > 0 ? PST : 1];
  const u32x4 sgn = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
#pragma unroll
  for (int t = 0; t < QST; ++t) {
    // head dims at or past DV: zero operands (their loads read the row's first chunk)
    const bool ok = 16 * t + 8 * hf < DV;
    const int c = ok ? 16 * t + 8 * hf : 0;
    const u32x4 z = {0u, 0u, 0u, 0u};
    kf[t] = ok ? scale_frag<QT>(ld16(Kp + keyc * p.sk[2] + c), LOG2 ? -p.scale * LOG2E : -p.scale) : z;
    vf[t] = (ok ? ld16(Vp + keyc * p.sv[2] + c) : z) ^ sgn;
  }
  if constexpr (RP > 0) {
#pragma unroll
    for (int t = 0; t < PST; ++t)
      pkf[t] = load_phi_chunk<PT>(PKp + keyc * p.spk[2], 16 * t + 8 * hf, p.R,
                                  (p.flags & FLAG_PHK_VEC) && 16 * t + 8 * hf + 8 <= p.R) ^ sgn;
  }

  f32x16 dvT[MBQ], dkT[MBQ + MBP];
#pragma unroll
  for (int i = 0; i < MBQ; ++i) dvT[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < MBQ + MBP; ++i) dkT[i] = f32x16{};

  const int nqt = (N + TR - 1) / TR;
  const int qt0 = CAUSAL ? (blk * kBwdRows) / TR : 0;   // earlier query tiles see none of these keys
  // Three tile buffers: tile qt + 2 streams in while tile qt is computed.  Every wavefront
  // issues the same number of loads per tile (NV: its chunk slots and one 4-byte copy of
  // the tile's L (even wavefronts) or Delta (odd) into the tile), so "at most NV
  // outstanding" means the next tile has landed.
  DmaPlan<D, RP, true, DV> plan;
  plan.init(wave, lane, (const char*)Qp, p.sq[2], (const char*)PQp, p.spq[2], npch, (const char*)Op, p.sdo[2]);
  constexpr int NI = DmaPlan<D, RP, true, DV>::NI, NV = NI + 1, NI0 = (NI + 1) / 2;
  const float* LDp = (wave & 1) ? Dp : Lp;
  // direct load j of a tile's NV: chunk slots, then the L / Delta copy
  // direct load j of a tile's NV: chunk slots, then the L / Delta copy
  auto issue_one = [&](int j, const typename DmaPlan<D, RP, true, DV>::Bases& tb, unsigned char* dst, int r0)
      __attribute__((always_inline)) {
    if (j < NI) plan.issue(j, tb, dst, wave);
    else dma4_async(LDp + r0 + min(lane, N - 1 - r0), lds_addr(dst + T::LOFF + 256 * (wave & 1)));
  };

  constexpr int NS = 2 * QST + PST;     // score / dP MFMAs per block: S (X), dP (Y) alternating, then S (F)
  constexpr int NCU = 2 * MBQ + MBP;    // gradient MFMAs per k-step u: dV^T, dK^T, dphi_k^T
  constexpr int NC = 2 * NCU;
  constexpr int NVB = (NV + 1) / 2;     // direct loads in the first block of a tile
  static_assert(NVB <= NS && NV - NVB <= NS, "direct loads per block");
  auto opS = [&](const unsigned char* tl, int qb, int k) __attribute__((always_inline)) {
    if (k < 2 * QST) return (k & 1) ? ay.rowA(tl + T::YOFF, qb, k >> 1) : ax.rowA(tl + T::XOFF, qb, k >> 1);
    return af.rowA(tl + T::FOFF, qb, k - 2 * QST);
  };
  auto opG = [&](const unsigned char* tl, int qb, int c) __attribute__((always_inline)) {
    const int u = c / NCU, j = c % NCU;
    if (j < MBQ) return ay.trA(tl + T::YOFF, qb, u, j);
    if (j < 2 * MBQ) return ax.trA(tl + T::XOFF, qb, u, j - MBQ);
    return af.trA(tl + T::FOFF, qb, u, j - 2 * MBQ);
  };

  // One code path for every block (a second, masked copy of the block costs registers):
  // blocks with a query past N or (causal) a query before one of the keys take a uniform
  // branch to the mask; fully masked blocks are computed and contribute zeros.
  auto compute = [&](const unsigned char* tl, int qt, unsigned char* nb, int qn) __attribute__((always_inline)) {
    const int q0 = qt * TR;
    const auto tb = plan.bases(qn * TR, N);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qb0 = q0 + 32 * qb;
      // register i holds query qb0 + 16 hf + i; the chains start at L and Delta
      const f32x4* lq = (const f32x4*)(tl + T::LOFF + 4 * (32 * qb + 16 * hf));
      const f32x4* dq = (const f32x4*)(tl + T::LOFF + 256 + 4 * (32 * qb + 16 * hf));
      f32x16 s, dp;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 L4 = lq[g], D4 = dq[g];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s[4 * g + c] = LOG2 ? L4[c] * LOG2E : L4[c];
          dp[4 * g + c] = D4[c];
        }
      }
      u32x4 a[NS];
#pragma unroll
      for (int k = 0; k < PD_ROW && k < NS; ++k) a[k] = opS(tl, qb, k);
      fence();
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if (k < 2 * QST) {
          if (k & 1) dp = Mma<QT>::run(a[k], vf[k >> 1], dp);
          else s = Mma<QT>::run(a[k], kf[k >> 1], s);
        } else {
          s = Mma<PT>::run(a[k], pkf[k - 2 * QST], s);
        }
        if (k + PD_ROW < NS) a[k + PD_ROW] = opS(tl, qb, k + PD_ROW);
        if (qb == 0 && k < NVB) issue_one(k, tb, nb, qn * TR);
        if (qb == 1 && k < NV - NVB) issue_one(NVB + k, tb, nb, qn * TR);
        fence();
      }
      u32x4 g[NC];
#pragma unroll
      for (int c = 0; c < PD_TR; ++c) g[c] = opG(tl, qb, c);
      fence();
      if (qb0 + 32 > N || (CAUSAL && qb0 < kw0 + 31)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = qb0 + 16 * hf + i;
          s[i] = qi < N && (!CAUSAL || qi >= key) ? s[i] : INFINITY;
        }
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(LOG2 ? -s[i] : s[i] * -LOG2E);
        dsv[i] = pv[i] * dp[i];
      }
      u32x4 pb[2], dsb[2], dsp[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pb[u] = pack8<QT>(pv + 8 * u);
        dsb[u] = pack8<QT>(dsv + 8 * u);
        if constexpr (RP > 0) dsp[u] = pack8<PT>(dsv + 8 * u);
      }
      fence();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int u = c / NCU, j = c % NCU;
        if (j < MBQ) dvT[j] = Mma<QT>::run(g[c], pb[u], dvT[j]);
        else if (j < 2 * MBQ) dkT[j - MBQ] = Mma<QT>::run(g[c], dsb[u], dkT[j - MBQ]);
        else dkT[j - MBQ] = Mma<PT>::run(g[c], dsp[u], dkT[j - MBQ]);
        if (c + PD_TR < NC) g[c + PD_TR] = opG(tl, qb, c + PD_TR);
        fence();
      }
    }
  };
  auto run = [&](const unsigned char* tl, int qt, unsigned char* nb) __attribute__((always_inline)) {
    compute(tl, qt, nb, min(qt + 2, nqt - 1));   // past the end: a copy nothing reads
  };

  if (qt0 < nqt) {
#pragma unroll
    for (int j = 0; j < NV; ++j) issue_one(j, plan.bases(qt0 * TR, N), s0, qt0 * TR);
#pragma unroll
    for (int j = 0; j < NV; ++j) issue_one(j, plan.bases(min(qt0 + 1, nqt - 1) * TR, N), s1, min(qt0 + 1, nqt - 1) * TR);
    wait_loads_barrier<NV>();
    // tile qt + 2 goes to the buffer of tile qt - 1
    for (int qt = qt0; qt < nqt; qt += 3) {
      run(s0, qt, s2);
      wait_loads_barrier<NV>();
      if (qt + 1 < nqt) {
        run(s1, qt + 1, s0);
        wait_loads_barrier<NV>();
      }
      if (qt + 2 < nqt) {
        run(s2, qt + 2, s1);
        wait_loads_barrier<NV>();
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // no copy outlives the workgroup
  }

  // register i of block mb: column 32 mb + 8 (i / 4) + 4 hf + i % 4 of this lane's key
  if (key < N) {
    QT* dVp = (QT*)p.dv + ((int64_t)bb * p.sdv[0] + (int64_t)hh * p.sdv[1] + (int64_t)key * p.sdv[2]);
    QT* dKp = (QT*)p.dk + ((int64_t)bb * p.sdk[0] + (int64_t)hh * p.sdk[1] + (int64_t)key * p.sdk[2]);
    typedef QT T4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int mb = 0; mb < MBQ; ++mb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        T4 v4, k4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v4[c] = (QT)dvT[mb][4 * a + c];
          k4[c] = (QT)(dkT[mb][4 * a + c] * -p.scale);   // dK = dS^T (Q s); dkT holds -dS^T Q
        }
        const int col = 32 * mb + 8 * a + 4 * hf;
        if (col < DV) {
          *(u32x2*)(dVp + col) = __builtin_bit_cast(u32x2, v4);
          *(u32x2*)(dKp + col) = __builtin_bit_cast(u32x2, k4);
        }
      }
    if constexpr (RP > 0) {   // this (b, h)'s dphi_k row (its partial when summed): 4 columns a store
      float* g = p.dphk + ((int64_t)bb * p.sdpk[0] + (int64_t)hh * p.sdpk[1] + (int64_t)key * p.sdpk[2]);
#pragma unroll
      for (int mb = 0; mb < MBP; ++mb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int col = 32 * mb + 8 * a + 4 * hf;
          const float f = LOG2 ? -LN2 : -1.f;   // dphi_k = dS^T phi_q (ln 2 dS^T phi_q with LOG2)
          const f32x4 v = {f * dkT[MBQ + mb][4 * a], f * dkT[MBQ + mb][4 * a + 1], f * dkT[MBQ + mb][4 * a + 2],
                           f * dkT[MBQ + mb][4 * a + 3]};
          if (col < p.R) *(f32x4*)(g + col) = v;
        }
    }
  }
}

// ---------------------------------------------------------------------------------
// dQ (and dphi_q): one workgroup per 128 queries of one (b, h).
template <typename QT, typename PT, int D, int RP, bool CAUSAL, int DV = D, bool LOG2 = false>
__global__ __launch_bounds__(BTH, D > 64 ? 1 : 2) void attn_bwd_dq_kernel(BwdParams p) {
  typedef Tile<D, RP, false> T;
  constexpr int QST = D / 16, PST = RP / 16;
  constexpr int MBQ = D / 32, MBP = (RP + 31) / 32;
  __shared__ __attribute__((aligned(16))) unsigned char s0[T::BYTES];   // three tile buffers
  __shared__ __attribute__((aligned(16))) unsigned char s1[T::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s2[T::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = xcd_order((int)blockIdx.x, (int)gridDim.x);
  int blk = L % p.nblk, bh = L / p.nblk;
  if (CAUSAL) {   // longest first over the grid: the last query blocks see the most key tiles
    const int BH = p.B * p.H;
    blk = p.nblk - 1 - (int)blockIdx.x / BH;
    bh = (int)blockIdx.x % BH;
  }
  const int hh = bh % p.H, bb = bh / p.H, N = p.N;
  const int qw0 = blk * kBwdRows + wave * 32;
  const int qrow = qw0 + ln;
  RegionAddr<T::KCH> ax, ay;
  RegionAddr<(T::FCH > 0 ? T::FCH : 4)> af;
  ax.init(lane);
  ay.init(lane);
  af.init(lane);
  const int qc = min(qrow, N - 1);

  const QT* Qp = (const QT*)p.q + ((int64_t)bb * p.sq[0] + (int64_t)hh * p.sq[1]);
  const QT* Kp = (const QT*)p.k + ((int64_t)bb * p.sk[0] + (int64_t)hh * p.sk[1]);
  const QT* Vp = (const QT*)p.v + ((int64_t)bb * p.sv[0] + (int64_t)hh * p.sv[1]);
  const QT* Op = (const QT*)p.dout + ((int64_t)bb * p.sdo[0] + (int64_t)hh * p.sdo[1]);
  const PT* PQp = nullptr;
  const PT* PKp = nullptr;
  if constexpr (RP > 0) {
    PQp = (const PT*)p.phq + ((int64_t)bb * p.spq[0] + (int64_t)hh * p.spq[1]);
    PKp = (const PT*)p.phk + ((int64_t)bb * p.spk[0] + (int64_t)hh * p.spk[1]);
  }
  const int npch = RP > 0 ? p.R / 8 : 0;

  // B operands of this wavefront's queries: Q*s (rounded once, as the forward), phi_q, dO
  u32x4 qf[QST], of[QST], pqf[PST > 0 ? PST : 1];
#pragma unroll
  for (int t = 0; t < QST; ++t) {
    const bool ok = 16 * t + 8 * hf < DV;   // head dims at or past DV: zero operands
    const int c = ok ? 16 * t + 8 * hf : 0;
    const u32x4 z = {0u, 0u, 0u, 0u};
    qf[t] = ok ? scale_frag<QT>(ld16(Qp + qc * p.sq[2] + c), LOG2 ? p.scale * LOG2E : p.scale) : z;
    of[t] = ok ? ld16(Op + qc * p.sdo[2] + c) : z;
  }
  if constexpr (RP > 0) {
#pragma unroll
    for (int t = 0; t < PST; ++t)
      pqf[t] = load_phi_chunk<PT>(PQp + qc * p.spq[2], 16 * t + 8 * hf, p.R,
                                  (p.flags & FLAG_PHQ_VEC) && 16 * t + 8 * hf + 8 <= p.R);
  }
  // L (in exp2 units) and Delta of this lane's query
  const float L2q = p.lse[(int64_t)bh * N + qc] * LOG2E;
  const float Dq = p.delta[(int64_t)bh * N + qc];

  f32x16 dqT[MBQ + MBP];
#pragma unroll
  for (int i = 0; i < MBQ + MBP; ++i) dqT[i] = f32x16{};

  const int kend = CAUSAL ? min(N, blk * kBwdRows + kBwdRows) : N;
  const int nkt = (kend + TR - 1) / TR;
  // three tile buffers: tile kt + 2 streams in while tile kt is computed (NI loads per
  // wavefront and tile, so "at most NI outstanding" means the next tile has landed)
  DmaPlan<D, RP, false, DV> plan;
  plan.init(wave, lane, (const char*)Kp, p.sk[2], (const char*)PKp, p.spk[2], npch, (const char*)Vp, p.sv[2]);
  constexpr int NI = DmaPlan<D, RP, false, DV>::NI;

  constexpr int NS = 2 * QST + PST;   // S^T (X) and dP^T (Y) alternating, then S^T (F)
  constexpr int NCU = MBQ + MBP;      // gradient MFMAs per k-step u: dQ^T, dphi_q^T
  constexpr int NC = 2 * NCU;
  constexpr int NVB = (NI + 1) / 2;
  static_assert(NVB <= NS, "direct loads per block");
  auto opS = [&](const unsigned char* tl, int kb, int k) __attribute__((always_inline)) {
    if (k < 2 * QST) return (k & 1) ? ay.rowA(tl + T::YOFF, kb, k >> 1) : ax.rowA(tl + T::XOFF, kb, k >> 1);
    return af.rowA(tl + T::FOFF, kb, k - 2 * QST);
  };
  auto opG = [&](const unsigned char* tl, int kb, int c) __attribute__((always_inline)) {
    const int u = c / NCU, j = c % NCU;
    if (j < MBQ) return ax.trA(tl + T::XOFF, kb, u, j);
    return af.trA(tl + T::FOFF, kb, u, j - MBQ);
  };

  // one code path for every block: blocks with a key past N or (causal) a key after one of
  // the queries take a uniform branch to the mask; fully masked blocks contribute zeros
  auto compute = [&](const unsigned char* tl, int kt, unsigned char* nb, int kn) __attribute__((always_inline)) {
    const int k0 = kt * TR;
    const auto tb = plan.bases(kn * TR, N);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kb0 = k0 + 32 * kb;
      f32x16 s = f32x16{}, dp = f32x16{};
      u32x4 a[NS];
#pragma unroll
      for (int k = 0; k < PD_ROW && k < NS; ++k) a[k] = opS(tl, kb, k);
      fence();
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if (k < 2 * QST) {
          if (k & 1) dp = Mma<QT>::run(a[k], of[k >> 1], dp);
          else s = Mma<QT>::run(a[k], qf[k >> 1], s);
        } else {
          s = Mma<PT>::run(a[k], pqf[k - 2 * QST], s);
        }
        if (k + PD_ROW < NS) a[k + PD_ROW] = opS(tl, kb, k + PD_ROW);
        if (kb == 0 && k < NVB) plan.issue(k, tb, nb, wave);
        if (kb == 1 && k < NI - NVB) plan.issue(NVB + k, tb, nb, wave);
        fence();
      }
      u32x4 g[NC];
#pragma unroll
      for (int c = 0; c < PD_TR; ++c) g[c] = opG(tl, kb, c);
      fence();
      // register i holds key kb0 + 16 hf + i
      if (kb0 + 32 > N || (CAUSAL && kb0 + 31 > qw0)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kj = kb0 + 16 * hf + i;
          s[i] = kj < N && (!CAUSAL || kj <= qrow) ? s[i] : -INFINITY;
        }
      }
      float dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        dsv[i] = __builtin_amdgcn_exp2f(LOG2 ? s[i] - L2q : __builtin_fmaf(s[i], LOG2E, -L2q)) * (dp[i] - Dq);
      u32x4 dsb[2], dsp[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        dsb[u] = pack8<QT>(dsv + 8 * u);
        if constexpr (RP > 0) dsp[u] = pack8<PT>(dsv + 8 * u);
      }
      fence();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int u = c / NCU, j = c % NCU;
        if (j < MBQ) dqT[j] = Mma<QT>::run(g[c], dsb[u], dqT[j]);
        else dqT[j] = Mma<PT>::run(g[c], dsp[u], dqT[j]);
        if (c + PD_TR < NC) g[c + PD_TR] = opG(tl, kb, c + PD_TR);
        fence();
      }
    }
  };
  auto run = [&](const unsigned char* tl, int kt, unsigned char* nb) __attribute__((always_inline)) {
    compute(tl, kt, nb, min(kt + 2, nkt - 1));   // past the end: a copy nothing reads
  };

  if (nkt > 0) {
#pragma unroll
    for (int j = 0; j < NI; ++j) plan.issue(j, plan.bases(0, N), s0, wave);
#pragma unroll
    for (int j = 0; j < NI; ++j) plan.issue(j, plan.bases(min(1, nkt - 1) * TR, N), s1, wave);
    wait_loads_barrier<NI>();
    for (int kt = 0; kt < nkt; kt += 3) {
      run(s0, kt, s2);
      wait_loads_barrier<NI>();
      if (kt + 1 < nkt) {
        run(s1, kt + 1, s0);
        wait_loads_barrier<NI>();
      }
      if (kt + 2 < nkt) {
        run(s2, kt + 2, s1);
        wait_loads_barrier<NI>();
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // no copy outlives the workgroup
  }

  if (qrow < N) {
    QT* dQp = (QT*)p.dq + ((int64_t)bb * p.sdq[0] + (int64_t)hh * p.sdq[1] + (int64_t)qrow * p.sdq[2]);
    typedef QT T4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int mb = 0; mb < MBQ; ++mb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        T4 q4;
#pragma unroll
        for (int c = 0; c < 4; ++c) q4[c] = (QT)(dqT[mb][4 * a + c] * p.scale);
        if (32 * mb + 8 * a + 4 * hf < DV) *(u32x2*)(dQp + 32 * mb + 8 * a + 4 * hf) = __builtin_bit_cast(u32x2, q4);
      }
    if constexpr (RP > 0) {   // this (b, h)'s dphi_q row (its partial when summed): 4 columns a store
      float* g = p.dphq + ((int64_t)bb * p.sdpq[0] + (int64_t)hh * p.sdpq[1] + (int64_t)qrow * p.sdpq[2]);
#pragma unroll
      for (int mb = 0; mb < MBP; ++mb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int col = 32 * mb + 8 * a + 4 * hf;
          const float f = LOG2 ? LN2 : 1.f;   // dphi_q = dS phi_k (ln 2 dS phi_k with LOG2)
          const f32x4 v = {f * dqT[MBQ + mb][4 * a], f * dqT[MBQ + mb][4 * a + 1], f * dqT[MBQ + mb][4 * a + 2],
                           f * dqT[MBQ + mb][4 * a + 3]};
          if (col < p.R) *(f32x4*)(g + col) = v;
        }
    }
  }
}

}  // namespace attnb
}  // namespace fb
