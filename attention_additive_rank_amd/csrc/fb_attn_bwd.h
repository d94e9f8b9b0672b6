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
// global->LDS loads (1 KB of consecutive rows per load) one tile ahead, double-buffered.
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

// Issue the direct loads of one tile (rows r0 .. r0 + 63 of the three sources) into dst.
// Load n of the tile: regions X, F, Y in turn (1 KB = 64 chunk slots each).  Wavefront w
// issues loads w, w + 4, ...  A chunk that is not wanted (a row past N, a factor column at
// or beyond R) copies a finite stand-in: the last row, or the row's first chunk.
template <int D, int RP, bool LD>
__device__ __forceinline__ void load_tile(unsigned char* dst, int r0, int N, int wave, int lane, const char* xb,
                                          int xs, const char* fb, int fs, int npch, const char* yb, int ys) {
  typedef Tile<D, RP, LD> T;
#pragma unroll
  for (int i = 0; i < (T::NLOAD + BW - 1) / BW; ++i) {
    const int n = wave + BW * i;
    if (n < T::NLOAD) {
      {
        int region, nr, cpr;
        if (n < T::NX) { region = 0; nr = n; cpr = T::KCH; }
        else if (n < T::NX + T::NF) { region = 1; nr = n - T::NX; cpr = T::FCH; }
        else { region = 2; nr = n - T::NX - T::NF; cpr = T::KCH; }
        const int row = nr * (64 / cpr) + lane / cpr;
        int c = (lane % cpr) ^ swzb(cpr, row);
        const int srow = min(r0 + row, N - 1) - r0;
        if (region == 1 && c >= npch) c = 0;
        const char* base = region == 0 ? xb : region == 1 ? fb : yb;
        const int stride = region == 0 ? xs : region == 1 ? fs : ys;
        const int off = region == 0 ? T::XOFF : region == 1 ? T::FOFF : T::YOFF;
        dma16(base + (int64_t)(r0 + srow) * stride * 2 + c * 16, dst + off + nr * 1024);
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// dK, dV (and dphi_k): one workgroup per 128 keys of one (b, h).
template <typename QT, typename PT, int D, int RP, bool CAUSAL>
__global__ __launch_bounds__(BTH, 2) void attn_bwd_dkv_kernel(BwdParams p) {
  typedef Tile<D, RP, true> T;
  constexpr int QST = D / 16, PST = RP / 16;
  constexpr int MBQ = D / 32, MBP = (RP + 31) / 32;
  static_assert(D % 32 == 0, "head dim multiple of 32");
  __shared__ __attribute__((aligned(16))) unsigned char sA[T::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sB[T::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = blockIdx.x % p.nblk;
  const int bh = blockIdx.x / p.nblk;
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

  // B operands of this wavefront's keys: K*s (scores; the tile holds Q unscaled, so the
  // scale goes to K here: identical products to the forward's (Q*s) K when s is a power of
  // two, one rounding apart otherwise), phi_k (factor chain), V (dP)
  u32x4 kf[QST], vf[QST], pkf[PST > 0 ? PST : 1];
#pragma unroll
  for (int t = 0; t < QST; ++t) {
    kf[t] = scale_frag<QT>(ld16(Kp + keyc * p.sk[2] + 16 * t + 8 * hf), p.scale);
    vf[t] = ld16(Vp + keyc * p.sv[2] + 16 * t + 8 * hf);
  }
  if constexpr (RP > 0) {
#pragma unroll
    for (int t = 0; t < PST; ++t)
      pkf[t] = load_phi_chunk<PT>(PKp + keyc * p.spk[2], 16 * t + 8 * hf, p.R,
                                  (p.flags & FLAG_PHK_VEC) && 16 * t + 8 * hf + 8 <= p.R);
  }

  f32x16 dvT[MBQ], dkT[MBQ + MBP];
#pragma unroll
  for (int i = 0; i < MBQ; ++i) dvT[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < MBQ + MBP; ++i) dkT[i] = f32x16{};

  const int nqt = (N + TR - 1) / TR;
  const int qt0 = CAUSAL ? (blk * kBwdRows) / TR : 0;   // earlier query tiles see none of these keys
  // L and Delta of a query tile: threads 0..63 / 64..127 load one value each when the tile's
  // copies are issued and store it into the tile before the barrier that publishes it
  float lval = 0.f;
  auto issue = [&](unsigned char* dst, int qt) __attribute__((always_inline)) {
    const int r0 = qt * TR;
    load_tile<D, RP, true>(dst, r0, N, wave, lane, (const char*)Qp, p.sq[2], (const char*)PQp, p.spq[2], npch,
                           (const char*)Op, p.sdo[2]);
    if (tid < 128) lval = (tid < 64 ? Lp : Dp)[min(r0 + (tid & 63), N - 1)];
  };
  auto publish = [&](unsigned char* dst) __attribute__((always_inline)) {
    if (tid < 128) ((float*)(dst + T::LOFF))[tid] = lval;
  };

  auto compute = [&](const unsigned char* tl, int qt) __attribute__((always_inline)) {
    const int q0 = qt * TR;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qb0 = q0 + 32 * qb;
      if (CAUSAL && qb0 + 31 < kw0) continue;        // every query of the block precedes every key
      if (qb0 >= N) continue;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < QST; ++t) s = Mma<QT>::run(ax.rowA(tl + T::XOFF, qb, t), kf[t], s);
      if constexpr (RP > 0) {
#pragma unroll
        for (int t = 0; t < PST; ++t) s = Mma<PT>::run(af.rowA(tl + T::FOFF, qb, t), pkf[t], s);
      }
#pragma unroll
      for (int t = 0; t < QST; ++t) dp = Mma<QT>::run(ay.rowA(tl + T::YOFF, qb, t), vf[t], dp);
      // register i holds query qb0 + 16 hf + i
      const f32x4* lq = (const f32x4*)(tl + T::LOFF + 4 * (32 * qb + 16 * hf));
      const f32x4* dq = (const f32x4*)(tl + T::LOFF + 256 + 4 * (32 * qb + 16 * hf));
      float pv[16], dsv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 L4 = lq[g], D4 = dq[g];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 4 * g + c;
          const int qi = qb0 + 16 * hf + i;
          const bool ok = qi < N && (!CAUSAL || qi >= key);
          const float e = __builtin_amdgcn_exp2f((s[i] - L4[c]) * LOG2E);
          pv[i] = ok ? e : 0.f;
          dsv[i] = pv[i] * (dp[i] - D4[c]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 pb = pack8<QT>(pv + 8 * u);
        const u32x4 dsb = pack8<QT>(dsv + 8 * u);
#pragma unroll
        for (int mb = 0; mb < MBQ; ++mb) dvT[mb] = Mma<QT>::run(ay.trA(tl + T::YOFF, qb, u, mb), pb, dvT[mb]);
#pragma unroll
        for (int mb = 0; mb < MBQ; ++mb) dkT[mb] = Mma<QT>::run(ax.trA(tl + T::XOFF, qb, u, mb), dsb, dkT[mb]);
        if constexpr (RP > 0) {
          const u32x4 dsp = pack8<PT>(dsv + 8 * u);
#pragma unroll
          for (int mb = 0; mb < MBP; ++mb)
            dkT[MBQ + mb] = Mma<PT>::run(af.trA(tl + T::FOFF, qb, u, mb), dsp, dkT[MBQ + mb]);
        }
      }
    }
  };

  if (qt0 < nqt) {
    issue(sA, qt0);
    publish(sA);
    __syncthreads();
  }
  for (int qt = qt0; qt < nqt; qt += 2) {
    if (qt + 1 < nqt) issue(sB, qt + 1);
    compute(sA, qt);
    if (qt + 1 < nqt) publish(sB);
    __syncthreads();
    if (qt + 1 < nqt) {
      if (qt + 2 < nqt) issue(sA, qt + 2);
      compute(sB, qt + 1);
      if (qt + 2 < nqt) publish(sA);
      __syncthreads();
    }
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
          k4[c] = (QT)(dkT[mb][4 * a + c] * p.scale);   // dK = dS^T (Q s)
        }
        const int col = 32 * mb + 8 * a + 4 * hf;
        *(u32x2*)(dVp + col) = __builtin_bit_cast(u32x2, v4);
        *(u32x2*)(dKp + col) = __builtin_bit_cast(u32x2, k4);
      }
    if constexpr (RP > 0) {
      float* g = p.dphk + ((int64_t)bb * p.sdpk[0] + (int64_t)hh * p.sdpk[1] + (int64_t)key * p.sdpk[2]);
#pragma unroll
      for (int mb = 0; mb < MBP; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int col = 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
          if (col < p.R) atomicAdd(g + col, dkT[MBQ + mb][i]);
        }
    }
  }
}

// ---------------------------------------------------------------------------------
// dQ (and dphi_q): one workgroup per 128 queries of one (b, h).
template <typename QT, typename PT, int D, int RP, bool CAUSAL>
__global__ __launch_bounds__(BTH, 2) void attn_bwd_dq_kernel(BwdParams p) {
  typedef Tile<D, RP, false> T;
  constexpr int QST = D / 16, PST = RP / 16;
  constexpr int MBQ = D / 32, MBP = (RP + 31) / 32;
  __shared__ __attribute__((aligned(16))) unsigned char sA[T::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sB[T::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = blockIdx.x % p.nblk;
  const int bh = blockIdx.x / p.nblk;
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
    qf[t] = scale_frag<QT>(ld16(Qp + qc * p.sq[2] + 16 * t + 8 * hf), p.scale);
    of[t] = ld16(Op + qc * p.sdo[2] + 16 * t + 8 * hf);
  }
  if constexpr (RP > 0) {
#pragma unroll
    for (int t = 0; t < PST; ++t)
      pqf[t] = load_phi_chunk<PT>(PQp + qc * p.spq[2], 16 * t + 8 * hf, p.R,
                                  (p.flags & FLAG_PHQ_VEC) && 16 * t + 8 * hf + 8 <= p.R);
  }
  const float Lq = p.lse[(int64_t)bh * N + qc];
  const float Dq = p.delta[(int64_t)bh * N + qc];

  f32x16 dqT[MBQ + MBP];
#pragma unroll
  for (int i = 0; i < MBQ + MBP; ++i) dqT[i] = f32x16{};

  const int kend = CAUSAL ? min(N, blk * kBwdRows + kBwdRows) : N;
  const int nkt = (kend + TR - 1) / TR;
  auto issue = [&](unsigned char* dst, int kt) __attribute__((always_inline)) {
    load_tile<D, RP, false>(dst, kt * TR, N, wave, lane, (const char*)Kp, p.sk[2], (const char*)PKp, p.spk[2], npch,
                            (const char*)Vp, p.sv[2]);
  };

  auto compute = [&](const unsigned char* tl, int kt) __attribute__((always_inline)) {
    const int k0 = kt * TR;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kb0 = k0 + 32 * kb;
      if (CAUSAL && kb0 > qw0 + 31) continue;        // every key of the block follows every query
      if (kb0 >= N) continue;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < QST; ++t) s = Mma<QT>::run(ax.rowA(tl + T::XOFF, kb, t), qf[t], s);
      if constexpr (RP > 0) {
#pragma unroll
        for (int t = 0; t < PST; ++t) s = Mma<PT>::run(af.rowA(tl + T::FOFF, kb, t), pqf[t], s);
      }
#pragma unroll
      for (int t = 0; t < QST; ++t) dp = Mma<QT>::run(ay.rowA(tl + T::YOFF, kb, t), of[t], dp);
      float dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = kb0 + 16 * hf + i;
        const bool ok = kj < N && (!CAUSAL || kj <= qrow);
        const float e = __builtin_amdgcn_exp2f((s[i] - Lq) * LOG2E);
        dsv[i] = ok ? e * (dp[i] - Dq) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 dsb = pack8<QT>(dsv + 8 * u);
#pragma unroll
        for (int mb = 0; mb < MBQ; ++mb) dqT[mb] = Mma<QT>::run(ax.trA(tl + T::XOFF, kb, u, mb), dsb, dqT[mb]);
        if constexpr (RP > 0) {
          const u32x4 dsp = pack8<PT>(dsv + 8 * u);
#pragma unroll
          for (int mb = 0; mb < MBP; ++mb)
            dqT[MBQ + mb] = Mma<PT>::run(af.trA(tl + T::FOFF, kb, u, mb), dsp, dqT[MBQ + mb]);
        }
      }
    }
  };

  if (nkt > 0) {
    issue(sA, 0);
    __syncthreads();
  }
  for (int kt = 0; kt < nkt; kt += 2) {
    if (kt + 1 < nkt) issue(sB, kt + 1);
    compute(sA, kt);
    __syncthreads();
    if (kt + 1 < nkt) {
      if (kt + 2 < nkt) issue(sA, kt + 2);
      compute(sB, kt + 1);
      __syncthreads();
    }
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
        *(u32x2*)(dQp + 32 * mb + 8 * a + 4 * hf) = __builtin_bit_cast(u32x2, q4);
      }
    if constexpr (RP > 0) {
      float* g = p.dphq + ((int64_t)bb * p.sdpq[0] + (int64_t)hh * p.sdpq[1] + (int64_t)qrow * p.sdpq[2]);
#pragma unroll
      for (int mb = 0; mb < MBP; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int col = 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
          if (col < p.R) atomicAdd(g + col, dqT[MBQ + mb][i]);
        }
    }
  }
}

}  // namespace attnb
}  // namespace fb
