// Fused low-rank forward for short sequences on gfx950: the whole K' = [K, phi_k] and V of
// one (batch, head) resident in LDS.
//
//   O = softmax(s Q K^T + phi_q phi_k^T) V,  scores in exp2 units (phi_q given times log2(e))
//
// The augmented contraction is the pages' (FlashBias rebuttal, answer to Reviewer UJUf, Q2:
// the factor functions concatenated to queries and keys); what differs from the streaming
// kernel in fb_attn_kernel.h is the schedule:
//   * One workgroup = 4 wavefronts (one per SIMD) = one (b, h).  It copies every 64-key tile
//     of K' and V into LDS once (direct global->LDS loads, the streaming kernel's tile layout
//     and slot map) and each wavefront runs its query blocks of 32 rows over all key tiles
//     with at most two barriers in all: one after the copies (after the first half of them
//     with four or more tiles) and, with four or more tiles, one in the first block pair's
//     key loop before the second half is read.  On short sequences the streaming kernel
//     spends much of each tile waiting at its barrier for the slowest of its wavefronts
//     (8 key tiles per item there, a barrier per tile).
//   * Two workgroups share a compute unit (at most 80 KB of LDS each): one's copies and
//     set-up run under the other's key loop.
//   * Each wavefront carries TWO query blocks, A and B, half a key step apart, so its matrix
//     and vector work interleave in one instruction stream: while the MFMAs of one block run
//     (O += V(t)^T P(t)^T, then the next tile's scores), the vector unit exponentiates the
//     other block's scores.  With one block per wavefront a wavefront alternates between a
//     matrix phase that waits on its LDS reads and a softmax phase that waits on its own
//     vector chain, and even four of them per SIMD left the matrix core and the vector unit
//     each less than half busy (counters); two blocks need twice the registers (up to 256
//     per lane, one wavefront per SIMD per workgroup).
//   * Per tile and block: S^T = K' Q'^T on 32x32x16 MFMAs (a factor chain in the factor dtype
//     into the same fp32 accumulator, every chain started from -M, M the running max in exp2
//     units), the online softmax with lazy rescaling (M moves only when a tile's max exceeds
//     it by 2^15), P^T rounded to the input dtype as the B operand of O^T = V^T P^T, and the
//     row sum of P as one 16x16x32 MFMA per P V k-step.  The softmax's max and rescale (a
//     uniform branch) run before the interleaved part; the exponentials, conversions and
//     MFMAs after it form one scheduling region.
// Only non-causal launches with D + RP <= 48 whose key tiles fit (res_max_keys) take this
// kernel: with wider Q' the state of two blocks spills out of 256 registers.
#pragma once

#include <type_traits>

#include "fb_attn_kernel.h"

namespace fb {
namespace attn {

// Lazy rescaling headroom in exp2 units: M moves only when a tile's max exceeds it by more than
// 15, so P <= 2^15 (an f16 P must stay below its 65504 limit).  P is rounded to bf16 / f16
// with the same relative precision at any magnitude and O, l accumulate in fp32, so the wide
// headroom costs no accuracy; it makes the rescale (about 50 vector operations for the
// wavefront) rare also for wide bias ranges, where a 2^8 headroom rescaled in about one key
// step in seven.
constexpr float RES_GROW = 15.f;
constexpr int RNW = 4;                  // wavefronts per workgroup
constexpr int RNT = RNW * 64;           // threads per workgroup
// LDS per workgroup and tiles that fit: kResLdsBytes, res_max_tiles (fb_tile_map.h)

template <typename QT, typename PT, int D, int RP>
__global__ __launch_bounds__(RNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_res_kernel(AttnParams p) {
  static_assert(sizeof(QT) == 2 && sizeof(PT) == 2, "16-bit operands");
  constexpr int KS = 16;                  // k per MFMA
  constexpr int CE = 8;                   // elements per 16-byte chunk
  constexpr int DP = D < 32 ? 32 : D;     // V width in LDS
  constexpr int DB = DP / 32;             // 32-wide head-dim blocks of the output
  constexpr int QSTEPS = D / KS;
  constexpr int PSTEPS = RP / KS;
  constexpr int KCH = D / CE, PCH = RP / CE, VCH = DP / CE;
  constexpr int KREG = BN * KCH * 16;
  constexpr int SKB = KREG + BN * PCH * 16;   // one K' tile
  constexpr int SVB = BN * VCH * 16;          // one V tile
  constexpr int NDMA = KCH + PCH + VCH;       // 1 KB loads per tile
  constexpr int TMAX = res_max_tiles(D, RP);
  static_assert(SKB + SVB == res_tile_bytes(D, RP), "tile bytes");
  static_assert(TMAX >= 1 && D % KS == 0 && RP % KS == 0, "bad tile widths");
  static_assert((KCH & (KCH - 1)) == 0 && (PCH & (PCH - 1)) == 0 && (VCH & (VCH - 1)) == 0 && VCH >= 4,
                "tile rows must be a power-of-two number of chunks");
  __shared__ __attribute__((aligned(16))) unsigned char sK[TMAX * SKB];
  __shared__ __attribute__((aligned(16))) unsigned char sV[TMAX * SVB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int bh = (int)blockIdx.x;
  const int hh = bh % p.H;
  const int bb = bh / p.H;
  const int N = p.N;
  const int nkt = (N + BN - 1) / BN;   // at most TMAX (the host checks)
  const int nrb = (N + 31) / 32;       // query blocks

  const QT* Qp = (const QT*)p.q + ((int64_t)bb * p.sq[0] + (int64_t)hh * p.sq[1]);
  const QT* Kp = (const QT*)p.k + ((int64_t)bb * p.sk[0] + (int64_t)hh * p.sk[1]);
  const QT* Vp = (const QT*)p.v + ((int64_t)bb * p.sv[0] + (int64_t)hh * p.sv[1]);
  QT* Op = (QT*)p.o + ((int64_t)bb * p.so[0] + (int64_t)hh * p.so[1]);
  const PT* PQp = nullptr;
  const PT* PKp = nullptr;
  if constexpr (RP > 0) {
    PQp = (const PT*)p.phq + ((int64_t)bb * p.spq[0] + (int64_t)hh * p.spq[1]);
    PKp = (const PT*)p.phk + ((int64_t)bb * p.spk[0] + (int64_t)hh * p.spk[1]);
  }

  // ---- every key tile into LDS ------------------------------------------------------
  // A tile takes NDMA loads of 1 KB, load n filling slots of the K region, then phi_k, then V
  // (tile_slot; lane l fills chunk slot l of the load's 1 KB).  Every slot is written: a row past N copies row N - 1 (its scores are masked, its P is 0), a chunk
  // without data an in-row stand-in (loader_src_byte: it meets zero phi_q columns or feeds
  // head dims >= D only), so everything the MFMAs read is finite.
  // With four or more tiles the copies go in two halves: tiles [0, th) before the first
  // barrier, tiles [th, nkt) right after it, waited for at a second barrier in the first
  // block pair's key loop before any read of tile th (the workgroups of a launch start
  // together, so their copies would otherwise all wait on HBM at once).
  const bool split = nkt >= 4;
  const int th = split ? (nkt + 1) / 2 : nkt;
  // This wavefront issues loads n = wave + RNW i (< NDMA) of every tile; their per-lane source
  // rows and bytes are fixed, only the tile's first row moves (and the clamp to row N - 1 in
  // the last tile).
  constexpr int LPW = (NDMA + RNW - 1) / RNW;
  int lrow[LPW], lbyte[LPW];
  {
    const int npch = RP > 0 ? p.R / CE : 0;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const TileSlot d = tile_slot(min(wave + RNW * i, NDMA - 1), lane, KCH, PCH, VCH);
      lrow[i] = d.row;
      lbyte[i] = loader_src_byte(d, KCH, npch);
    }
  }
  auto copy_tiles = [&](int t0, int t1) __attribute__((always_inline)) {
    for (int t = t0; t < t1; ++t) {
      const int kb = t * BN;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int n = wave + RNW * i;
        if (n < NDMA) {
          const int region = n < KCH ? 0 : n < KCH + PCH ? 1 : 2;
          const int stride = region == 0 ? p.sk[2] : region == 1 ? p.spk[2] : p.sv[2];
          const char* base = region == 0 ? (const char*)(Kp + (int64_t)kb * p.sk[2])
                           : region == 1 ? (const char*)(PKp + (int64_t)kb * p.spk[2])
                                         : (const char*)(Vp + (int64_t)kb * p.sv[2]);
          unsigned char* dst = region == 2 ? sV + t * SVB + (n - KCH - PCH) * 1024 : sK + t * SKB + n * 1024;
          const int row = kb + BN > N ? min(lrow[i], N - 1 - kb) : lrow[i];
          dma16(base + (row * stride * 2 + lbyte[i]), dst);
        }
      }
    }
  };
  copy_tiles(0, th);

  // ---- per-block state ------------------------------------------------------------
  struct Blk {
    f32x16 s[NKB];          // S^T of the tile being processed, minus M (exp2 units)
    u32x4 pr[NKB * 2];      // P^T, B operand of the P V product
    f32x16 o[DB];
    f32x4 l;                // row sum of P (matrix core), the lane's own row in every register
    float m;                // running max in exp2 units
    f32x16 mi;              // -m in every register: the score chains' starting accumulator
    u32x4 qf[QSTEPS];       // Q' fragments (B operand of S^T = K' Q'^T)
    u32x4 pf[PSTEPS > 0 ? PSTEPS : 1];
  };
  Blk A, B;

  // Q' fragments of query row qc: k-step t of lane half h covers chunk 2t + h: Q s log2(e)
  // rounded once, phi_q as given (already in exp2 units), zero past R
  const float qscale = p.scale * LOG2E;
  auto load_frags = [&](Blk& b, int qc) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) b.qf[t] = scale_frag<QT>(ld16(Qp + qc * p.sq[2] + KS * t + CE * hf), qscale);
    if constexpr (RP > 0) {
      const PT* prow = PQp + qc * p.spq[2];
#pragma unroll
      for (int t = 0; t < PSTEPS; ++t) {
        const int c0 = KS * t + CE * hf;
        b.pf[t] = load_phi_chunk<PT>(prow, c0, p.R, (p.flags & FLAG_PHQ_VEC) && c0 + CE <= p.R);
      }
    }
  };
  // this wavefront's block pairs: (a, a + RNW) for a = wave, wave + 2 RNW, ...; a second block
  // past the last one computes clamped rows and stores nothing
  auto row_of = [&](int rb) __attribute__((always_inline)) { return min(rb * 32 + ln, N - 1); };
  int a0 = wave;
  load_frags(A, row_of(a0));
  load_frags(B, row_of(a0 + RNW));
  __builtin_amdgcn_s_waitcnt(0);   // this wavefront's tile copies have landed
  __syncthreads();                 // ... and everyone else's
  copy_tiles(th, nkt);             // the second half, waited for at the split barrier
  bool split_pending = split;
  auto split_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    split_pending = false;
  };

  // ---- LDS operand addresses (tile-relative; the streaming kernel's maps) ------------
  // Score operand of k-step t, key block kb2: key row 32 kb2 + inv_perm_row(ln), logical
  // chunk 2t + hf; per lane four (eight) distinct addresses, the rest an immediate.
  auto kaddr = [&](int cpr, int j) __attribute__((always_inline)) {
    const int c = (2 * j + hf) & (cpr - 1);
    return inv_perm_row(ln) * cpr * 16 + 16 * (c ^ swz_key(cpr, inv_perm_row(ln)));
  };
  constexpr int KA = KCH >= 16 ? 8 : 4, PA = PCH >= 16 ? 8 : 4;
  int ka_k[KA], ka_p[PA];
#pragma unroll
  for (int j = 0; j < KA; ++j) ka_k[j] = kaddr(KCH, j);
#pragma unroll
  for (int j = 0; j < PA; ++j) ka_p[j] = KREG + (PCH > 0 ? kaddr(PCH, j) : 0);
  auto kread = [&](const unsigned char* sKt, bool phi, int t, int kb2) __attribute__((always_inline)) {
    const int cpr = phi ? PCH : KCH;
    const int na = phi ? PA : KA;
    const int* a = phi ? ka_p : ka_k;
    return ld16(sKt + a[t % na] + 32 * na * (t / na) + 32 * kb2 * cpr * 16);
  };
  // P V operand, key block kb2, k-step u, head-dim block db: two 64-bit transpose reads of
  // rows 32 kb2 + 16 hf + 8 u + 4 q + jj (q = 0, 1)
  const int tr_a = lane & 3, tr_jj = (lane >> 2) & 3, tr_gg = (lane >> 4) & 1;
  int va[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int r = 16 * hf + tr_jj;
    const int c = (4 * e + 2 * tr_gg + (tr_a >> 1)) & (VCH - 1);
    va[e] = r * VCH * 16 + 16 * (c ^ swz_quad(VCH, r)) + 8 * (tr_a & 1);
  }
  auto vread_tr = [&](const unsigned char* sVt, int kb2, int u, int db) __attribute__((always_inline)) {
    const unsigned char* r0 = sVt + va[db & 1] + 128 * (db >> 1) + (32 * kb2 + 8 * u) * VCH * 16;
    const s16x4 a[2] = {lds_read_tr16(r0), lds_read_tr16(r0 + 4 * VCH * 16)};
    return __builtin_bit_cast(u32x4, a);
  };

  // Row-sum A operand: 1 where the k group's parity (lane / 16) equals the parity of the
  // output row's quad, so every register of l holds the lane's own row (l % 32) sum.
  const uint32_t one2 = __is_same(QT, bf16_t) ? 0x3F803F80u : 0x3C003C00u;   // two 1.0 values of QT
  const u32x4 ones = (((lane >> 2) ^ (lane >> 4)) & 1) == 0 ? u32x4{one2, one2, one2, one2} : u32x4{0u, 0u, 0u, 0u};
  auto reset = [&](Blk& b) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) b.o[db] = f32x16{};
    b.l = f32x4{};
    b.m = 0.f;
  };
  auto set_m = [&](Blk& b, float m) __attribute__((always_inline)) {
    b.m = m;
#pragma unroll
    for (int r = 0; r < 16; ++r) b.mi[r] = -m;
  };

  // S^T = K'(0) Q'^T of a block's first tile (chains start from 0: M is not set yet)
  auto qk0 = [&](Blk& b) __attribute__((always_inline)) {
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) b.s[kb2] = f32x16{};
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t)
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) b.s[kb2] = Mma<QT>::run(kread(sK, false, t, kb2), b.qf[t], b.s[kb2]);
#pragma unroll
    for (int t = 0; t < PSTEPS; ++t)
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) b.s[kb2] = Mma<PT>::run(kread(sK, true, t, kb2), b.pf[t], b.s[kb2]);
  };
  // The matrix work of block x in one key step: O += V(t)^T P(t)^T (with the row sum), then
  // (with_qk) S(t+1) = K'(t+1) Q'^T, every score chain starting from the block's -M vector;
  // LDS operands read one group ahead (group = the MFMAs of one k-step: DB P V MFMAs and a
  // row-sum MFMA, or NKB score MFMAs).  (The two blocks read the same operands; reading them
  // once for both needs 40 more registers, which the -M vectors use to better effect: the
  // vector unit, not the LDS, bounds this kernel.)
  constexpr int NPV = NKB * 2;
  constexpr int NQK = QSTEPS + PSTEPS;
  auto mma = [&](Blk& x, const unsigned char* sKn, const unsigned char* sVt, auto with_qk) __attribute__((always_inline)) {
    constexpr int NG = NPV + (decltype(with_qk)::value ? NQK : 0);
    u32x4 opnd[NG][NKB > DB ? NKB : DB];
    auto issue = [&](int g) __attribute__((always_inline)) {
      if (g < NPV) {
#pragma unroll
        for (int db = 0; db < DB; ++db) opnd[g][db] = vread_tr(sVt, g >> 1, g & 1, db);
      } else {
        const int t = g - NPV;
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
          opnd[g][kb2] = t < QSTEPS ? kread(sKn, false, t, kb2) : kread(sKn, true, t - QSTEPS, kb2);
      }
    };
    issue(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) issue(g + 1);
      if (g < NPV) {
#pragma unroll
        for (int db = 0; db < DB; ++db) x.o[db] = Mma<QT>::run(opnd[g][db], x.pr[g], x.o[db]);
        x.l = Mma16<QT>::run(ones, x.pr[g], x.l);
      } else {
        const int t = g - NPV;
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
          const f32x16 c = t == 0 ? x.mi : x.s[kb2];
          x.s[kb2] = t < QSTEPS ? Mma<QT>::run(opnd[g][kb2], x.qf[t], c) : Mma<PT>::run(opnd[g][kb2], x.pf[t - QSTEPS], c);
        }
      }
    }
  };
  // First part of the softmax of tile t (scores S log2(e) - M in y.s): keys past N masked, the
  // row max; the first tile sets M to its max (key 0 is always visible), later tiles move it
  // when they exceed it by RES_GROW, rescaling O and the row sum.  (A uniform branch: it
  // stays outside the interleaved region.)
  auto rowmax = [&](Blk& y, int t, auto may_mask) __attribute__((always_inline)) {
    const int kb = t * BN;
    if (decltype(may_mask)::value && kb + BN > N) {
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const int lim = N - (kb + 32 * kb2 + 16 * hf);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          y.s[kb2][r] = r < lim ? y.s[kb2][r] : -INFINITY;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, y.s[kb2][r]);
    mx = halves_max(mx);
    const bool first = t == 0;
    const bool grow = first || mx > RES_GROW;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float d = grow ? mx : 0.f;
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(-d);
#pragma unroll
        for (int db = 0; db < DB; ++db) y.o[db] *= alpha;
        y.l *= alpha;
      }
      set_m(y, y.m + d);
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) y.s[kb2] -= d;
    }
  };
  // Second part: P = exp2(scores), rounded to the input dtype (straight-line vector work).
  // The empty asm that takes P keeps the work in the region where it is written (otherwise
  // the compiler sinks it past the next branch, out of the MFMAs' region, next to its use).
  auto expo = [&](Blk& y) __attribute__((always_inline)) {
    typedef QT T8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        T8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = from_f32<QT>(__builtin_amdgcn_exp2f(y.s[kb2][8 * u + j]));
        y.pr[kb2 * 2 + u] = __builtin_bit_cast(u32x4, pb);
      }
#pragma unroll
    for (int i = 0; i < NKB * 2; ++i) asm volatile("" : "+v"(y.pr[i]));
  };
  // epilogue of a block: O = O / l, LSE = (M + log2 l) ln 2.  Register r of lane half hf in
  // head-dim block db holds head dim 32 db + 8 (r / 4) + 4 hf + r % 4.
  auto store = [&](Blk& b, int rb) __attribute__((always_inline)) {
    const int qrow = rb * 32 + ln;
    if (qrow < N) {
      const float l_tot = b.l[0];
      const float inv = 1.f / l_tot;
      QT* orow = Op + qrow * p.so[2];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int d0 = 32 * db + 8 * c + 4 * hf;
          if (d0 < D) {
            typedef QT T4 __attribute__((ext_vector_type(4)));
            T4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = from_f32<QT>(b.o[db][4 * c + j] * inv);
            *(T4*)(orow + d0) = v;
          }
        }
      if (p.lse && hf == 0) p.lse[((int64_t)bb * p.H + hh) * N + qrow] = (b.m + __log2f(l_tot)) * LN2;
    }
  };

  const std::true_type QK, MASK;
  const std::false_type NOQK, NOMASK;
  // ---- the block pairs of this wavefront --------------------------------------------
  // Schedule (block B half a step behind A): after the prologue A holds P_A(0) and B the
  // scores S_B(0); key step t then runs
  //   rowmax_B(t)   | MFMA_A(t) = {O_A += V(t) P_A(t), S_A(t+1)}  with  expo_B(t)
  //   rowmax_A(t+1) | MFMA_B(t) = {O_B += V(t) P_B(t), S_B(t+1)}  with  expo_A(t+1)
  // where "with" puts both into one straight-line region (independent registers), so the
  // vector work issues while the MFMAs run.  Only the last tile can have keys past N: the
  // steps before the last two carry no mask code (a branch would split the regions).  The
  // last step has no next scores.
  auto step = [&](int t, auto mask_next) __attribute__((always_inline)) {
    const unsigned char* kn = sK + (t + 1) * SKB;
    const unsigned char* vt = sV + t * SVB;
    rowmax(B, t, NOMASK);
    mma(A, kn, vt, QK);
    expo(B);
    rowmax(A, t + 1, mask_next);
    mma(B, kn, vt, QK);
    expo(A);
  };
  for (; a0 < nrb; a0 += 2 * RNW) {
    reset(A);
    reset(B);
    qk0(A);
    rowmax(A, 0, MASK);
    qk0(B);
    expo(A);
    int t = 0;
    for (; t + 2 < nkt; ++t) {
      // step t reads tile t + 1 (K') and t (V); tile th first at step th - 1 >= 1, inside this
      // loop since th <= nkt - 2; every wavefront with a block pair gets here in its first one
      if (split_pending && t == th - 1) split_barrier();
      step(t, NOMASK);
    }
    if (t + 1 < nkt) step(t++, MASK);
    {
      const unsigned char* vt = sV + t * SVB;
      rowmax(B, t, MASK);
      mma(A, sK, vt, NOQK);
      expo(B);
      mma(B, sK, vt, NOQK);
    }
    // the next pair's fragments (their loads run under this pair's stores)
    if (a0 + 2 * RNW < nrb) {
      load_frags(A, row_of(a0 + 2 * RNW));
      load_frags(B, row_of(a0 + 3 * RNW));
    }
    store(A, a0);
    store(B, a0 + RNW);
  }
  // a wavefront without a block pair (short N) still takes its part in the split barrier
  if (split_pending) split_barrier();
}

}  // namespace attn
}  // namespace fb
