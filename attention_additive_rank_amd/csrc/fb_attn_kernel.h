// Fused forward kernel for attention with an additive bias on gfx950 (CDNA4).
//
//   O = softmax(s Q K^T + b) V
//
// MODE 0 (low rank, FlashBias): b = phi_q phi_k^T is folded into one augmented
// contraction Q' = [Q*s, phi_q], K' = [K, phi_k] (FlashBias rebuttal, answer to
// Reviewer UJUf, Q2: concatenate the factor functions with queries and keys,
// then run FlashAttention).  MODE 1 (dense bias, the baseline): the contraction
// is Q*s K^T and a bias tile is read from HBM for every (query, key) tile pair,
// the quadratic IO of the abstract and Fig. 1(c).
//
// Work decomposition
//   * One workgroup = 8 wavefronts = 256 query rows of one (batch, head); each
//     wavefront owns 32 query rows for the whole key loop.  Waves w and w+4 run
//     on the same SIMD, so the two groups {0..3} and {4..7} pair up per SIMD.
//   * Ping-pong schedule: per key tile each wavefront has a matrix phase
//     (S(t+1) = K'(t+1) Q'^T and O += Vt(t) P(t)^T on the MFMA units) and a
//     vector phase (online softmax of S(t+1)); the two groups run opposite
//     phases between workgroup barriers, so on every SIMD one wave keeps the
//     matrix core busy while the other does exp2/max/sum on the VALU.  The
//     group in its vector phase also refills LDS for later tiles (group 1 the
//     K' rows, group 0 the V rows), from registers loaded two phases earlier.
//   * Key tiles of 64 keys are double-buffered in LDS: K' rows (K then phi_k,
//     zero-padded to RP columns) and V transposed (Vt[d][key]).  Rows past N
//     are clamped on load and masked in the scores (no bounds branches).
//   * Scores are computed transposed, S^T = K' Q'^T, with 32x32 MFMAs
//     (32x32x16 bf16/f16, 32x32x2 fp32).  With that orientation every lane owns
//     ONE query (lane % 32) and 16 keys per 32-key block, so the row max / row
//     sum of the online softmax are in-lane reductions plus a single exchange
//     between the two half-waves, and P^T is already in the B-operand layout of
//     the next product O^T = Vt P^T: P never leaves registers.
//   * Lazy rescaling: the running row max only moves (and O, l are rescaled)
//     when a tile's max exceeds it by more than 2^8 in exp2 units, so most
//     tiles skip the O rescale; P then stays <= 2^8, exact in range for bf16.
//   * K' rows and Vt rows are permuted in LDS so that lane half h holds keys
//     16h..16h+15 of each 32-key block (and, in the output, head dims
//     16h..16h+15 of each 32-dim block): bias reads, the causal mask and the
//     O stores then touch contiguous runs.
//   * The factor columns of K' / Q' go through their own MFMA chain in the
//     factor dtype (PT), accumulating into the same fp32 score tile.
//   * Workgroup ids are remapped so that the query blocks of one (b, h) run on
//     one XCD (dispatch is round-robin over the 8 XCDs): their K'/V tiles are
//     then shared in that XCD's L2.  Causal launches take the longest query
//     blocks first.
#pragma once

#include "fb_internal.h"

namespace fb {
namespace attn {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 8;          // wavefronts per workgroup: two groups of four
constexpr int NT = NW * 64;    // threads per workgroup
constexpr int GT = NT / 2;     // threads per group
constexpr int BM = 32 * NW;    // query rows per workgroup
static_assert(BM == kAttnBlockM, "host and kernel block sizes differ");
constexpr int BN = 64;         // keys per LDS tile
constexpr int NKB = BN / 32;   // 32-key blocks per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_GAP = 8.0f / LOG2E;   // 2^8 in exp2 units, as a natural-log gap

template <typename T> struct Elem;
template <> struct Elem<bf16_t> { typedef u32x4 Frag; static constexpr int KW = 8; };
template <> struct Elem<f16_t>  { typedef u32x4 Frag; static constexpr int KW = 8; };
template <> struct Elem<float>  { typedef float Frag; static constexpr int KW = 1; };

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<f16_t> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ f32x16 run(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// A 16-byte chunk viewed as a vector of its elements.
template <typename T> struct ChunkOf;
template <> struct ChunkOf<bf16_t> { typedef bf16x8 type; };
template <> struct ChunkOf<f16_t>  { typedef f16x8 type; };
template <> struct ChunkOf<float>  { typedef f32x4 type; };
template <typename T> using ChunkV = typename ChunkOf<T>::type;

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }

// Position inside a 32-row MFMA block that holds logical index k (key or head dim):
// MFMA row m = 8a + 4h + c carries index 16h + 4a + c, so that output register r
// of lane half h corresponds to index 16h + r.
__host__ __device__ constexpr int perm_row(int k) {
  return (k & ~31) | (((k & 15) >> 2) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// Scale the KW query elements of one fragment by s and round them back to T.
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag scale_frag(typename Elem<T>::Frag f, float s) {
  if constexpr (Elem<T>::KW == 1) {
    return f * s;
  } else {
    typedef T T8 __attribute__((ext_vector_type(8)));
    T8 v = __builtin_bit_cast(T8, f);
    T8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = from_f32<T>(to_f32<T>(v[j]) * s);
    return __builtin_bit_cast(u32x4, r);
  }
}

// All ones when i < lim, else zero (branch-free: no per-element lane masks).
__device__ __forceinline__ uint32_t below_mask(int i, int lim) { return (uint32_t)((i - lim) >> 31); }

// CE elements of row[c0..] (row has `len` valid elements), zero past len; element loads
// are clamped into the row and the excess is zeroed arithmetically.
template <typename T>
__device__ __forceinline__ u32x4 load_partial_chunk(const T* row, int c0, int len) {
  constexpr int CE = 16 / (int)sizeof(T);
  u32x4 r;
  if constexpr (sizeof(T) == 2) {
    const uint16_t* src = (const uint16_t*)row;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = src[min(c0 + 2 * w, len - 1)] & below_mask(c0 + 2 * w, len);
      const uint32_t hi = src[min(c0 + 2 * w + 1, len - 1)] & below_mask(c0 + 2 * w + 1, len);
      r[w] = lo | (hi << 16);
    }
  } else {
    const uint32_t* src = (const uint32_t*)row;
#pragma unroll
    for (int w = 0; w < CE; ++w) r[w] = src[min(c0 + w, len - 1)] & below_mask(c0 + w, len);
  }
  return r;
}

// One 16-byte chunk of a factor row (CE elements starting at column c0), zero past R.
template <typename T>
__device__ __forceinline__ u32x4 load_phi_chunk(const T* row, int c0, int R, bool vec) {
  if (vec) return ld16(row + c0);
  return load_partial_chunk<T>(row, c0, R);
}

// max / sum of a value over the two half-waves (lanes l and l ^ 32).  v_permlane32_swap
// exchanges the upper half of one register with the lower half of the other, so after
// swapping two copies of x every lane holds x and x of lane l ^ 32 in (a, b).  Written as
// asm: the compiler's intrinsic folds the swap of two equal values into a no-op, and the
// portable shuffle goes through ds_bpermute (an LDS round trip).  s_nop 1 covers the
// VALU-write -> permlane-read hazard.
__device__ __forceinline__ float halves_max(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}
__device__ __forceinline__ float halves_sum(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}

template <typename QT, typename PT, int D, int RP, int MODE, typename BT, bool CAUSAL>
__global__ __launch_bounds__(NT, 1) void attn_fwd_kernel(AttnParams p) {
  typedef typename Elem<QT>::Frag QFrag;
  typedef typename Elem<PT>::Frag PFrag;
  constexpr int ES = (int)sizeof(QT);
  static_assert(sizeof(PT) == sizeof(QT), "factor and query element sizes must match");
  static_assert(MODE == 0 || RP == 0, "dense-bias mode has no factor columns");
  constexpr int KW = Elem<QT>::KW;        // k elements per lane per MFMA
  constexpr int KS = 2 * KW;              // k per MFMA
  constexpr int CE = 16 / ES;             // elements per 16-byte chunk
  constexpr int W = D + RP;               // width of the augmented contraction
  constexpr int PITCH_K = W * ES + 16;    // LDS bytes per K' row (+16: conflict-free 128-bit reads)
  constexpr int DP = D < 32 ? 32 : D;     // Vt rows, padded to one 32-row MFMA block
  constexpr int PITCH_V = BN * ES + 16;
  constexpr int DB = DP / 32;             // 32-wide head-dim blocks of the output
  constexpr int QSTEPS = D / KS;
  constexpr int PSTEPS = RP / KS;
  constexpr int KCH = D / CE;             // chunks per K / V row
  constexpr int PCH = RP / CE;            // chunks per phi_k row
  constexpr int K_TOT = BN * KCH;         // K chunks per tile
  constexpr int P_TOT = BN * PCH;         // phi_k chunks per tile
  constexpr int V_TOT = (BN / 2) * KCH;   // V tasks per tile: one chunk column of a key pair
  constexpr int KPT = (K_TOT + GT - 1) / GT;
  constexpr int PPT = P_TOT > 0 ? (P_TOT + GT - 1) / GT : 0;
  constexpr int VPT = (V_TOT + GT - 1) / GT;
  constexpr int SK_BYTES = BN * PITCH_K;
  constexpr int SV_BYTES = DP * PITCH_V;
  static_assert(D % KS == 0 && RP % KS == 0 && D % CE == 0 && RP % CE == 0, "bad tile widths");

  __shared__ __attribute__((aligned(16))) unsigned char sK[2 * SK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sV[2 * SV_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;     // waves w and w+4 share a SIMD: one of each group per SIMD
  const int gtid = tid & (GT - 1);
  const int ln = lane & 31;
  const int hf = lane >> 5;

  // ---- workgroup -> (query block, head, batch), XCD-aware -------------------
  const int G = (int)gridDim.x;
  const int wg = (int)blockIdx.x;
  const int xcd = wg & 7, idx = wg >> 3;
  const int per = G >> 3, rem = G & 7;
  const int L = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  int qb = L % p.nqb;
  const int bh = L / p.nqb;
  if (CAUSAL) qb = p.nqb - 1 - qb;
  const int hh = bh % p.H;
  const int bb = bh / p.H;
  const int N = p.N;

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
  const BT* Bp = nullptr;
  if constexpr (MODE == 1) Bp = (const BT*)p.bias + ((int64_t)bb * p.sb[0] + (int64_t)hh * p.sb[1]);

  const int q0 = qb * BM;
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + ln;
  const bool qvalid = qrow < N;
  const int qclamp = qvalid ? qrow : N - 1;
  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int nkt = (kend + BN - 1) / BN;

  // Vt rows of head dims >= D (only when D < 32) are never written by the tile
  // stores: clear them once in both buffers so the discarded output rows stay finite.
  if constexpr (D < DP) {
    for (int i = tid; i < 2 * (DP - D) * BN; i += NT) {
      const int buf = i / ((DP - D) * BN), r = i % ((DP - D) * BN);
      const int d = D + r / BN, key = r % BN;
      unsigned char* dst = sV + buf * SV_BYTES + perm_row(d) * PITCH_V + key * ES;
      if constexpr (ES == 2) *(uint16_t*)dst = 0; else *(uint32_t*)dst = 0;
    }
  }

  // ---- Q' fragments (B operand of S^T = K' Q'^T), resident for the whole loop
  QFrag qf[QSTEPS];
  PFrag pf[PSTEPS > 0 ? PSTEPS : 1];
#pragma unroll
  for (int t = 0; t < QSTEPS; ++t) {
    if constexpr (KW == 1) qf[t] = scale_frag<QT>(Qp[qclamp * p.sq[2] + KS * t + hf], p.scale);
    else qf[t] = scale_frag<QT>(ld16(Qp + qclamp * p.sq[2] + KS * t + KW * hf), p.scale);
  }
  if constexpr (RP > 0) {
    const PT* prow = PQp + qclamp * p.spq[2];
#pragma unroll
    for (int t = 0; t < PSTEPS; ++t) {
      const int c0 = KS * t + KW * hf;
      if constexpr (KW == 1) pf[t] = c0 < p.R ? prow[c0] : 0.f;
      else pf[t] = load_phi_chunk<PT>(prow, c0, p.R, (p.flags & FLAG_PHQ_VEC) && c0 + KW <= p.R);
    }
  }

  // ---- staging: group 1 streams K' tiles (K then phi_k), group 0 V tiles ----
  // K chunk i of a group-1 thread covers row c / KCH, chunk column c % KCH (c = gtid + i*GT).
  const QT* k_ptr[KPT];
  int k_row[KPT], k_lds[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int c = gtid + i * GT;
    const int cc = c < K_TOT ? c : 0;
    k_row[i] = cc / KCH;
    k_ptr[i] = Kp + k_row[i] * p.sk[2] + (cc % KCH) * CE;
    k_lds[i] = perm_row(k_row[i]) * PITCH_K + (cc % KCH) * 16;
  }
  const PT* p_ptr[PPT > 0 ? PPT : 1];
  int p_row[PPT > 0 ? PPT : 1], p_col[PPT > 0 ? PPT : 1], p_lds[PPT > 0 ? PPT : 1];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int c = gtid + i * GT;
    const int cc = c < P_TOT ? c : 0;
    p_row[i] = cc / PCH;
    p_col[i] = (cc % PCH) * CE;
    p_ptr[i] = PKp + p_row[i] * p.spk[2];
    p_lds[i] = perm_row(p_row[i]) * PITCH_K + D * ES + (cc % PCH) * 16;
  }
  // factor rows: 16-byte vector loads when every chunk is either full or past R
  const bool phk_fast = (RP == 0) || ((p.flags & FLAG_PHK_VEC) && p.R % CE == 0);
  // V task i of a group-0 thread: key pair pr (keys 2pr, 2pr+1), chunk column vc;
  // pairs run fastest across lanes so each 32-bit LDS write hits distinct banks.
  const QT* v_ptr[VPT];
  int v_pair[VPT], v_col[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = gtid + i * GT;
    const int cc = c < V_TOT ? c : 0;
    v_pair[i] = cc % (BN / 2);
    v_col[i] = cc / (BN / 2);
    v_ptr[i] = Vp + (2 * v_pair[i]) * p.sv[2] + v_col[i] * CE;
  }

  u32x4 kr[KPT], vr0[VPT], vr1[VPT];
  u32x4 pr[PPT > 0 ? PPT : 1];

  auto load_k = [&](int kb) {          // group 1: K' rows of the tile starting at key kb
    const bool full = kb + BN <= N;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (K_TOT % GT == 0 || gtid + i * GT < K_TOT) {
        const int key = full ? kb + k_row[i] : min(kb + k_row[i], N - 1);
        kr[i] = ld16(k_ptr[i] + (key - k_row[i]) * p.sk[2]);
      }
    if constexpr (PPT > 0) {
#pragma unroll
      for (int i = 0; i < PPT; ++i)
        if (P_TOT % GT == 0 || gtid + i * GT < P_TOT) {
          const int key = min(kb + p_row[i], N - 1);
          const PT* row = p_ptr[i] + (key - p_row[i]) * p.spk[2];
          if (phk_fast) pr[i] = p_col[i] < p.R ? ld16(row + p_col[i]) : u32x4{};
          else pr[i] = load_partial_chunk<PT>(row, p_col[i], p.R);
        }
    }
  };
  auto store_k = [&](int buf) {
    unsigned char* base = sK + buf * SK_BYTES;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (K_TOT % GT == 0 || gtid + i * GT < K_TOT) st16(base + k_lds[i], kr[i]);
    if constexpr (PPT > 0) {
#pragma unroll
      for (int i = 0; i < PPT; ++i)
        if (P_TOT % GT == 0 || gtid + i * GT < P_TOT) st16(base + p_lds[i], pr[i]);
    }
  };
  auto load_v = [&](int kb) {          // group 0: V rows of the tile starting at key kb
    const bool full = kb + BN <= N;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (V_TOT % GT == 0 || gtid + i * GT < V_TOT) {
        const int k0 = full ? kb + 2 * v_pair[i] : min(kb + 2 * v_pair[i], N - 1);
        const int k1 = full ? k0 + 1 : min(kb + 2 * v_pair[i] + 1, N - 1);
        vr0[i] = ld16(v_ptr[i] + (k0 - 2 * v_pair[i]) * p.sv[2]);
        vr1[i] = ld16(v_ptr[i] + (k1 - 2 * v_pair[i]) * p.sv[2]);
      }
  };
  auto store_v = [&](int buf) {        // transposed: Vt[d][key]
    unsigned char* base = sV + buf * SV_BYTES;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (V_TOT % GT == 0 || gtid + i * GT < V_TOT) {
        unsigned char* dst = base + 2 * v_pair[i] * ES;
        const int d0 = v_col[i] * CE;
        if constexpr (ES == 2) {
          // element j of both keys -> one 32-bit word (key 2pr low, key 2pr+1 high)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t lo = __builtin_amdgcn_perm(vr1[i][m], vr0[i][m], 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(vr1[i][m], vr0[i][m], 0x07060302u);
            *(uint32_t*)(dst + perm_row(d0 + 2 * m) * PITCH_V) = lo;
            *(uint32_t*)(dst + perm_row(d0 + 2 * m + 1) * PITCH_V) = hi;
          }
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            u32x2 w2 = {vr0[i][m], vr1[i][m]};
            *(u32x2*)(dst + perm_row(d0 + m) * PITCH_V) = w2;
          }
        }
      }
    }
  };

  // ---- per-wave state ----------------------------------------------------------
  f32x16 sacc[NKB];                    // S^T of the tile being processed
  u32x4 pfrag[KW == 1 ? 1 : NKB * 2];  // P^T (16-bit), B operand of the P V product
  float p32[KW == 1 ? NKB : 1][16];    // P^T (fp32 path)
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // dense bias of this lane's row, keys kb + 32*kb2 + 16*hf + [0, 16), loaded one tile ahead
  constexpr int BES = MODE == 1 ? (int)sizeof(BT) : 2;
  constexpr int BCH = BES;                  // 16-byte chunks per 16 keys
  constexpr int NBR = MODE == 1 ? NKB * BCH : 1;
  u32x4 braw[NBR];
  auto load_bias = [&](int kb) {
    if constexpr (MODE == 1) {
      const BT* brow = Bp + qclamp * p.sb[2];
      constexpr int BCE = 16 / BES;
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const int j0 = kb + 32 * kb2 + 16 * hf;
        if ((p.flags & FLAG_BIAS_VEC) && j0 + 16 <= N) {
#pragma unroll
          for (int c = 0; c < BCH; ++c) braw[kb2 * BCH + c] = ld16(brow + j0 + c * BCE);
        } else {
#pragma unroll
          for (int c = 0; c < BCH; ++c) braw[kb2 * BCH + c] = load_partial_chunk<BT>(brow, j0 + c * BCE, N);
        }
      }
    }
  };

  // A wavefront whose queries all precede a key tile has nothing to do there.
  auto active = [&](int t) { return !CAUSAL || t * BN <= q0w + 31; };

  // S^T = K'(t) Q'^T from LDS buffer `buf`
  auto qk = [&](int buf) {
    const unsigned char* k_base = sK + buf * SK_BYTES + ln * PITCH_K;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = f32x16{};
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const unsigned char* a = k_base + 32 * kb2 * PITCH_K + (KS * t + KW * hf) * ES;
        if constexpr (KW == 1) sacc[kb2] = Mma<QT>::run(*(const float*)a, qf[t], sacc[kb2]);
        else sacc[kb2] = Mma<QT>::run(ld16(a), qf[t], sacc[kb2]);
      }
    }
    if constexpr (RP > 0) {
#pragma unroll
      for (int t = 0; t < PSTEPS; ++t) {
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
          const unsigned char* a = k_base + 32 * kb2 * PITCH_K + (D + KS * t + KW * hf) * ES;
          if constexpr (KW == 1) sacc[kb2] = Mma<PT>::run(*(const float*)a, pf[t], sacc[kb2]);
          else sacc[kb2] = Mma<PT>::run(ld16(a), pf[t], sacc[kb2]);
        }
      }
    }
  };

  // O^T += Vt(t) P(t)^T from LDS buffer `buf`
  auto pv = [&](int buf) {
    const unsigned char* v_base = sV + buf * SV_BYTES + ln * PITCH_V + 16 * hf * ES;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) {
      if constexpr (KW == 1) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const float a = *(const float*)(v_base + 32 * db * PITCH_V + (32 * kb2 + u) * ES);
            oacc[db] = Mma<QT>::run(a, p32[kb2][u], oacc[db]);
          }
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x4 a = ld16(v_base + 32 * db * PITCH_V + (32 * kb2 + 8 * u) * ES);
            oacc[db] = Mma<QT>::run(a, pfrag[kb2 * 2 + u], oacc[db]);
          }
      }
    }
  };

  // online softmax of tile t (scores in sacc) -> P(t); lazy rescaling of O and l
  auto softmax = [&](int t) {
    const int kb = t * BN;
    if constexpr (MODE == 1) {
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int c = 0; c < BCH; ++c) {
          const ChunkV<BT> e = __builtin_bit_cast(ChunkV<BT>, braw[kb2 * BCH + c]);
#pragma unroll
          for (int j = 0; j < 16 / BES; ++j) sacc[kb2][c * (16 / BES) + j] += to_f32<BT>(e[j]);
        }
      if (t + 1 < nkt) load_bias(kb + BN);
    }
    // mask: keys past N, and keys after the query when causal
    const bool need_mask = (kb + BN > N) || (CAUSAL && kb + BN - 1 > q0w);
    if (need_mask) {
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const int j0 = kb + 32 * kb2 + 16 * hf;
        int lim = N - j0;
        if constexpr (CAUSAL) lim = min(lim, qrow + 1 - j0);
        // One compare-select at a time: the scheduling fence keeps the compiler from
        // hoisting all compares into simultaneously live scalar lane masks.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[kb2][r] = r < lim ? sacc[kb2][r] : -INFINITY;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
    mx = halves_max(mx);
    const bool grow = mx > m_run + RESCALE_GAP;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - mx) * LOG2E) : 1.f;  // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = grow ? mx : m_run;
    }
    const float ms = (m_run == -INFINITY ? 0.f : m_run) * LOG2E;
    if constexpr (KW == 1) {
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][r], LOG2E, -ms));
          p32[kb2][r] = e;
          l_run += e;
        }
    } else {
      typedef QT T8 __attribute__((ext_vector_type(8)));
      typedef QT T2 __attribute__((ext_vector_type(2)));
      float lsum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          T8 pb;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            pb[j] = from_f32<QT>(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][8 * u + j], LOG2E, -ms)));
          pfrag[kb2 * 2 + u] = __builtin_bit_cast(u32x4, pb);
          // row sum of the rounded probabilities (what the P V product uses)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const T2 two = {pb[2 * m], pb[2 * m + 1]};
            const T2 one = {from_f32<QT>(1.f), from_f32<QT>(1.f)};
            if constexpr (__is_same(QT, bf16_t))
              lsum = __builtin_amdgcn_fdot2_f32_bf16(two, one, lsum, false);
            else
              lsum = __builtin_amdgcn_fdot2(two, one, lsum, false);
          }
        }
      l_run += lsum;
    }
  };

  // Matrix phase of tile t: S(t+1) = K'(t+1) Q'^T and O += Vt(t) P(t)^T.
  auto mma_phase = [&](int t) {
    if (t + 1 < nkt && active(t + 1)) qk((t + 1) & 1);
    if (active(t)) pv(t & 1);
  };

  // ---- prologue: K'(0), K'(1), V(0) in LDS; K'(2), V(1) in flight; P(0) -------
  if (grp == 1) {
    load_k(0);
    store_k(0);
    if (nkt > 1) {
      load_k(BN);
      store_k(1);
    }
    if (nkt > 2) load_k(2 * BN);
  } else {
    load_v(0);
    store_v(0);
    if (nkt > 1) load_v(BN);
  }
  load_bias(0);
  __syncthreads();
  qk(0);
  softmax(0);
  __syncthreads();

  // ---- ping-pong: per SIMD, one wave multiplies while the other does softmax ----
  // group 0: phase A = MFMA(t) [S(t+1) = K'(t+1) Q'^T, O += Vt(t) P(t)], phase B = softmax(t+1)
  // group 1: phase A = softmax(t) (t > 0),                               phase B = MFMA(t)
  // The softmax group also refills LDS: group 1 K'(t+2) in phase A, group 0 V(t+1) in phase B.
  for (int t = 0; t < nkt; ++t) {
    const int kb = t * BN;
    // ---- phase A ----
    if (grp == 0) {
      mma_phase(t);
    } else {
      if (t + 2 < nkt) {
        store_k(t & 1);
        if (t + 3 < nkt) load_k(kb + 3 * BN);
      }
      if (t > 0 && active(t)) softmax(t);
    }
    __syncthreads();
    // ---- phase B ----
    if (grp == 0) {
      if (t + 1 < nkt) {
        store_v((t + 1) & 1);
        if (t + 2 < nkt) load_v(kb + 2 * BN);
      }
      if (t + 1 < nkt && active(t + 1)) softmax(t + 1);
    } else {
      mma_phase(t);
    }
    __syncthreads();
  }

  // ---- epilogue: O = O / l, LSE = m + ln l -----------------------------------
  const float l_tot = halves_sum(l_run);
  if (qvalid) {
    const float inv = 1.f / l_tot;
    QT* orow = Op + qrow * p.so[2];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = 32 * db + 16 * hf;
      if (d0 < D) {
#pragma unroll
        for (int c = 0; c < 16 / CE; ++c) {
          ChunkV<QT> v;
#pragma unroll
          for (int j = 0; j < CE; ++j) v[j] = from_f32<QT>(oacc[db][c * CE + j] * inv);
          st16(orow + d0 + c * CE, __builtin_bit_cast(u32x4, v));
        }
      }
    }
    if (p.lse && hf == 0) p.lse[((int64_t)bb * p.H + hh) * N + qrow] = m_run + logf(l_tot);
  }
}

}  // namespace attn
}  // namespace fb
