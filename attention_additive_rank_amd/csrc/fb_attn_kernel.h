// Fused forward kernel for attention with an additive bias on gfx950 (CDNA4).
//
//   O = softmax(s Q K^T + b) V
//
// MODE 0 (low rank, FlashBias): b = phi_q phi_k^T is folded into one augmented
// contraction Q' = [Q*s, phi_q], K' = [K, phi_k] (FlashBias rebuttal, answer to
// Reviewer UJUf, Q2: concatenate the factor functions with queries and keys,
// then run FlashAttention).  MODE 1 (dense bias, the baseline): the contraction
// is Q*s K^T and a bias tile is read from HBM for every (query, key) tile pair,
// the quadratic IO the abstract and Fig. 1(c) describe.
//
// Work decomposition
//   * One workgroup = 4 wavefronts = 128 query rows of one (batch, head); each
//     wavefront owns 32 query rows for the whole key loop.
//   * Key tiles of 64 keys are staged in LDS once per workgroup: K' rows
//     (K then phi_k, zero-padded to RP columns) and V transposed (Vt[d][key]).
//   * Scores are computed transposed, S^T = K' Q'^T, with 32x32 MFMAs
//     (32x32x16 bf16/f16, 32x32x2 fp32).  With that orientation every lane owns
//     ONE query (lane % 32) and 16 keys per 32-key block, so the row max / row
//     sum of the online softmax are in-lane reductions plus a single exchange
//     between the two half-waves, and P^T is already in the B-operand layout of
//     the next product O^T = Vt P^T: P never leaves registers.
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int NW = 4;          // wavefronts per workgroup
constexpr int NT = NW * 64;    // threads per workgroup
constexpr int BM = 32 * NW;    // query rows per workgroup
constexpr int BN = 64;         // keys per LDS tile
constexpr float LOG2E = 1.4426950408889634f;

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
__device__ __forceinline__ int perm_row(int k) {
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

// One 16-byte chunk of a factor row (CE elements starting at column c0), zero past R.
template <typename T>
__device__ __forceinline__ u32x4 load_phi_chunk(const T* row, int c0, int R, int vec) {
  constexpr int CE = 16 / (int)sizeof(T);
  if (vec && c0 + CE <= R) return ld16(row + c0);
  ChunkV<T> v;
#pragma unroll
  for (int e = 0; e < CE; ++e) v[e] = (c0 + e < R) ? row[c0 + e] : from_f32<T>(0.f);
  return __builtin_bit_cast(u32x4, v);
}

template <typename QT, typename PT, int D, int RP, int MODE, typename BT>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(AttnParams p) {
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
  constexpr int KPT = (BN * KCH + NT - 1) / NT;
  constexpr int PPT = PCH > 0 ? (BN * PCH + NT - 1) / NT : 0;
  static_assert(D % KS == 0 && RP % KS == 0 && D % CE == 0 && RP % CE == 0, "bad tile widths");

  __shared__ __attribute__((aligned(16))) unsigned char sK[BN * PITCH_K];
  __shared__ __attribute__((aligned(16))) unsigned char sV[DP * PITCH_V];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  if (p.causal) qb = p.nqb - 1 - qb;
  const int hh = bh % p.H;
  const int bb = bh / p.H;
  const int N = p.N;

  const QT* Qp = (const QT*)p.q + bb * p.sq[0] + hh * p.sq[1];
  const QT* Kp = (const QT*)p.k + bb * p.sk[0] + hh * p.sk[1];
  const QT* Vp = (const QT*)p.v + bb * p.sv[0] + hh * p.sv[1];
  QT* Op = (QT*)p.o + bb * p.so[0] + hh * p.so[1];
  const PT* PQp = nullptr;
  const PT* PKp = nullptr;
  if constexpr (RP > 0) {
    PQp = (const PT*)p.phq + bb * p.spq[0] + hh * p.spq[1];
    PKp = (const PT*)p.phk + bb * p.spk[0] + hh * p.spk[1];
  }
  const BT* Bp = nullptr;
  if constexpr (MODE == 1) Bp = (const BT*)p.bias + bb * p.sb[0] + hh * p.sb[1];

  const int q0 = qb * BM;
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + ln;
  const bool qvalid = qrow < N;

  // Vt rows of head dims >= D (only when D < 32) are never written by the tile
  // stores: clear them once so that the discarded output rows stay finite.
  if constexpr (D < DP) {
    for (int i = tid; i < (DP - D) * BN; i += NT) {
      const int d = D + i / BN, key = i % BN;
      unsigned char* dst = sV + perm_row(d) * PITCH_V + key * ES;
      if constexpr (ES == 2) *(uint16_t*)dst = 0; else *(uint32_t*)dst = 0;
    }
  }

  // ---- Q' fragments (B operand of S^T = K' Q'^T), resident for the whole loop
  QFrag qf[QSTEPS];
  PFrag pf[PSTEPS > 0 ? PSTEPS : 1];
#pragma unroll
  for (int t = 0; t < QSTEPS; ++t) {
    if (qvalid) {
      if constexpr (KW == 1) qf[t] = scale_frag<QT>(Qp[qrow * p.sq[2] + KS * t + hf], p.scale);
      else qf[t] = scale_frag<QT>(ld16(Qp + qrow * p.sq[2] + KS * t + KW * hf), p.scale);
    } else {
      qf[t] = QFrag{};
    }
  }
  if constexpr (RP > 0) {
    const PT* prow = PQp + (int64_t)(qvalid ? qrow : 0) * p.spq[2];
#pragma unroll
    for (int t = 0; t < PSTEPS; ++t) {
      const int c0 = KS * t + KW * hf;
      if constexpr (KW == 1) {
        pf[t] = (qvalid && c0 < p.R) ? prow[c0] : 0.f;
      } else {
        pf[t] = qvalid ? load_phi_chunk<PT>(prow, c0, p.R, p.phq_vec) : u32x4{};
      }
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int kend = p.causal ? min(N, q0 + BM) : N;
  const int nkt = (kend + BN - 1) / BN;

  // ---- cooperative tile loads: global -> registers -> LDS ------------------
  u32x4 kr[KPT], vr[KPT];
  u32x4 pr[PPT > 0 ? PPT : 1];

  auto load_tile = [&](int kb) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if ((BN * KCH) % NT == 0 || c < BN * KCH) {
        const int row = c / KCH, col = c % KCH, key = kb + row;
        if (key < N) {
          kr[i] = ld16(Kp + (int64_t)key * p.sk[2] + col * CE);
          vr[i] = ld16(Vp + (int64_t)key * p.sv[2] + col * CE);
        } else {
          kr[i] = u32x4{};
          vr[i] = u32x4{};
        }
      }
    }
    if constexpr (PPT > 0) {
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int c = tid + i * NT;
        if ((BN * PCH) % NT == 0 || c < BN * PCH) {
          const int row = c / PCH, col = c % PCH, key = kb + row;
          pr[i] = key < N ? load_phi_chunk<PT>(PKp + (int64_t)key * p.spk[2], col * CE, p.R, p.phk_vec)
                          : u32x4{};
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if ((BN * KCH) % NT == 0 || c < BN * KCH) {
        const int row = c / KCH, col = c % KCH;
        st16(sK + perm_row(row) * PITCH_K + col * 16, kr[i]);
        // V goes in transposed: Vt[d][key]
        if constexpr (ES == 2) {
          const u16x8 e = __builtin_bit_cast(u16x8, vr[i]);
#pragma unroll
          for (int j = 0; j < CE; ++j)
            *(uint16_t*)(sV + perm_row(col * CE + j) * PITCH_V + row * ES) = e[j];
        } else {
#pragma unroll
          for (int j = 0; j < CE; ++j)
            *(uint32_t*)(sV + perm_row(col * CE + j) * PITCH_V + row * ES) = vr[i][j];
        }
      }
    }
    if constexpr (PPT > 0) {
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int c = tid + i * NT;
        if ((BN * PCH) % NT == 0 || c < BN * PCH) {
          const int row = c / PCH, col = c % PCH;
          st16(sK + perm_row(row) * PITCH_K + D * ES + col * 16, pr[i]);
        }
      }
    }
  };

  if (nkt > 0) {
    load_tile(0);
    store_tile();
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int kb = kt * BN;
    const bool has_next = kt + 1 < nkt;
    if (has_next) load_tile(kb + BN);

    // dense bias of this lane's row and keys kb + 32*kb2 + 16*hf + [0, 16)
    float bias_v[MODE == 1 ? 2 : 1][16];
    if constexpr (MODE == 1) {
      const BT* brow = Bp + (int64_t)(qvalid ? qrow : 0) * p.sb[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int j0 = kb + 32 * kb2 + 16 * hf;
        if (p.bias_vec && qvalid && j0 + 16 <= N) {
          constexpr int BCE = 16 / (int)sizeof(BT);
#pragma unroll
          for (int c = 0; c < 16 / BCE; ++c) {
            const ChunkV<BT> e = __builtin_bit_cast(ChunkV<BT>, ld16(brow + j0 + c * BCE));
#pragma unroll
            for (int j = 0; j < BCE; ++j) bias_v[kb2][c * BCE + j] = to_f32<BT>(e[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j)
            bias_v[kb2][j] = (qvalid && j0 + j < N) ? to_f32<BT>(brow[j0 + j]) : 0.f;
        }
      }
    }

    // A wavefront whose queries all precede this key tile has nothing to do here.
    const bool active = !p.causal || kb <= q0w + 31;
    if (active) {
      // ---- S^T = K' Q'^T for two 32-key blocks ----------------------------
      f32x16 sacc[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const unsigned char* arow = sK + (32 * kb2 + ln) * PITCH_K;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int t = 0; t < QSTEPS; ++t) {
          if constexpr (KW == 1) acc = Mma<QT>::run(*(const float*)(arow + (KS * t + hf) * ES), qf[t], acc);
          else acc = Mma<QT>::run(ld16(arow + (KS * t + KW * hf) * ES), qf[t], acc);
        }
        if constexpr (RP > 0) {
#pragma unroll
          for (int t = 0; t < PSTEPS; ++t) {
            if constexpr (KW == 1)
              acc = Mma<PT>::run(*(const float*)(arow + (D + KS * t + hf) * ES), pf[t], acc);
            else
              acc = Mma<PT>::run(ld16(arow + (D + KS * t + KW * hf) * ES), pf[t], acc);
          }
        }
        sacc[kb2] = acc;
      }
      if constexpr (MODE == 1) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb2][r] += bias_v[kb2][r];
      }
      // ---- mask: keys past N, and keys after the query when causal -----------
      const bool need_mask = (kb + BN > N) || (p.causal && kb + BN - 1 > q0w);
      if (need_mask) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kb + 32 * kb2 + 16 * hf + r;
            if (j >= N || (p.causal && j > qrow)) sacc[kb2][r] = -INFINITY;
          }
      }
      // ---- online softmax (row = this lane's query) ---------------------------
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * LOG2E);
      const float ms = m_use * LOG2E;
      float lsum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][r], LOG2E, -ms));
          sacc[kb2][r] = e;
          lsum += e;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

      // ---- O^T += Vt P^T ----------------------------------------------------
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        if constexpr (KW == 1) {
#pragma unroll
          for (int u = 0; u < 16; ++u) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const float a = *(const float*)(sV + (32 * db + ln) * PITCH_V + (32 * kb2 + 16 * hf + u) * ES);
              oacc[db] = Mma<QT>::run(a, sacc[kb2][u], oacc[db]);
            }
          }
        } else {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            typedef QT T8 __attribute__((ext_vector_type(8)));
            T8 pb;
#pragma unroll
            for (int j = 0; j < 8; ++j) pb[j] = from_f32<QT>(sacc[kb2][8 * u + j]);
            const u32x4 bfrag = __builtin_bit_cast(u32x4, pb);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const u32x4 a = ld16(sV + (32 * db + ln) * PITCH_V + (32 * kb2 + 16 * hf + 8 * u) * ES);
              oacc[db] = Mma<QT>::run(a, bfrag, oacc[db]);
            }
          }
        }
      }
    }

    __syncthreads();
    if (has_next) {
      store_tile();
      __syncthreads();
    }
  }

  // ---- epilogue: O = O / l, LSE = m + ln l -----------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qvalid) {
    const float inv = 1.f / l_tot;
    QT* orow = Op + (int64_t)qrow * p.so[2];
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
