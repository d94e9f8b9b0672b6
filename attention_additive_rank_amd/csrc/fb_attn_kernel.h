// Fused forward kernel for attention with an additive bias on gfx950 (CDNA4).
//
//   O = softmax(s Q K^T + b) V
//
// MODE 0 (low rank, FlashBias): b = phi_q phi_k^T is folded into one augmented
// contraction Q' = [Q*s, phi_q], K' = [K, phi_k] (FlashBias rebuttal, answer to
// Reviewer UJUf, Q2: concatenate the factor functions with queries and keys,
// then run FlashAttention).  MODE 1 (dense bias, the baseline): the contraction
// is Q*s K^T and a bias tile is read from HBM for every (query, key) tile pair,
// the quadratic IO of the abstract and Fig. 1(c).  MODE 2 and MODE 4 form the ALiBi and
// Sandwich factor columns inside the kernel; MODE 3 is MODE 0 with the scores in exp2 units.
//
// Work decomposition
//   * One workgroup = 8 wavefronts = 256 query rows of one (batch, head); each
//     wavefront owns 32 query rows for the whole key loop.  Waves w and w+4 run
//     on the same SIMD, so the two groups {0..3} and {4..7} pair up per SIMD.
//   * Per key tile each wavefront has a matrix phase (S(t+1) = K'(t+1) Q'^T and
//     O += V(t)^T P(t)^T on the MFMA units) and a vector phase (online softmax of
//     S(t+1)).  With loader wavefronts there is one workgroup barrier per tile:
//     group 0 runs matrix then softmax, group 1 softmax (at raised priority) then
//     matrix, so on every SIMD one wave's MFMAs overlap the other's softmax.
//     Without them the two groups run opposite phases between per-phase barriers.
//   * Non-causal kernels with narrow Q' can take several (b, h, query block) work
//     items per workgroup, one key-tile stream running across them.
//   * Key tiles of 64 keys are double-buffered in LDS (three stages with loader
//     wavefronts): K' rows (K then phi_k,
//     zero-padded to RP columns) and V rows, each region row-major with a
//     per-row XOR swizzle of its 16-byte chunks (conflict-free MFMA operand
//     reads, whole rows per copy).  Tiles arrive by direct global->LDS loads
//     (16 bytes per lane, no register round trip, no VALU), two tiles ahead for
//     K' and one for V; each load fills 1 KB of consecutive rows, so its lanes
//     read whole row segments.  For bf16/fp16 operands four more wavefronts
//     (one per SIMD) issue every copy, keeping the matrix and softmax waves
//     free of the address unit's stalls; otherwise the softmax phase issues
//     them.  Rows past N are not loaded and are masked in the scores.
//   * V stays row-major in LDS; the A operand of O^T = V^T P^T comes from
//     64-bit transpose reads (ds_read_b64_tr_b16), four keys per read.
//   * The softmax row sum (16-bit low-rank operands) is one more, 16x16x32 MFMA
//     per P V k-step with a ones / zeros A operand, so it costs matrix-core
//     cycles instead of VALU adds and is rescaled together with O.
//   * Scores are computed transposed, S^T = K' Q'^T, with 32x32 MFMAs
//     (32x32x16 bf16/f16, 32x32x2 fp32).  With that orientation every lane owns
//     ONE query (lane % 32) and 16 keys per 32-key block, so the row max / row
//     sum of the online softmax are in-lane reductions plus a single exchange
//     between the two half-waves, and P^T is already in the B-operand layout of
//     the next product O^T = V^T P^T: P never leaves registers.
//   * Lazy rescaling: the running row max only moves (and O, l are rescaled)
//     when a tile's max exceeds it by more than 2^8 in exp2 units, so most
//     tiles skip the O rescale; P then stays <= 2^8, exact in range for bf16.
//   * K' rows are permuted in LDS so that lane half h holds keys 16h..16h+15
//     of each 32-key block: bias reads and the causal mask touch contiguous runs.
//   * The factor columns of K' / Q' go through their own MFMA chain in the
//     factor dtype (PT), accumulating into the same fp32 score tile.
//   * Workgroup ids are remapped so that the query blocks of one (b, h) run on
//     one XCD (dispatch is round-robin over the 8 XCDs): their K'/V tiles are
//     then shared in that XCD's L2.  Causal launches take the longest query
//     blocks first, over the whole grid.
#pragma once

#include "fb_internal.h"
#include "fb_tile_map.h"

namespace fb {
namespace attn {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 8;          // wavefronts per workgroup: two groups of four
constexpr int NT = NW * 64;    // threads per workgroup
constexpr int GT = NT / 2;     // threads per group
constexpr int BM = 32 * NW;    // query rows per workgroup
constexpr int NLW = 4;         // loader wavefronts (kernels with a loader)
static_assert(BM == kAttnBlockM, "host and kernel block sizes differ");
constexpr int BN = 64;         // keys per LDS tile
constexpr int NKB = BN / 32;   // 32-key blocks per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_GAP = 8.0f / LOG2E;   // 2^8 in exp2 units, as a natural-log gap

// Kernels whose workgroups take several work items ((b, h, query block) triples) one after
// another, with one stream of key tiles across them and the next item's query rows loaded
// while the current item runs: non-causal 16-bit kernels with loader wavefronts (not the
// dense-bias mode) whose Q' fragments are narrow enough to hold the next item's as well
// (D + RP <= 80; the rest of the item switch spills a few registers there, outside the
// matrix and softmax phases).
constexpr bool attn_multi_item(int D, int RP, int MODE, bool loader, bool causal, int es) {
  return loader && !causal && es == 2 && MODE != 1 && D + RP <= 80;
}

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
// 16x16x32 MFMA (lane l: A row / B column l % 16, k elements 8 (l / 16) .. + 7; D column
// l % 16, rows 4 (l / 16) .. + 3)
template <typename T> struct Mma16;
template <> struct Mma16<bf16_t> {
  static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};
template <> struct Mma16<f16_t> {
  static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
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

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16 bytes global -> LDS without a register round trip: lane l of the wavefront writes
// lds_base + 16 * l (lds_base must be the same for the whole wavefront).
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  // The low 32 bits of a generic pointer into LDS are its LDS address (the shared aperture
  // sits in the high half); going through the integer avoids the generic-to-LDS null
  // check, which the compiler mis-encodes in some contexts.
  lds_void* dst = (lds_void*)(uint32_t)(uintptr_t)lds_base;
  __builtin_amdgcn_global_load_lds((global_void*)src, dst, 16, 0, 0);
}

// Workgroup barrier that orders LDS accesses only: outstanding global loads and stores
// (prefetches, output stores) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Scheduling-group pins of the matrix phase (see mma_phase): for group G, its MFMAs
// (MPV in a P V group, NKB in a score group), then the LDS reads of group G + 2
// (two transpose reads per head-dim block, or one 128-bit read per key block).
// 0x008 selects MFMA instructions and 0x100 LDS reads.
template <int G, int NG, int NPV, int DB, int NKB, int MPV>
__device__ __forceinline__ void mma_pins() {
  if constexpr (G < NG) {
    __builtin_amdgcn_sched_group_barrier(0x008, G < NPV ? MPV : NKB, 0);
    if constexpr (G + 2 < NG) __builtin_amdgcn_sched_group_barrier(0x100, G + 2 < NPV ? 2 * DB : NKB, 0);
    mma_pins<G + 1, NG, NPV, DB, NKB, MPV>();
  }
}

// (cos, sin) of 2 pi x nu for an integer 0 <= x < 2^16, with nu = n0 + n1 + n2 split on the
// host so that n0 and n1 have at most 8 significant bits: x n0 and x n1 are exact in fp32, so
// their fractional parts are exact, and x n2 is below 2^-8 of a revolution per 2^8 of x; the
// reduced angle (in revolutions, the unit of v_sin_f32 / v_cos_f32) is off by about 2^-24.
__device__ __forceinline__ void sincos_rev(int x, float n0, float n1, float n2, float& c, float& s) {
  const float xf = (float)x;
  const float a = __builtin_amdgcn_fractf(xf * n0);
  const float b = __builtin_amdgcn_fractf(xf * n1);
  const float r = __builtin_amdgcn_fractf(a + b + xf * n2);
  c = __builtin_amdgcn_cosf(r);
  s = __builtin_amdgcn_sinf(r);
}

// 64-bit transpose read of 16-bit elements (ds_read_b64_tr_b16): within each group of
// 16 lanes, value j of output lane 4a + c is element c of the 64-bit row read by lane 4j + a.
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// LOADER: NLW more wavefronts (one per SIMD) issue every tile copy (see the key loop).
// ITEMS: the instance that takes several work items per workgroup (attn_multi_item kernels
// launched with more items than compute units); the one-item instance has none of its code.
template <typename QT, typename PT, int D, int RP, int MODE, typename BT, bool CAUSAL, bool PHI_DMA, bool LOADER,
          bool ITEMS = false>
__global__ __launch_bounds__(LOADER ? NT + NLW * 64 : NT, 1) void attn_fwd_kernel(AttnParams p) {
  typedef typename Elem<QT>::Frag QFrag;
  typedef typename Elem<PT>::Frag PFrag;
  constexpr int ES = (int)sizeof(QT);
  static_assert(sizeof(PT) == sizeof(QT), "factor and query element sizes must match");
  static_assert(MODE != 1 || RP == 0, "dense-bias mode has no factor columns");
  // MODE 2: ALiBi with its factor columns formed in registers from the slope and the
  // query / key indices (the pages' in-kernel factor tiles, rebuttal answer to Reviewer
  // BRmd, Q2), one 16-wide f16 factor k-step, nothing read from memory for them
  constexpr bool JIT = MODE == 2;
  // MODE 3: low rank with phi_q given in exp2 units (phi_q log2(e), rounded once where the
  // factors are made; RP 0 is plain attention).  MODE 3 computes the scores in exp2 units
  // with the running max already subtracted: Q s is rounded as Q s log2(e), and every score
  // chain starts from an accumulator holding -M (M the running max in exp2 units), so the
  // softmax applies exp2 to the MFMA result directly, one vector operation per score fewer.
  // (Scaling general phi_q by log2(e) in the kernel would round it a second time and break
  // factors that are exact by construction, such as split pieces.)
  // MODE 4: Sandwich with its cos / sin factor columns formed in the kernel (the pages'
  // in-kernel factor tiles, rebuttal answers to Reviewer BRmd, Q2 and Reviewer UJUf, Q1):
  // phi_q in exp2 units (as MODE 3) from the query index at the start, and each key tile's
  // phi_k region written into LDS by the loader wavefronts instead of copied; nothing is read
  // from memory for the factors.
  constexpr bool SWJIT = MODE == 4;
  constexpr bool FOLD = Elem<QT>::KW > 1 && (MODE == 3 || MODE == 4);
  static_assert(!JIT || (RP == 16 && sizeof(QT) == 2 && __is_same(PT, f16_t)), "in-kernel factors: 16-bit, RP 16");
  static_assert(!SWJIT || (LOADER && sizeof(QT) == 2 && __is_same(PT, f16_t) && RP >= 16 && RP <= 64),
                "in-kernel Sandwich factors: 16-bit with loader wavefronts, RP 16..64");
  constexpr int KW = Elem<QT>::KW;        // k elements per lane per MFMA
  constexpr int KS = 2 * KW;              // k per MFMA
  constexpr int CE = 16 / ES;             // elements per 16-byte chunk
  constexpr int DP = D < 32 ? 32 : D;     // V width in LDS, at least one 32-wide MFMA block
  constexpr int DB = DP / 32;             // 32-wide head-dim blocks of the output
  constexpr int QSTEPS = D / KS;
  constexpr int PSTEPS = RP / KS;
  constexpr int KCH = D / CE;             // chunks per K row (and data chunks per V row)
  constexpr int PCH = JIT ? 0 : RP / CE;  // chunks per (padded) phi_k row in LDS
  constexpr int VCH = DP / CE;            // chunks per V row in LDS
  // A K' tile is two swizzled row-major regions, K (64 x KCH chunks) then phi_k
  // (64 x PCH chunks), a V tile one region of 64 x VCH chunks; row = key, and chunk c of
  // key row r sits at position c ^ swz_key(r) (K, phi_k) or c ^ swz_quad(r) (V).  The
  // score MFMA reads key inv_perm_row(ln) in lane ln of a 32-key block, so that lane
  // half h of the scores holds keys 16h..16h+15.
  constexpr int KREG = BN * KCH * 16;
  constexpr int SK_BYTES = KREG + BN * PCH * 16;
  constexpr int SV_BYTES = BN * VCH * 16;
  // Tile copies: one direct load fills 1 KB = 64 consecutive chunk slots of a region
  // (whole rows), so its 64 lanes read whole row segments from global memory.
  constexpr int NDMA = KCH + PCH + VCH;   // loads per tile: K, phi_k, V
  constexpr int DPW = (NDMA + NW - 1) / NW;   // loads per compute wavefront and tile
  static_assert(BN == 64 && BN == kAttnKeyTile, "one direct load per 1 KB of a 64-row tile");
  static_assert(D % KS == 0 && RP % KS == 0 && D % CE == 0 && RP % CE == 0, "bad tile widths");
  static_assert(KW > 1 || (D % 8 == 0 && RP % 8 == 0), "fp32 k order pairs chunks");
  static_assert((KCH & (KCH - 1)) == 0 && (PCH & (PCH - 1)) == 0 && (VCH & (VCH - 1)) == 0 && VCH >= 4,
                "tile rows must be a power-of-two number of chunks");

  // Two stages of K' and V tiles (three with loader wavefronts), the key loop unrolled by the
  // stage count: every access names its buffer statically, so the compiler can tell that a
  // direct load in flight never writes the buffer being read, and does not wait for it.
  __shared__ __attribute__((aligned(16))) unsigned char sK0[SK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sK1[SK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sV0[SV_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sV1[SV_BYTES];
  // third stage of the loader pipeline
  __shared__ __attribute__((aligned(16))) unsigned char sK2[LOADER ? SK_BYTES : 16];
  __shared__ __attribute__((aligned(16))) unsigned char sV2[LOADER ? SV_BYTES : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;     // waves w and w+4 share a SIMD: one of each group per SIMD
  const int ln = lane & 31;
  const int hf = lane >> 5;

  // ---- workgroup -> (query block, head, batch), XCD-aware -------------------
  const int G = (int)gridDim.x;
  const int wg = (int)blockIdx.x;
  const int xcd = wg & 7, idx = wg >> 3;
  const int per = G >> 3, rem = G & 7;
  const int L = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  // work items: (b, h, query block), query block fastest; this workgroup takes items
  // item0 .. item0 + nitems - 1 (one item unless MULTI)
  constexpr bool MULTI = ITEMS && attn_multi_item(D, RP, MODE, LOADER, CAUSAL, ES);
  int item0 = L, nitems = 1;
  if constexpr (MULTI) {
    item0 = L * p.ipw;
    nitems = min(p.ipw, p.n_items - item0);
  }
  int qb = item0 % p.nqb;
  int bh = item0 / p.nqb;
  if (CAUSAL) {
    // longest first over the whole grid (dispatch order): all last query blocks, then the
    // ones before; (b, h) fastest, so with B H a multiple of 8 each (b, h) stays on one
    // XCD (hardware id mod 8) at every level
    const int BH = p.B * p.H;
    qb = p.nqb - 1 - wg / BH;
    bh = wg % BH;
  }
  int hh = bh % p.H;
  int bb = bh / p.H;
  const int N = p.N;

  const QT* Qp = (const QT*)p.q + ((int64_t)bb * p.sq[0] + (int64_t)hh * p.sq[1]);
  const QT* Kp = (const QT*)p.k + ((int64_t)bb * p.sk[0] + (int64_t)hh * p.sk[1]);
  const QT* Vp = (const QT*)p.v + ((int64_t)bb * p.sv[0] + (int64_t)hh * p.sv[1]);
  QT* Op = (QT*)p.o + ((int64_t)bb * p.so[0] + (int64_t)hh * p.so[1]);
  const PT* PQp = nullptr;
  const PT* PKp = nullptr;
  if constexpr (RP > 0 && !JIT) {
    PQp = (const PT*)p.phq + ((int64_t)bb * p.spq[0] + (int64_t)hh * p.spq[1]);
    PKp = (const PT*)p.phk + ((int64_t)bb * p.spk[0] + (int64_t)hh * p.spk[1]);
  }
  const BT* Bp = nullptr;
  if constexpr (MODE == 1) Bp = (const BT*)p.bias + ((int64_t)bb * p.sb[0] + (int64_t)hh * p.sb[1]);

  int q0 = qb * BM;
  const int kend = CAUSAL ? min(N, q0 + BM) : N;   // (MULTI: not causal, the same for every item)
  const int nkt = (kend + BN - 1) / BN;
  // the workgroup's key tiles in order: tile t of item i is step i nkt + t
  const int nsteps = nitems * nkt;

  // ---- tile copies -----------------------------------------------------------------
  // Load n of a tile: n < KCH fills K-region bytes [1024 n, 1024 (n+1)), then the
  // phi_k region, then V.  Lane l of a load writes chunk slot l of its 1 KB: row
  // n' (64 / cpr) + l / cpr, chunk position l % cpr, i.e. logical chunk (l % cpr) ^ swz(row).
  // One load thus reads 1 KB of consecutive rows from global memory (the concurrent
  // workgroups of a head read the same tiles: scattered rows there cost L2 throughput).
  // Without loader wavefronts, chunks that are never loaded (phi_k at or beyond R, V past
  // D) hold zeros; the loader wavefronts copy in-row stand-ins there (loader_src_byte).
  // With PHI_DMA false (phi_k rows not 16-byte loadable: unaligned, or R not a multiple of
  // a chunk) the phi_k region is staged through registers instead (phi_load / phi_store).
  constexpr bool phk_fast = PHI_DMA;
  const int npch = phk_fast ? p.R / CE : 0;     // phi_k chunks that the direct path loads
  auto slot_of = [&](int n) __attribute__((always_inline)) { return tile_slot(n, lane, KCH, PCH, VCH); };
  // source byte offset of this lane's chunk of load n relative to the tile's first row, ~0
  // for a chunk that is not loaded
  auto src_offset = [&](int n) __attribute__((always_inline)) {
    const TileSlot d = slot_of(n);
    const int stride = d.region == 0 ? p.sk[2] : d.region == 1 ? p.spk[2] : p.sv[2];
    return slot_has_data(d, KCH, npch) ? (uint32_t)(d.row * (stride * ES) + d.c * 16) : ~0u;
  };
  // issue load n of K'(kbk) (into dK) or V(kbv) (into dV), given its offset; rows past N
  // are not loaded (their scores are masked; V rows keep finite data)
  auto dma_load = [&](int n, uint32_t off, int kbk, int kbv, unsigned char* dK, unsigned char* dV) __attribute__((always_inline)) {
    const int region = n < KCH ? 0 : n < KCH + PCH ? 1 : 2;
    const int kb = region == 2 ? kbv : kbk;
    const char* base = region == 0 ? (const char*)(Kp + (int64_t)kb * p.sk[2])
                     : region == 1 ? (const char*)(PKp + (int64_t)kb * p.spk[2])
                                   : (const char*)(Vp + (int64_t)kb * p.sv[2]);
    unsigned char* dst = region == 2 ? dV + (n - KCH - PCH) * 1024 : dK + n * 1024;
    bool ok = off != ~0u;
    if (kb + BN > N) {
      const TileSlot d = slot_of(n);
      ok = ok && d.row < N - kb;
    }
    if (ok) dma16(base + off, dst);
  };
  // Chunks that are never loaded must hold finite values: the V buffers start zeroed (a
  // first tile may have rows past N) and so do the phi_k chunks at or beyond R.  (The
  // loader wavefronts fill every chunk slot instead.)
  if constexpr (!LOADER) {
#pragma unroll
    for (int i = 0; i < (SV_BYTES / 16 + NT - 1) / NT; ++i) {
      const int s = tid + NT * i;
      if (s < SV_BYTES / 16) {
        st16(sV0 + 16 * s, u32x4{0, 0, 0, 0});
        st16(sV1 + 16 * s, u32x4{0, 0, 0, 0});
      }
    }
  }
  if constexpr (RP > 0 && !LOADER) {
    for (int s = tid; s < BN * PCH; s += NT) {
      const int r = s / PCH, c = s % PCH;
      if (c >= npch) {
        const int o = KREG + (r * PCH + (c ^ swz_key(PCH, r))) * 16;
        st16(sK0 + o, u32x4{0, 0, 0, 0});
        st16(sK1 + o, u32x4{0, 0, 0, 0});
      }
    }
  }
  __syncthreads();   // the zero fills land before any direct load into those buffers

  // ---- the loader wavefronts ------------------------------------------------------
  // A direct load holds the wavefront that issues it until the address unit takes it.
  // With LOADER, NLW more wavefronts (one per SIMD, doing nothing else) issue them all,
  // so no compute wavefront stalls on them, into three stages of K' and V buffers.  They
  // keep the compute wavefronts' barrier sequence: two prologue barriers, then per tile t
  // the barrier that ends phase A and the one that ends phase B (group 0's MFMA / group
  // 1's softmax, then the reverse), and the final one.  During tile t they copy K'(t+3)
  // into K'(t)'s buffer and V(t+2) into V(t-1)'s, half of each wavefront's share in each
  // phase; before the barrier that ends tile t they wait only for the copies issued
  // before tile t (K'(t+2), V(t+1), needed from tile t+1 on), so copies stay in flight
  // across barriers instead of draining every tile.  That wait counts this wavefront's
  // outstanding loads, so every load is issued with all lanes active: a lane whose chunk
  // is not wanted copies a finite stand-in from inside the tensor: for a row past N the
  // last row's chunk (the scores mask it), for a phi_k chunk at or beyond R or a V chunk
  // past D (VCH > KCH when D < 32) the row's first chunk (it meets zero phi_q columns, or
  // feeds only head dims >= D, which are never stored).
  if constexpr (LOADER) {
    static_assert(PHI_DMA, "the loaders copy phi_k directly");
    if (wave >= NW) {
      // loads m = 0 .. NLD-1 of a tile, tile load n_of(m) (MODE 4 skips the phi_k region)
      constexpr int NLD = NDMA - (SWJIT ? PCH : 0);
      constexpr int PER = (NLD + NLW - 1) / NLW;    // most loads per loader wavefront and tile
      constexpr int PMIN = NLD / NLW;               // fewest
      static_assert(PMIN >= 1 && PMIN <= 15, "loads per wavefront and tile");
      auto n_of = [&](int m) __attribute__((always_inline)) { return SWJIT && m >= KCH ? m + PCH : m; };
      const int lw = wave - NW;
      int rowi[PER], cbyte[PER];
      uint32_t off[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int n = n_of(lw + NLW * i);
        rowi[i] = cbyte[i] = 0;
        off[i] = 0;
        if (lw + NLW * i < NLD) {
          const TileSlot d = slot_of(n);
          rowi[i] = d.row;
          cbyte[i] = loader_src_byte(d, KCH, npch);
          const int stride = d.region == 0 ? p.sk[2] : d.region == 1 ? p.spk[2] : p.sv[2];
          off[i] = (uint32_t)(d.row * stride * ES + cbyte[i]);
        }
      }
      // Source of step vv of the workgroup's tile stream: the first rows of its K, phi_k and
      // V tiles and its first key.  Steps past the last are replaced by the last one (their
      // copies land in buffers that nothing reads again).
      struct Src {
        const char* k;
        const char* pk;
        const char* v;
        int kb;
      };
      auto src_of = [&](int vv) __attribute__((always_inline)) {
        vv = min(vv, nsteps - 1);
        Src r;
        if constexpr (MULTI) {
          const int it = vv / nkt;
          r.kb = (vv - it * nkt) * BN;
          const int bhi = (item0 + it) / p.nqb;
          const int64_t b = bhi / p.H, h = bhi % p.H;
          r.k = (const char*)((const QT*)p.k + (b * p.sk[0] + h * p.sk[1] + (int64_t)r.kb * p.sk[2]));
          r.v = (const char*)((const QT*)p.v + (b * p.sv[0] + h * p.sv[1] + (int64_t)r.kb * p.sv[2]));
          r.pk = nullptr;
          if constexpr (RP > 0 && !JIT)
            r.pk = (const char*)((const PT*)p.phk + (b * p.spk[0] + h * p.spk[1] + (int64_t)r.kb * p.spk[2]));
        } else {
          r.kb = vv * BN;
          r.k = (const char*)(Kp + (int64_t)r.kb * p.sk[2]);
          r.pk = (const char*)(PKp + (int64_t)r.kb * p.spk[2]);
          r.v = (const char*)(Vp + (int64_t)r.kb * p.sv[2]);
        }
        return r;
      };
      // loads [i0, i1) of this wavefront for K' of stream step vk into dK and V of step vv
      // into dV
      auto loads = [&](int i0, int i1, int vk, int vv, unsigned char* dK, unsigned char* dV, bool do_k, bool do_v)
          __attribute__((always_inline)) {
        const Src sk = src_of(vk), sv = src_of(vv);
#pragma unroll
        for (int i = i0; i < i1; ++i) {
          const int n = n_of(lw + NLW * i);
          const int region = n < KCH ? 0 : n < KCH + PCH ? 1 : 2;
          if (lw + NLW * i < NLD && (region == 2 ? do_v : do_k)) {
            const int kb = region == 2 ? sv.kb : sk.kb;
            const int stride = region == 0 ? p.sk[2] : region == 1 ? p.spk[2] : p.sv[2];
            const char* base = region == 0 ? sk.k : region == 1 ? sk.pk : sv.v;
            unsigned char* dst = region == 2 ? dV + (n - KCH - PCH) * 1024 : dK + n * 1024;
            uint32_t o = off[i];
            if (kb + BN > N) o = (uint32_t)(min(rowi[i], N - 1 - kb) * stride * ES + cbyte[i]);
            dma16(base + o, dst);
          }
        }
      };
      // MODE 4: the phi_k region of each tile, [cos(j w_f), sin(j w_f)] in f16 for the 64 keys j
      // of the tile and the RP / 2 column pairs f (zero past the C / 2 frequencies).  Loader lane
      // g = 64 lw + lane owns pair f = g % NPAIR of the rows g / NPAIR + RSTEP m.  With the tile's
      // first key kb, cos / sin (kb + r) w = rotation of (cos r w, sin r w) by kb w: the offsets r
      // are evaluated once (fp32, exact revolution reduction), the rotation by kb w advances by 64 w
      // per tile in fp64 (rotation of 64 w from the host in fp64), so no error builds up.
      constexpr int NPAIR = SWJIT ? RP / 2 : 4;
      constexpr int RSTEP = NLW * 64 / NPAIR;
      constexpr int NROW = 64 / RSTEP;
      double bc = 1.0, bs = 0.0, rc = 1.0, rs = 0.0;
      float tc[NROW], ts[NROW];
      uint32_t woff[NROW];
      if constexpr (SWJIT) {
        const int g = lw * 64 + lane;
        const int f = g % NPAIR;
        const bool live = f < p.sw_pairs;
        rc = live ? p.sw_rot[0][f] : 1.0;
        rs = live ? p.sw_rot[1][f] : 0.0;
#pragma unroll
        for (int m = 0; m < NROW; ++m) {
          const int r = g / NPAIR + RSTEP * m;
          sincos_rev(r, p.sw_nu[0][f], p.sw_nu[1][f], p.sw_nu[2][f], tc[m], ts[m]);
          tc[m] *= live ? 1.f : 0.f;
          ts[m] *= live ? 1.f : 0.f;
          woff[m] = KREG + r * PCH * 16 + 16 * ((f >> 2) ^ swz_key(PCH, r)) + 4 * (f & 3);
        }
      }
      // phi_k of stream step vv (generated in stream order; each item's keys start at 0)
      auto gen_phk = [&](unsigned char* dK, int vv) __attribute__((always_inline)) {
        if constexpr (SWJIT) {
          if (MULTI && vv < nsteps && vv % nkt == 0) {
            bc = 1.0;
            bs = 0.0;
          }
          const float c = (float)bc, sn = (float)bs;
#pragma unroll
          for (int m = 0; m < NROW; ++m) {
            const f16x2 v = {(f16_t)(c * tc[m] - sn * ts[m]), (f16_t)(sn * tc[m] + c * ts[m])};
            *(uint32_t*)(dK + woff[m]) = __builtin_bit_cast(uint32_t, v);
          }
          const double nc = bc * rc - bs * rs;
          bs = bs * rc + bc * rs;
          bc = nc;
        }
      };
      gen_phk(sK0, 0);
      gen_phk(sK1, 1);
      loads(0, PER, 0, 0, sK0, sV0, true, true);          // K'(0), V(0)
      loads(0, PER, 1, 0, sK1, sV0, true, false);         // K'(1)
      __syncthreads();                                    // (waits for them)
      gen_phk(sK2, 2);
      loads(0, PER, 2, 1, sK2, sV1, true, true);          // K'(2), V(1)
      __builtin_amdgcn_s_barrier();
      // one barrier per tile (see the key loop of the compute wavefronts)
      auto lstep = [&](int t, unsigned char* kd, unsigned char* vd) __attribute__((always_inline)) {
        gen_phk(kd, t + 3);
        loads(0, PER, t + 3, t + 2, kd, vd, true, true);
        // vmcnt(PMIN): at most PMIN loads outstanding, so all of the previous tile's are done;
        // MODE 4 also waits for its LDS writes (lgkmcnt(0))
        __builtin_amdgcn_s_waitcnt(PMIN | (SWJIT ? 0x0070 : 0x0F70));
        __builtin_amdgcn_s_barrier();
      };
      for (int t = 0; t < nsteps; t += 3) {
        lstep(t, sK0, sV2);
        if (t + 1 < nsteps) lstep(t + 1, sK1, sV0);
        if (t + 2 < nsteps) lstep(t + 2, sK2, sV1);
      }
      __builtin_amdgcn_s_waitcnt(0);   // no copy outlives the workgroup
      __builtin_amdgcn_s_barrier();
      return;
    }
  }

  // this wavefront's query rows of the current item
  int q0w = q0 + wave * 32;
  int qrow = q0w + ln;
  bool qvalid = qrow < N;
  int qclamp = qvalid ? qrow : N - 1;

  // ---- Q' fragments (B operand of S^T = K' Q'^T), resident for the whole loop
  // 16-bit: k-step t of lane half h covers chunk 2t + h.  fp32 (one element per lane and
  // k-step): k-step t of half h takes element t % 4 of chunk 2 (t / 4) + h, i.e.
  // column 8 (t / 4) + 4 h + t % 4, so one 128-bit read of K' serves four k-steps.
  QFrag qf[QSTEPS];
  PFrag pf[PSTEPS > 0 ? PSTEPS : 1];
  auto col32 = [&](int t) __attribute__((always_inline)) { return 8 * (t >> 2) + 4 * hf + (t & 3); };
#pragma unroll
  for (int t = 0; t < QSTEPS; ++t) {
    if constexpr (KW == 1) qf[t] = scale_frag<QT>(Qp[qclamp * p.sq[2] + col32(t)], p.scale);
    else qf[t] = scale_frag<QT>(ld16(Qp + qclamp * p.sq[2] + KS * t + KW * hf), FOLD ? p.scale * LOG2E : p.scale);
  }
  // In-kernel ALiBi factors: with the slope m = m_hi + m_lo (two f16) and an index
  // x = x_hi + x_lo (x_hi a multiple of 2048, both exact in f16),
  //   phi_q(i) = [m_hi, m_hi, m_lo, m_lo, -i_hi, -i_lo, -i_hi, -i_lo, 0 ...],
  //   phi_k(j) = [j_hi, j_lo, j_hi, j_lo,  m_hi,  m_hi,  m_lo,  m_lo, 0 ...]:
  // every product is exact in fp32 and their sum is m (j - i) to the 22 bits of m.
  // Lane half 1 holds k = 8..15: zeros.
  f16_t jm_hi = (f16_t)0.f, jm_lo = (f16_t)0.f;
  auto set_slope = [&](int h) __attribute__((always_inline)) {
    if constexpr (JIT) {
      const uint32_t mb = p.alibi_m[h];
      jm_hi = __builtin_bit_cast(f16_t, (uint16_t)(mb & 0xffffu));
      jm_lo = __builtin_bit_cast(f16_t, (uint16_t)(mb >> 16));
    }
  };
  set_slope(hh);
  auto jit_pair = [&](int x) __attribute__((always_inline)) {
    f16x2 r = {(f16_t)(float)(x & ~2047), (f16_t)(float)(x & 2047)};
    return r;
  };
  auto jit_phk = [&](int j) __attribute__((always_inline)) {
    const f16x2 jx = jit_pair(j);
    const f16x8 v = {jx[0], jx[1], jx[0], jx[1], jm_hi, jm_hi, jm_lo, jm_lo};
    const u32x4 r = __builtin_bit_cast(u32x4, v);
    return hf ? u32x4{0u, 0u, 0u, 0u} : r;
  };
  // phi_q fragments formed in the kernel (in-kernel factor modes) for query row qc
  auto make_pf = [&](int qc) __attribute__((always_inline)) {
    if constexpr (SWJIT) {
      // phi_q(i) in exp2 units: lane half h of k-step t holds column pairs f = 8t + 4h + e (e < 4)
      // of the query row, [cos(i w_f), sin(i w_f)] log2(e), zero past the C / 2 frequencies
#pragma unroll
      for (int t = 0; t < PSTEPS; ++t) {
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int f = 8 * t + 4 * hf + e;
          float c, sn;
          sincos_rev(qc, p.sw_nu[0][f], p.sw_nu[1][f], p.sw_nu[2][f], c, sn);
          const float w = f < p.sw_pairs ? LOG2E : 0.f;
          v[2 * e] = (f16_t)(c * w);
          v[2 * e + 1] = (f16_t)(sn * w);
        }
        pf[t] = __builtin_bit_cast(u32x4, v);
      }
    } else if constexpr (JIT) {
      const f16x2 ix = jit_pair(qc);
      const f16x8 v = {jm_hi, jm_hi, jm_lo, jm_lo, (f16_t)(-(float)ix[0]), (f16_t)(-(float)ix[1]),
                       (f16_t)(-(float)ix[0]), (f16_t)(-(float)ix[1])};
      pf[0] = hf ? u32x4{0u, 0u, 0u, 0u} : __builtin_bit_cast(u32x4, v);
    }
  };
  make_pf(qclamp);
  if constexpr (RP > 0 && !JIT && !SWJIT) {
    const PT* prow = PQp + qclamp * p.spq[2];
#pragma unroll
    for (int t = 0; t < PSTEPS; ++t) {
      if constexpr (KW == 1) {
        const int c = col32(t);
        pf[t] = c < p.R ? prow[c] : 0.f;
      } else {
        const int c0 = KS * t + KW * hf;
        pf[t] = load_phi_chunk<PT>(prow, c0, p.R, (p.flags & FLAG_PHQ_VEC) && c0 + KW <= p.R);
      }
    }
  }

  // ---- MULTI: the next work item ----------------------------------------------------
  // Its Q' (and phi_q) rows are loaded into qnx / pnx as soon as the current item starts and
  // become the fragments at the step whose score MFMAs first need them.
  int cur = item0;     // current item
  int vbase = 0;       // its first stream step
  u32x4 qnx[MULTI ? QSTEPS : 1];
  PFrag pnx[MULTI && RP > 0 && !JIT && !SWJIT ? PSTEPS : 1];
  struct ItemRows {
    int b, h, q0, qc;
  };
  auto item_rows = [&](int item) __attribute__((always_inline)) {
    ItemRows r;
    const int bhi = item / p.nqb;
    r.q0 = (item - bhi * p.nqb) * BM;
    r.h = bhi % p.H;
    r.b = bhi / p.H;
    r.qc = min(r.q0 + wave * 32 + ln, N - 1);
    return r;
  };
  auto prefetch_q = [&](int item) __attribute__((always_inline)) {
    if constexpr (MULTI) {
      const ItemRows r = item_rows(item);
      const QT* qp = (const QT*)p.q + ((int64_t)r.b * p.sq[0] + (int64_t)r.h * p.sq[1] + (int64_t)r.qc * p.sq[2]);
#pragma unroll
      for (int t = 0; t < QSTEPS; ++t) qnx[t] = ld16(qp + KS * t + KW * hf);
      if constexpr (RP > 0 && !JIT && !SWJIT) {
        const PT* pr =
            (const PT*)p.phq + ((int64_t)r.b * p.spq[0] + (int64_t)r.h * p.spq[1] + (int64_t)r.qc * p.spq[2]);
#pragma unroll
        for (int t = 0; t < PSTEPS; ++t) {
          const int c0 = KS * t + KW * hf;
          pnx[t] = load_phi_chunk<PT>(pr, c0, p.R, (p.flags & FLAG_PHQ_VEC) && c0 + KW <= p.R);
        }
      }
    }
  };
  if (MULTI && nitems > 1) prefetch_q(item0 + 1);

  // tile copies by the compute wavefronts (no loader): wavefront w issues loads w, w+8, ...
  uint32_t coff[LOADER ? 1 : DPW];
  if constexpr (!LOADER) {
#pragma unroll
    for (int i = 0; i < DPW; ++i) coff[i] = wave + NW * i < NDMA ? src_offset(wave + NW * i) : ~0u;
  }
  auto dma_tile = [&](int kbk, int kbv, unsigned char* dK, unsigned char* dV, bool do_k, bool do_v) __attribute__((always_inline)) {
    if constexpr (!LOADER) {
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int n = wave + NW * i;
        const bool is_k = n < KCH + PCH;
        if (n < NDMA && (is_k ? do_k : do_v)) dma_load(n, coff[i], kbk, kbv, dK, dV);
      }
    }
  };
  // phi_k region through registers (PHI_DMA false): group 1 loads and stores tile t+3
  // during its softmax(t+1).  Chunk s of a tile: row s / PCH, logical chunk s % PCH, zero
  // beyond R.
  constexpr int NPS = (BN * (PCH > 0 ? PCH : 1) + GT - 1) / GT;
  u32x4 phreg[NPS];
  const int gtid = tid & (GT - 1);
  auto phi_load = [&](int kb) __attribute__((always_inline)) {
    if constexpr (PCH > 0 && !phk_fast) {
#pragma unroll
      for (int i = 0; i < NPS; ++i) {
        int s = gtid + GT * i;
        // opaque to loop-invariant code motion: otherwise every element offset of the
        // chunk is precomputed and held in registers for the whole key loop
        asm volatile("" : "+v"(s));
        if (s < BN * PCH) {
          const int key = min(kb + s / PCH, N - 1);
          phreg[i] = load_partial_chunk<PT>(PKp + key * p.spk[2], (s % PCH) * CE, p.R);
        }
      }
    }
  };
  auto phi_store = [&](unsigned char* dK) __attribute__((always_inline)) {
    if constexpr (PCH > 0 && !phk_fast) {
#pragma unroll
      for (int i = 0; i < NPS; ++i) {
        const int s = gtid + GT * i;
        const int r = s / PCH, c = s % PCH;
        if (s < BN * PCH) st16(dK + KREG + (r * PCH + (c ^ swz_key(PCH, r))) * 16, phreg[i]);
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
  float l_run = 0.f;      // row sum (vector-unit path)
  float M2 = 0.f;                 // FOLD: running max in exp2 units
  // Low-rank mode, 16-bit: the row sum of P rides on the matrix core as one 16x16x32 MFMA
  // per P V k-step (32 keys of P's B-operand registers read as 16 columns x 32 k), lacc +=
  // A P: lane l of the B operand holds query row l % 32 (keys of lane half l / 32), i.e.
  // column l % 16 and k group l / 16 there; A is 1 where the k group's parity equals the
  // parity of the row's quad ((row / 4) % 2), 0 elsewhere, so D rows 4g..4g+3 of column c,
  // which lane 16 g + c holds, sum the k groups of g's parity: query row 16 (g % 2) + c,
  // the lane's own row (l % 32).  Every register of lacc thus holds the lane's row sum in
  // both halves, and the rescaling of O scales it with the lane's own factor.  This takes
  // 36 adds per tile off the vector unit for 8 registers (lacc, A) and 4 MFMAs per tile, each
  // half the size of a P V MFMA.  (Dense-bias mode keeps the adds: its bias registers leave
  // no room.)
  constexpr bool MROW = KW > 1 && MODE != 1;
  // FOLD: every score chain starts from -M2 in all 16 registers, kept as a copy (minit,
  // rewritten only when M2 moves) instead of 16 moves into the accumulator when each chain
  // starts: the softmax phase is the longer one on narrow heads and in the causal kernel.
  // Multi-item instances with D + RP > 48 write it into the accumulator instead: with the
  // next item's fragments the copy does not fit in their registers.
  constexpr bool MINIT = FOLD && !(MULTI && D + RP > 48);
  f32x16 minit = f32x16{};
  auto chain_init = [&]() __attribute__((always_inline)) {
    if constexpr (MINIT) {
      return minit;
    } else {
      f32x16 c = f32x16{};
      if constexpr (FOLD) {
#pragma unroll
        for (int r = 0; r < 16; ++r) c[r] = -M2;
      }
      return c;
    }
  };
  f32x4 lacc = f32x4{};
  const uint32_t one2 = __is_same(QT, bf16_t) ? 0x3F803F80u : 0x3C003C00u;   // two 1.0 values of QT
  const u32x4 ones = (((lane >> 2) ^ (lane >> 4)) & 1) == 0 ? u32x4{one2, one2, one2, one2} : u32x4{0u, 0u, 0u, 0u};

  // dense bias of this lane's row, keys kb + 32*kb2 + 16*hf + [0, 16), loaded one tile ahead
  constexpr int BES = MODE == 1 ? (int)sizeof(BT) : 2;
  constexpr int BCH = BES;                  // 16-byte chunks per 16 keys
  constexpr int NBR = MODE == 1 ? NKB * BCH : 1;
  u32x4 braw[NBR];
  auto load_bias = [&](int kb) __attribute__((always_inline)) {
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
  auto active = [&](int t) __attribute__((always_inline)) { return !CAUSAL || t * BN <= q0w + 31; };

  // ---- LDS operand addresses ------------------------------------------------------
  // Score MFMA operand of k-step t (fp32: of 4-step group t), key block kb2: key row
  // 32 kb2 + inv_perm_row(ln), logical chunk c = 2t + hf of the K region (or of the phi_k
  // region for the factor steps).  The row swizzle depends on ln only and flips the low
  // three bits of c (four with 16-chunk rows), so per lane there are four (eight)
  // distinct addresses, t mod 4 (8); the rest is an immediate.
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
  // P V operand (16-bit), key block kb2, k-step u, head-dim block db: two transpose reads,
  // rows 32 kb2 + 16 hf + 8 u + 4 q + jj (q = 0, 1), where lane 4 jj + a of a 16-lane group
  // g reads head dims 32 db + 16 (g & 1) + 4 a .. + 3: logical chunk
  // 4 db + 2 (g & 1) + (a >> 1), byte 8 (a & 1).  The quad swizzle of those rows depends on
  // jj only, so per lane there are two addresses (db even / odd).  Value j of output lane
  // 4 a + c of a transpose read is element c of lane 4 j + a's row: head dim
  // 32 db + lane % 32 for four consecutive keys.
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
  // fp32 P V operand: V[32 kb2 + 16 hf + u][32 db + ln]; the quad swizzle of row u depends
  // on u mod 4.
  int vf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * hf + j;
    vf[j] = r * VCH * 16 + 16 * ((ln >> 2) ^ swz_quad(VCH, r)) + 4 * (ln & 3);
  }

  // factor-chain A operand of k-step t, key block kb2, of the tile whose first key is kbt
  auto phik = [&](const unsigned char* sKt, int kbt, int t, int kb2) __attribute__((always_inline)) {
    if constexpr (JIT) return jit_phk(kbt + 32 * kb2 + inv_perm_row(ln));
    else return kread(sKt, true, t, kb2);
  };

  // S^T = K'(t) Q'^T from the K' tile at sKt (first key kbt)
  auto qk = [&](const unsigned char* sKt, int kbt) __attribute__((always_inline)) {
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = chain_init();
    if constexpr (KW == 1) {
#pragma unroll
      for (int t4 = 0; t4 < QSTEPS / 4; ++t4)
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
          const f32x4 a = __builtin_bit_cast(f32x4, kread(sKt, false, t4, kb2));
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[kb2] = Mma<QT>::run(a[e], qf[4 * t4 + e], sacc[kb2]);
        }
#pragma unroll
      for (int t4 = 0; t4 < PSTEPS / 4; ++t4)
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
          const f32x4 a = __builtin_bit_cast(f32x4, kread(sKt, true, t4, kb2));
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[kb2] = Mma<PT>::run(a[e], pf[4 * t4 + e], sacc[kb2]);
        }
    } else {
#pragma unroll
      for (int t = 0; t < QSTEPS; ++t)
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = Mma<QT>::run(kread(sKt, false, t, kb2), qf[t], sacc[kb2]);
#pragma unroll
      for (int t = 0; t < PSTEPS; ++t)
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = Mma<PT>::run(phik(sKt, kbt, t, kb2), pf[t], sacc[kb2]);
    }
  };

  // O^T += V(t)^T P(t)^T from the V tile at sVt.  MFMA row m of head-dim block db is head
  // dim 32 db + m; k-slot j of lane half h in k-step u of key block kb2 is key
  // 32 kb2 + 16 h + 8 u + j, matching the registers of P.
  auto pv = [&](const unsigned char* sVt) __attribute__((always_inline)) {
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) {
      if constexpr (KW == 1) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const float a = *(const float*)(sVt + vf[u & 3] + (32 * kb2 + (u & ~3)) * VCH * 16 + 128 * db);
            oacc[db] = Mma<QT>::run(a, p32[kb2][u], oacc[db]);
          }
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] = Mma<QT>::run(vread_tr(sVt, kb2, u, db), pfrag[kb2 * 2 + u], oacc[db]);
          if constexpr (MROW) lacc = Mma16<QT>::run(ones, pfrag[kb2 * 2 + u], lacc);
        }
      }
    }
  };


  // The whole matrix phase of a non-causal 16-bit tile in one scheduling region:
  // O += V(t)^T P(t)^T first (P dies, its registers take the new scores), then
  // S(t+1) = K'(t+1) Q'^T.  Operands are read two MFMA groups ahead of their use
  // (group = the MFMAs of one k-step), so the LDS latency hides behind the matrix
  // core instead of stalling it; the scheduling-group pins below keep that order.
  auto mma_phase = [&](const unsigned char* sKn, int kbn, const unsigned char* sVt) __attribute__((always_inline)) {
    if constexpr (KW > 1) {
      constexpr int NPV = NKB * 2;              // P V groups (kb2, u): 2 DB reads, DB (+1) MFMAs
      constexpr int NQK = QSTEPS + PSTEPS;      // score groups: NKB reads + NKB MFMAs
      constexpr int NG = NPV + NQK;
      u32x4 opnd[NG][NKB > DB ? NKB : DB];
      auto issue = [&](int g) __attribute__((always_inline)) {
        if (g < NPV) {
#pragma unroll
          for (int db = 0; db < DB; ++db) opnd[g][db] = vread_tr(sVt, g >> 1, g & 1, db);
        } else {
          const int t = g - NPV;
#pragma unroll
          for (int kb2 = 0; kb2 < NKB; ++kb2)
            opnd[g][kb2] = t < QSTEPS ? kread(sKn, false, t, kb2) : phik(sKn, kbn, t - QSTEPS, kb2);
        }
      };
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = chain_init();
      issue(0);
      issue(1);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g + 2 < NG) issue(g + 2);
        if (g < NPV) {
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] = Mma<QT>::run(opnd[g][db], pfrag[g], oacc[db]);
          if constexpr (MROW) lacc = Mma16<QT>::run(ones, pfrag[g], lacc);
        } else {
          const int t = g - NPV;
#pragma unroll
          for (int kb2 = 0; kb2 < NKB; ++kb2)
            sacc[kb2] = t < QSTEPS ? Mma<QT>::run(opnd[g][kb2], qf[t], sacc[kb2])
                                   : Mma<PT>::run(opnd[g][kb2], pf[t - QSTEPS], sacc[kb2]);
        }
      }
      // pins: reads of groups 0 and 1; then per group g its MFMAs and the reads of g + 2
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);
      mma_pins<0, NG, NPV, DB, NKB, DB + (MROW ? 1 : 0)>();
    }
  };

  // online softmax of tile t (scores in sacc) -> P(t); lazy rescaling of O and l
  auto softmax = [&](int t) __attribute__((always_inline)) {
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
        const int jb = kb + 32 * kb2;   // first key of the block (uniform)
        if (CAUSAL && (jb >= N || jb > q0w + 31)) {
          // every key of the block is past N or after every query of the wavefront
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb2][r] = -INFINITY;
        } else if (!CAUSAL || jb + 32 > N || jb + 31 > q0w) {
          const int j0 = jb + 16 * hf;
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
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
    mx = halves_max(mx);
    if constexpr (FOLD) {
      // scores are S log2(e) - M2; the first tile sets M2 to its max (key 0 is always
      // visible, so that max is finite), later tiles move it when they exceed it by 8
      const bool first = t == 0;
      const bool grow = first || mx > 8.f;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float d = grow ? mx : 0.f;
        if (!first) {
          const float alpha = __builtin_amdgcn_exp2f(-d);
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
          if constexpr (MROW)
            lacc *= alpha;
          else
            l_run *= alpha;
        }
        M2 += d;
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] -= d;
        if constexpr (MINIT) {
#pragma unroll
          for (int r = 0; r < 16; ++r) minit[r] = -M2;
        }
      }
      typedef QT T8 __attribute__((ext_vector_type(8)));
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          T8 pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float e = __builtin_amdgcn_exp2f(sacc[kb2][8 * u + j]);
            pb[j] = from_f32<QT>(e);
            if constexpr (!MROW) ls[j & 3] += e;
          }
          pfrag[kb2 * 2 + u] = __builtin_bit_cast(u32x4, pb);
        }
      if constexpr (!MROW) l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
      return;
    }
    const bool grow = mx > m_run + RESCALE_GAP;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - mx) * LOG2E) : 1.f;  // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      if constexpr (MROW) lacc *= alpha;
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
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          T8 pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][8 * u + j], LOG2E, -ms));
            pb[j] = from_f32<QT>(e);
            if constexpr (!MROW) l_run += e;
          }
          pfrag[kb2 * 2 + u] = __builtin_bit_cast(u32x4, pb);
        }
    }
  };

  // ---- prologue: K'(0), K'(1), V(0) in LDS; P(0) ------------------------------
  dma_tile(0, 0, sK0, sV0, true, true);
  dma_tile(BN, BN, sK1, sV1, nkt > 1, false);
  if (!phk_fast && grp == 1) {
    phi_load(0);
    phi_store(sK0);
    if (nkt > 1) {
      phi_load(BN);
      phi_store(sK1);
    }
  }
  load_bias(0);
  __syncthreads();
  qk(sK0, 0);
  softmax(0);
  __syncthreads();

  // ---- one item's epilogue: O = O / l, LSE = m + ln l ------------------------------
  auto store_item = [&]() __attribute__((always_inline)) {
    // register r of lane half hf in head-dim block db holds head dim 32 db + 8 (r / 4) + 4 hf + r % 4
    // (every register of lacc holds the lane's row sum, in both halves)
    const float l_tot = MROW ? lacc[0] : halves_sum(l_run);
    if (qvalid) {
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
            for (int j = 0; j < 4; ++j) v[j] = from_f32<QT>(oacc[db][4 * c + j] * inv);
            *(T4*)(orow + d0) = v;
          }
        }
      if (p.lse && hf == 0)
        p.lse[((int64_t)bb * p.H + hh) * N + qrow] = FOLD ? (M2 + __log2f(l_tot)) * LN2 : m_run + logf(l_tot);
    }
  };
  // MULTI: the next item's fragments, before the MFMA phase whose score MFMAs use them
  auto next_frags = [&]() __attribute__((always_inline)) {
    if constexpr (MULTI) {
      const ItemRows r = item_rows(cur + 1);
#pragma unroll
      for (int t = 0; t < QSTEPS; ++t) qf[t] = scale_frag<QT>(qnx[t], FOLD ? p.scale * LOG2E : p.scale);
      set_slope(r.h);
      make_pf(r.qc);
      if constexpr (RP > 0 && !JIT && !SWJIT) {
#pragma unroll
        for (int t = 0; t < PSTEPS; ++t) pf[t] = pnx[t];
      }
    }
  };
  // MULTI: after the current item's epilogue, the next item becomes the current one
  auto next_item = [&]() __attribute__((always_inline)) {
    if constexpr (MULTI) {
      ++cur;
      vbase += nkt;
      const ItemRows r = item_rows(cur);
      bb = r.b;
      hh = r.h;
      q0 = r.q0;
      q0w = q0 + wave * 32;
      qrow = q0w + ln;
      qvalid = qrow < N;
      qclamp = qvalid ? qrow : N - 1;
      Op = (QT*)p.o + ((int64_t)bb * p.so[0] + (int64_t)hh * p.so[1]);
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
      lacc = f32x4{};
      l_run = 0.f;
      m_run = -INFINITY;
      if (cur + 1 < item0 + nitems) prefetch_q(cur + 1);
    }
  };

  // ---- the key loop: per SIMD, one wavefront multiplies while the other does softmax ----
  // Every wavefront runs the same sequence  MFMA(t) | softmax(t+1) | MFMA(t+1) | ...  with
  // MFMA(t) = {S(t+1) = K'(t+1) Q'^T, O += V(t)^T P(t)}.  With loader wavefronts: one
  // barrier per tile (see step).  Without: one phase per barrier, group 1 starting one phase
  // late, so on each SIMD the two wavefronts are always in opposite phases.  (One code path
  // for both groups: branching on the group around the accumulators makes the compiler copy
  // them at every join.)
  // Without loader wavefronts the tile copies go out from the softmax phases, which read
  // nothing from LDS (the compiler cannot order LDS reads after an outstanding direct load
  // by the counter, and would wait for all of them), split between the groups: group 0,
  // in its softmax(t+1) (tile t's second phase), issues its loads of K'(t+2) and V(t+1)
  // into the buffers that tile t-1 released; group 1, in its softmax(t+1) (tile t+1's
  // first phase), its loads of K'(t+3) and V(t+2), into the buffers that K'(t+1) and V(t)
  // have just released.  The barrier that closes each softmax phase waits for them.  With
  // phi_k staged through registers, group 1 also loads and stores the phi_k region of
  // tile t+3 there.
  // kt / kn: K' buffers of tiles t / t+1; vt / vn: V buffers of tiles t / t+1.
  auto step = [&](int t, unsigned char* kt, unsigned char* kn, unsigned char* vt,
                  unsigned char* vn) __attribute__((always_inline)) {
    const int kb = t * BN;
    if constexpr (LOADER) {
      // One barrier per tile: group 0 runs MFMA(t) then softmax(t+1), group 1 the same
      // sequence with its barrier between them, i.e. softmax(t) then MFMA(t) within a tile.
      // Each wavefront goes on to its next phase as soon as its own work allows, so one
      // wavefront's matrix work overlaps the other's softmax without either waiting at a
      // barrier for the other's phase to end.  Both groups read K'(t+1) and V(t) in tile t;
      // the loaders overwrite those buffers only after the barrier that ends it.  Group 1's
      // softmax, which opens the tile and is followed by its MFMA phase, issues at a raised
      // wavefront priority: group 0's softmax, which closes the tile, would otherwise take
      // the vector unit from it where they overlap (the older wavefront wins the issue).
      // MULTI: at the last step of an item the score MFMAs already work on the first tile
      // of the next item (its fragments are swapped in first), then the item is stored.
      const int tt = t - vbase;          // tile of the current item
      const bool last = tt == nkt - 1;
      const bool more = MULTI && last && t + 1 < nsteps;
      const int tn = last ? 0 : tt + 1;  // tile whose scores the MFMA phase computes
      if (more) next_frags();
      mma_phase(kn, tn * BN, vt);
      if (more) {
        store_item();
        next_item();
      }
      if (grp == 1) lds_barrier();
      if (grp == 1) __builtin_amdgcn_s_setprio(2);
      if (!last || more) softmax(tn);
      __builtin_amdgcn_s_setprio(0);
      if (grp == 0) lds_barrier();
      return;
    }
    if constexpr (KW > 1) {
      // past the last tile the scores of a stale buffer are computed and never used.
      // Causal: also the tiles past a wavefront's queries (near the diagonal) go through
      // the same fused phase, with all-masked scores and P = 0: one code path (a second
      // one costs registers) and no time lost, as the ping-pong keeps the wavefronts of
      // a workgroup in step anyway.
      mma_phase(kn, kb + BN, vt);
    } else {
      if (t + 1 < nkt && active(t + 1)) qk(kn, kb + BN);
      if (active(t)) pv(vt);
    }
    __builtin_amdgcn_s_barrier();
    if constexpr (!LOADER) {
      const int kbk = kb + (2 + grp) * BN, kbv = kb + (1 + grp) * BN;
      dma_tile(kbk, kbv, grp ? kn : kt, grp ? vt : vn, kbk < nkt * BN, kbv < nkt * BN);
    }
    if (!phk_fast && grp == 1 && t + 3 < nkt) phi_load(kb + 3 * BN);
    if (t + 1 < nkt && (KW > 1 || active(t + 1))) softmax(t + 1);
    if (!phk_fast && grp == 1 && t + 3 < nkt) phi_store(kn);
    __syncthreads();
  };
  if (!LOADER && grp == 1) {
    // group 1's first phase: its loads of K'(2) (into K'(0)'s buffer, free now) and V(1),
    // and the phi_k region of tile 2
    dma_tile(2 * BN, BN, sK0, sV1, 2 < nkt, 1 < nkt);
    if (!phk_fast && nkt > 2) {
      phi_load(2 * BN);
      phi_store(sK0);
    }
    __syncthreads();
  }
  if constexpr (LOADER) {
    for (int t = 0; t < nsteps; t += 3) {
      step(t, sK0, sK1, sV0, sV1);
      if (t + 1 < nsteps) step(t + 1, sK1, sK2, sV1, sV2);
      if (t + 2 < nsteps) step(t + 2, sK2, sK0, sV2, sV0);
    }
  } else {
    for (int t = 0; t < nkt; t += 2) {
      step(t, sK0, sK1, sV0, sV1);
      if (t + 1 < nkt) step(t + 1, sK1, sK0, sV1, sV0);
    }
  }
  // matches group 1's extra first phase (with loader wavefronts: their final barrier)
  if (LOADER || grp == 0) __builtin_amdgcn_s_barrier();

  // ---- epilogue: O = O / l, LSE = m + ln l -----------------------------------
  store_item();
}

}  // namespace attn
}  // namespace fb
