// Kernel instances of the fused attention forward for one head dimension and one
// Q/K/V element type.  Compiled once per (head dim, type) pair with
// -DFB_ATTN_D=<16|32|64|128> -DFB_ATTN_QT=<0 bf16 | 1 f16 | 2 fp32> so that the
// instances build in parallel.
#include "fb_attn_resident.h"

#include <cstdlib>

#if !defined(FB_ATTN_D) || !defined(FB_ATTN_QT)
#error "compile with -DFB_ATTN_D=<head dim> -DFB_ATTN_QT=<0|1|2>"
#endif

namespace fb {
namespace attn {

// FB_ATTN_STREAMING=1 in the environment turns the resident-K'/V kernel off (the streaming
// kernel then takes every launch), for comparisons; read at every launch
static bool resident_allowed() {
  const char* e = std::getenv("FB_ATTN_STREAMING");
  return !(e && e[0] == '1');
}

template <typename QT, typename PT, int D, int RP, int MODE, typename BT, bool PHI_DMA>
static fb_status launch_kernel(const AttnParams& p, hipStream_t stream) {
  // loader wavefronts where their register budget (three wavefronts on one SIMD) holds
  constexpr bool LOADER = PHI_DMA && sizeof(QT) == 2 && D <= 64 && RP <= 64 && (MODE != 1 || sizeof(BT) == 2);
  const bool causal = (p.flags & FLAG_CAUSAL) != 0;
  // short non-causal sequences in exp2 units: the whole K' and V of a (b, h) in LDS, one
  // workgroup per (b, h), no barrier in the key loop (fb_attn_resident.h); narrow Q' only
  // (D + RP <= 48: two query blocks per wavefront and one step's operands fit 256 registers)
  if constexpr (MODE == 3 && sizeof(QT) == 2 && PHI_DMA && D + RP <= 48) {
    if (!causal && p.N <= res_max_keys(D, RP) && resident_allowed()) {
      const int64_t grid = (int64_t)p.B * p.H;
      hipLaunchKernelGGL((attn_fwd_res_kernel<QT, PT, D, RP>), dim3((unsigned)grid), dim3(RNT), 0, stream, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) {
        set_error("attention launch failed: %s", hipGetErrorString(e));
        return FB_EHIP;
      }
      return FB_OK;
    }
  }
  // work items (b, h, query block); with more items than compute units, kernels that can
  // take several items per workgroup get one workgroup per compute unit (ceil(items / CUs)
  // items each: the same number of item-times as one item per workgroup, without a
  // workgroup start and end per item)
  AttnParams q = p;
  const int64_t items = (int64_t)p.nqb * p.H * p.B;
  q.n_items = (int)items;
  q.ipw = 1;
  if (!causal && attn_multi_item(D, RP, MODE, LOADER, false, (int)sizeof(QT))) {
    const int ncu = device_cu_count();
    if (ncu > 0 && items > ncu) q.ipw = (int)((items + ncu - 1) / ncu);
  }
  const int64_t grid = (items + q.ipw - 1) / q.ipw;
  const dim3 block(LOADER ? NT + NLW * 64 : NT);
  if (causal)
    hipLaunchKernelGGL((attn_fwd_kernel<QT, PT, D, RP, MODE, BT, true, PHI_DMA, LOADER>), dim3((unsigned)grid), block, 0,
                       stream, q);
  else if (q.ipw > 1) {
    if constexpr (attn_multi_item(D, RP, MODE, LOADER, false, (int)sizeof(QT)))
      hipLaunchKernelGGL((attn_fwd_kernel<QT, PT, D, RP, MODE, BT, false, PHI_DMA, LOADER, true>), dim3((unsigned)grid),
                         block, 0, stream, q);
  } else
    hipLaunchKernelGGL((attn_fwd_kernel<QT, PT, D, RP, MODE, BT, false, PHI_DMA, LOADER>), dim3((unsigned)grid), block, 0,
                       stream, q);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention launch failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

// phi_k goes to LDS by direct 16-byte loads when its rows are 16-byte aligned and R is a
// multiple of a chunk; otherwise through registers.
template <typename QT, typename PT, int D, int RP, int MODE, typename BT>
static fb_status launch_one(const AttnParams& p, hipStream_t stream) {
  if constexpr (RP > 0) {
    constexpr int CE = 16 / (int)sizeof(PT);
    if (!((p.flags & FLAG_PHK_VEC) && p.R % CE == 0))
      return launch_kernel<QT, PT, D, RP, MODE, BT, false>(p, stream);
  }
  return launch_kernel<QT, PT, D, RP, MODE, BT, true>(p, stream);
}

template <typename QT, typename PT, int D, int MODE = 0>
static fb_status lowrank_rp(int RP, const AttnParams& p, hipStream_t s) {
  if constexpr (sizeof(QT) == 2) {
    switch (RP) {
      case 16: return launch_one<QT, PT, D, 16, MODE, QT>(p, s);
      case 32: return launch_one<QT, PT, D, 32, MODE, QT>(p, s);
      case 64: return launch_one<QT, PT, D, 64, MODE, QT>(p, s);
      case 128: return launch_one<QT, PT, D, 128, MODE, QT>(p, s);
    }
  } else if constexpr (MODE == 0) {
    switch (RP) {
      case 8: return launch_one<QT, PT, D, 8, 0, QT>(p, s);
      case 16: return launch_one<QT, PT, D, 16, 0, QT>(p, s);
      case 32: return launch_one<QT, PT, D, 32, 0, QT>(p, s);
    }
  }
  return FB_EUNSUPPORTED;
}

}  // namespace attn

#define FB_CAT3_(a, b, c) a##b##c
#define FB_CAT3(a, b, c) FB_CAT3_(a, b, c)
#if FB_ATTN_QT == 0
#define FB_QT_NAME _bf16
#elif FB_ATTN_QT == 1
#define FB_QT_NAME _f16
#else
#define FB_QT_NAME _f32
#endif

// mode 0: low rank (RP = padded factor width, 0 = plain attention); mode 1: dense bias;
// mode 2: ALiBi with in-kernel factors (16-bit Q/K/V); mode 3: low rank with phi_q in
// exp2 units (16-bit Q/K/V); mode 4: Sandwich with in-kernel factors in exp2 units
// (16-bit Q/K/V, D <= 64, RP = C rounded up to 16 <= 64).
fb_status FB_CAT3(launch_attention_d, FB_ATTN_D, FB_QT_NAME)(int mode, fb_dtype aux_dt, int RP,
                                                              const AttnParams& p, hipStream_t s) {
  using namespace attn;
  constexpr int D = FB_ATTN_D;
#if FB_ATTN_QT == 2 && FB_ATTN_D > 64
  // fp32 Q/K/V is limited to head dims <= 64 (the fp32 matrix-core path is for small checks)
  (void)mode; (void)aux_dt; (void)RP; (void)p; (void)s;
  return FB_EUNSUPPORTED;
#else
#if FB_ATTN_QT == 0
  typedef bf16_t QT;
  constexpr fb_dtype qdt = FB_BF16;
#elif FB_ATTN_QT == 1
  typedef f16_t QT;
  constexpr fb_dtype qdt = FB_F16;
#else
  typedef float QT;
  constexpr fb_dtype qdt = FB_F32;
#endif
  if (mode == 1) {
    if (aux_dt == qdt) return launch_one<QT, QT, D, 0, 1, QT>(p, s);
    return FB_EUNSUPPORTED;
  }
  if (mode == 2) {
#if FB_ATTN_QT != 2
    return launch_kernel<QT, f16_t, D, 16, 2, QT, true>(p, s);
#else
    return FB_EUNSUPPORTED;
#endif
  }
#if FB_ATTN_QT != 2
  if (mode == 3 && RP == 0) return launch_one<QT, QT, D, 0, 3, QT>(p, s);
  if (mode == 4) {
    // in-kernel Sandwich factors: the loader wavefronts write the phi_k tiles (D <= 64)
    if constexpr (D <= 64) {
      switch (RP) {
        case 16: return launch_kernel<QT, f16_t, D, 16, 4, QT, true>(p, s);
        case 32: return launch_kernel<QT, f16_t, D, 32, 4, QT, true>(p, s);
        case 64: return launch_kernel<QT, f16_t, D, 64, 4, QT, true>(p, s);
      }
    }
    return FB_EUNSUPPORTED;
  }
#endif
  if (RP == 0) return launch_one<QT, QT, D, 0, 0, QT>(p, s);
#if FB_ATTN_QT != 2
  if (mode == 3) {
#if FB_ATTN_QT == 0
    if (aux_dt == FB_BF16) return lowrank_rp<QT, bf16_t, D, 3>(RP, p, s);
#endif
    if (aux_dt == FB_F16) return lowrank_rp<QT, f16_t, D, 3>(RP, p, s);
    return FB_EUNSUPPORTED;
  }
#endif
#if FB_ATTN_QT == 0
  if (aux_dt == FB_BF16) return lowrank_rp<QT, bf16_t, D>(RP, p, s);
  if (aux_dt == FB_F16) return lowrank_rp<QT, f16_t, D>(RP, p, s);
#else
  if (aux_dt == qdt) return lowrank_rp<QT, QT, D>(RP, p, s);
#endif
  return FB_EUNSUPPORTED;
#endif
}

}  // namespace fb
