// Backward kernel instances for one head dimension (compiled with -DFB_BWD_D=<16|32|64|128>):
// bf16 / f16 operands, factor width RP in {0, 16, 32, 64}, causal or not.
#include "fb_attn_bwd.h"

#ifndef FB_BWD_D
#error "compile with -DFB_BWD_D=<head dim>"
#endif

namespace fb {
namespace attnb {

// head dim 16 runs in the head-dim-32 layout with the columns past 16 as zero operands
constexpr int KD = FB_BWD_D < 32 ? 32 : FB_BWD_D;

template <typename QT, typename PT, int RP, bool CAUSAL, bool LOG2>
static fb_status launch3(const BwdParams& p, hipStream_t s) {
  const int64_t grid = (int64_t)p.nblk * p.H * p.B;
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<QT, PT, KD, RP, CAUSAL, FB_BWD_D, LOG2>), dim3((unsigned)grid), dim3(BTH), 0,
                     s, p);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<QT, PT, KD, RP, CAUSAL, FB_BWD_D, LOG2>), dim3((unsigned)grid), dim3(BTH), 0,
                     s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention backward launch failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

// phi_q in exp2 units (FLAG_LOG2) only with factors
template <typename QT, typename PT, int RP, bool CAUSAL>
static fb_status launch2(const BwdParams& p, hipStream_t s) {
  if constexpr (RP > 0)
    if (p.flags & FLAG_LOG2) return launch3<QT, PT, RP, CAUSAL, true>(p, s);
  return launch3<QT, PT, RP, CAUSAL, false>(p, s);
}

template <typename QT, typename PT, int RP>
static fb_status launch_c(const BwdParams& p, hipStream_t s) {
  return (p.flags & FLAG_CAUSAL) ? launch2<QT, PT, RP, true>(p, s) : launch2<QT, PT, RP, false>(p, s);
}

template <typename QT, typename PT>
static fb_status launch_rp(int RP, const BwdParams& p, hipStream_t s) {
  switch (RP) {
    case 0: return launch_c<QT, QT, 0>(p, s);
    case 16: return launch_c<QT, PT, 16>(p, s);
    case 32: return launch_c<QT, PT, 32>(p, s);
    case 64: return launch_c<QT, PT, 64>(p, s);
  }
  return FB_EUNSUPPORTED;
}

}  // namespace attnb

#define FB_CAT2_(a, b) a##b
#define FB_CAT2(a, b) FB_CAT2_(a, b)

fb_status FB_CAT2(launch_attention_bwd_d, FB_BWD_D)(fb_dtype dt, fb_dtype phi_dt, int RP, const BwdParams& p,
                                                     hipStream_t s) {
  using namespace attnb;
  if (dt == FB_BF16) {
    if (RP == 0 || phi_dt == FB_BF16) return launch_rp<bf16_t, bf16_t>(RP, p, s);
    if (phi_dt == FB_F16) return launch_rp<bf16_t, f16_t>(RP, p, s);
  } else if (dt == FB_F16) {
    if (RP == 0 || phi_dt == FB_F16) return launch_rp<f16_t, f16_t>(RP, p, s);
  }
  return FB_EUNSUPPORTED;
}

}  // namespace fb
