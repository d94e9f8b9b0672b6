// Kernel instances of the fused attention forward for one head dimension.
// This file is compiled once per head dimension with -DFB_ATTN_D=<16|32|64|128>
// so that the instances build in parallel.
#include "fb_attn_kernel.h"

#ifndef FB_ATTN_D
#error "compile with -DFB_ATTN_D=<head dim>"
#endif

namespace fb {
namespace attn {

template <typename QT, typename PT, int D, int RP, int MODE, typename BT>
static fb_status launch_one(const AttnParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.nqb * p.H * p.B;
  hipLaunchKernelGGL((attn_fwd_kernel<QT, PT, D, RP, MODE, BT>), dim3((unsigned)grid), dim3(NT), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention launch failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

template <typename QT, typename PT, int D>
static fb_status lowrank_rp(int RP, const AttnParams& p, hipStream_t s) {
  if constexpr (sizeof(QT) == 2) {
    switch (RP) {
      case 16: return launch_one<QT, PT, D, 16, 0, QT>(p, s);
      case 32: return launch_one<QT, PT, D, 32, 0, QT>(p, s);
      case 64: return launch_one<QT, PT, D, 64, 0, QT>(p, s);
      case 128: return launch_one<QT, PT, D, 128, 0, QT>(p, s);
    }
  } else {
    switch (RP) {
      case 4: return launch_one<QT, PT, D, 4, 0, QT>(p, s);
      case 8: return launch_one<QT, PT, D, 8, 0, QT>(p, s);
      case 16: return launch_one<QT, PT, D, 16, 0, QT>(p, s);
      case 32: return launch_one<QT, PT, D, 32, 0, QT>(p, s);
    }
  }
  return FB_EUNSUPPORTED;
}

}  // namespace attn

#define FB_CAT2(a, b) a##b
#define FB_CAT(a, b) FB_CAT2(a, b)

// mode 0: low rank (RP = padded factor width, 0 = plain attention); mode 1: dense bias.
fb_status FB_CAT(launch_attention_d, FB_ATTN_D)(int mode, fb_dtype dt, fb_dtype aux_dt, int RP,
                                                 const AttnParams& p, hipStream_t s) {
  using namespace attn;
  constexpr int D = FB_ATTN_D;
  if (mode == 1) {
    if (dt == FB_BF16 && aux_dt == FB_BF16) return launch_one<bf16_t, bf16_t, D, 0, 1, bf16_t>(p, s);
    if (dt == FB_F16 && aux_dt == FB_F16) return launch_one<f16_t, f16_t, D, 0, 1, f16_t>(p, s);
    if (dt == FB_F32 && aux_dt == FB_F32) return launch_one<float, float, D, 0, 1, float>(p, s);
    return FB_EUNSUPPORTED;
  }
  if (RP == 0) {
    if (dt == FB_BF16) return launch_one<bf16_t, bf16_t, D, 0, 0, bf16_t>(p, s);
    if (dt == FB_F16) return launch_one<f16_t, f16_t, D, 0, 0, f16_t>(p, s);
    if (dt == FB_F32) return launch_one<float, float, D, 0, 0, float>(p, s);
    return FB_EUNSUPPORTED;
  }
  if (dt == FB_BF16 && aux_dt == FB_BF16) return lowrank_rp<bf16_t, bf16_t, D>(RP, p, s);
  if (dt == FB_BF16 && aux_dt == FB_F16) return lowrank_rp<bf16_t, f16_t, D>(RP, p, s);
  if (dt == FB_F16 && aux_dt == FB_F16) return lowrank_rp<f16_t, f16_t, D>(RP, p, s);
  if (dt == FB_F32 && aux_dt == FB_F32) return lowrank_rp<float, float, D>(RP, p, s);
  return FB_EUNSUPPORTED;
}

}  // namespace fb
