// Internal declarations shared by the C-ABI layer and the HIP kernels of libflashbias.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fb.h"

namespace fb {

// Everything one fused attention launch needs (passed by value as the kernel argument).
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t sq[3], sk[3], sv[3], so[3];
  // low-rank factors (R columns, zero-padded to the template's RP)
  const void* phq;
  const void* phk;
  int64_t spq[3], spk[3];
  int R;
  int phq_vec, phk_vec;   // 1: rows are 16-byte aligned and R fills whole chunks -> vector loads
  // dense bias
  const void* bias;
  int64_t sb[3];
  int bias_vec;           // 1: rows 16-byte aligned -> vector loads
  int B, H, N;
  int causal;
  float scale;
  int nqb;                // number of query blocks per (b, h)
};

// Launch one fused attention forward for head dim 16/32/64/128.  mode 0: low-rank
// factors padded to RP columns (0 = plain attention); mode 1: dense bias (RP = 0).
// aux_dt is the factor or bias dtype.  FB_EUNSUPPORTED when no kernel instance matches.
fb_status launch_attention_d16(int mode, fb_dtype dt, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d32(int mode, fb_dtype dt, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d64(int mode, fb_dtype dt, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d128(int mode, fb_dtype dt, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);

// Exact closed-form factors / dense bias.  slopes_host: [H] (H <= kMaxSlopes) or NULL.
constexpr int kMaxSlopes = 256;
fb_status launch_make_factors(fb_bias_kind kind, int H, int N, int C, const double* slopes_host,
                              fb_dtype out_dt, int split, void* phq, void* phk, int R_pad, int R_nat,
                              hipStream_t stream);

fb_status launch_make_dense_bias(fb_bias_kind kind, int H, int N, int C, const double* slopes_host,
                                 fb_dtype out_dt, void* bias, int64_t head_stride, int64_t row_stride,
                                 hipStream_t stream);

void set_error(const char* fmt, ...);

}  // namespace fb
