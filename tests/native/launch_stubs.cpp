// Host-only stand-ins for the kernel launchers of libflashbias, for the CPU build of the C-ABI
// layer (fb_abi.cpp) and the host SVD (fb_svd.cpp) under AddressSanitizer / UBSan: every
// launcher reports FB_EUNSUPPORTED.  The sanitizer driver only takes paths that end before a
// launch (argument validation, workspace sizes, the host SVD).
#include "fb_internal.h"

namespace fb {
#define FB_STUB_ATTN(name) \
  fb_status name(int, fb_dtype, int, const AttnParams&, hipStream_t) { return FB_EUNSUPPORTED; }
FB_STUB_ATTN(launch_attention_d16_bf16)
FB_STUB_ATTN(launch_attention_d16_f16)
FB_STUB_ATTN(launch_attention_d16_f32)
FB_STUB_ATTN(launch_attention_d32_bf16)
FB_STUB_ATTN(launch_attention_d32_f16)
FB_STUB_ATTN(launch_attention_d32_f32)
FB_STUB_ATTN(launch_attention_d64_bf16)
FB_STUB_ATTN(launch_attention_d64_f16)
FB_STUB_ATTN(launch_attention_d64_f32)
FB_STUB_ATTN(launch_attention_d128_bf16)
FB_STUB_ATTN(launch_attention_d128_f16)
FB_STUB_ATTN(launch_attention_d128_f32)
#undef FB_STUB_ATTN

fb_status launch_make_factors(fb_bias_kind, int, int, int, const double*, fb_dtype, int, void*, void*, int, int, double,
                              hipStream_t) {
  return FB_EUNSUPPORTED;
}
fb_status launch_make_dense_bias(fb_bias_kind, int, int, int, const double*, fb_dtype, void*, int64_t, int64_t,
                                 hipStream_t) {
  return FB_EUNSUPPORTED;
}
fb_status launch_mulbias_expand(fb_dtype, fb_dtype, const void*, const int64_t[3], const void*, const int64_t[3], int,
                                int, int, int, int, float, void*, void*, hipStream_t) {
  return FB_EUNSUPPORTED;
}
fb_status launch_attention_bwd_d16(fb_dtype, fb_dtype, int, const BwdParams&, hipStream_t) { return FB_EUNSUPPORTED; }
fb_status launch_attention_bwd_d32(fb_dtype, fb_dtype, int, const BwdParams&, hipStream_t) { return FB_EUNSUPPORTED; }
fb_status launch_attention_bwd_d64(fb_dtype, fb_dtype, int, const BwdParams&, hipStream_t) { return FB_EUNSUPPORTED; }
fb_status launch_attention_bwd_d128(fb_dtype, fb_dtype, int, const BwdParams&, hipStream_t) { return FB_EUNSUPPORTED; }
fb_status launch_attention_bwd_delta(fb_dtype, const void*, const int64_t[3], const void*, const int64_t[3], int, int,
                                     int, int, float*, hipStream_t) {
  return FB_EUNSUPPORTED;
}
fb_status launch_attention_bwd_reduce(const float*, int, int, int, int, float*, const int64_t[3], hipStream_t) {
  return FB_EUNSUPPORTED;
}
fb_status launch_attention_bwd_pad_factor(const void*, int, const int64_t[3], int, int, int, int, int, void*,
                                          hipStream_t) {
  return FB_EUNSUPPORTED;
}
fb_status launch_attention_bwd_delta_f32(const void*, const int64_t[3], const void*, const int64_t[3], int, int, int, int,
                                         float*, hipStream_t) {
  return FB_EUNSUPPORTED;
}
fb_status launch_attention_bwd_f32(const BwdParams&, int, hipStream_t) { return FB_EUNSUPPORTED; }
fb_status launch_attention_bwd_unpad(const float*, int, int, int, int, int, float*, const int64_t[3], hipStream_t) {
  return FB_EUNSUPPORTED;
}
}  // namespace fb
