// Internal declarations shared by the C-ABI layer and the HIP kernels of libflashbias.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fb.h"

namespace fb {

// Everything one fused attention launch needs (passed by value as the kernel argument).
// Strides are in elements and fit in 32 bits (checked by the C-ABI layer); the
// per-(batch, head) base offsets are formed in 64 bits inside the kernel.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const void* phq;        // low-rank factors (R columns, zero-padded to the template's RP)
  const void* phk;
  const void* bias;       // dense bias
  int sq[3], sk[3], sv[3], so[3];
  int spq[3], spk[3];
  int sb[3];
  int R;
  int flags;              // FLAG_* below
  int B, H, N;
  float scale;
  int nqb;                // number of query blocks per (b, h)
  // in-kernel ALiBi factors (mode 2): slope of head h as two f16 values, bits
  // m_hi | m_lo << 16 with m_hi + m_lo = m_h to 22 bits
  uint32_t alibi_m[128];
  // in-kernel Sandwich factors (mode 4): C / 2 frequencies w_f; nu_f = w_f / (2 pi) as three
  // fp32 pieces (the first two with at most 8 significant bits), and the rotation by 64 w_f
  // (cos, sin) in fp64; sw_pairs = C / 2
  float sw_nu[3][32];
  double sw_rot[2][32];
  int sw_pairs;
  // work items (b, h, query block), query block fastest: ipw consecutive items per
  // workgroup (instances with attn_multi_item only; 1 otherwise), n_items in all
  int ipw;
  int n_items;
};
constexpr int kMaxSandwichPairs = 32;
// compute units of the calling thread's current device (cached per device); 0 on error
int device_cu_count();
constexpr int kMaxJitHeads = 128;
constexpr int kAttnBlockM = 256;   // query rows per attention workgroup
constexpr int kAttnKeyTile = 64;   // keys per LDS tile of the attention kernels
constexpr int FLAG_CAUSAL = 1;
constexpr int FLAG_PHQ_VEC = 2;   // phi_q rows 16-byte aligned -> vector loads
constexpr int FLAG_PHK_VEC = 4;   // phi_k rows 16-byte aligned -> vector loads
constexpr int FLAG_BIAS_VEC = 8;  // bias rows 16-byte aligned -> vector loads
constexpr int FLAG_LOG2 = 16;     // backward: phi_q in exp2 units

// Launch one fused attention forward; one function per head dim (16/32/64/128) and Q/K/V
// element type.  mode 0: low-rank factors padded to RP columns (0 = plain attention);
// mode 1: dense bias (RP = 0); mode 2: ALiBi factors formed in the kernel (16-bit only).
// aux_dt is the factor or bias dtype.  FB_EUNSUPPORTED when
// no kernel instance matches.
fb_status launch_attention_d16_bf16(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d16_f16(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d16_f32(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d32_bf16(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d32_f16(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d32_f32(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d64_bf16(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d64_f16(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d64_f32(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d128_bf16(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d128_f16(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);
fb_status launch_attention_d128_f32(int mode, fb_dtype aux_dt, int RP, const AttnParams& p, hipStream_t s);

// Exact closed-form factors / dense bias.  slopes_host: [H] (H <= kMaxSlopes) or NULL.
constexpr int kMaxSlopes = 256;
fb_status launch_make_factors(fb_bias_kind kind, int H, int N, int C, const double* slopes_host,
                              fb_dtype out_dt, int split, void* phq, void* phk, int R_pad, int R_nat,
                              double qscale, hipStream_t stream);

fb_status launch_make_dense_bias(fb_bias_kind kind, int H, int N, int C, const double* slopes_host,
                                 fb_dtype out_dt, void* bias, int64_t head_stride, int64_t row_stride,
                                 hipStream_t stream);

// Multiplicative low-rank bias: writes first = [x phi_1] * scale ([B][H][N][D], contiguous)
// and rest = [x phi_2, ..., x phi_R] * scale ([B][H][N][(R-1) D], contiguous) for x with
// row strides sx and 16-byte aligned rows; dt is FB_BF16 or FB_F16.
fb_status launch_mulbias_expand(fb_dtype dt, fb_dtype phi_dt, const void* x, const int64_t sx[3], const void* phi,
                                const int64_t sphi[3], int B, int H, int N, int D, int R, float scale, void* first,
                                void* rest, hipStream_t stream);

// Everything one backward launch pair needs (kernel argument, by value).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* delta;
  const void* phq;
  const void* phk;
  void* dq;
  void* dk;
  void* dv;
  float* dphq;
  float* dphk;
  int sq[3], sk[3], sv[3], sdo[3], sdq[3], sdk[3], sdv[3];
  int spq[3], spk[3], sdpq[3], sdpk[3];
  int R;
  int flags;        // FLAG_CAUSAL, FLAG_PHQ_VEC, FLAG_PHK_VEC
  int B, H, N;
  float scale;
  int nblk;         // 128-row blocks per (b, h)
};
constexpr int kBwdRows = 128;     // rows (keys or queries) per backward workgroup

// Backward kernels (fb_attn_bwd.h): one function per head dim (16 / 32 / 64 / 128); phi_dt as the
// forward; RP in {0, 16, 32, 64}.  FB_EUNSUPPORTED when no instance matches.
fb_status launch_attention_bwd_d16(fb_dtype dt, fb_dtype phi_dt, int RP, const BwdParams& p, hipStream_t s);
fb_status launch_attention_bwd_d32(fb_dtype dt, fb_dtype phi_dt, int RP, const BwdParams& p, hipStream_t s);
fb_status launch_attention_bwd_d64(fb_dtype dt, fb_dtype phi_dt, int RP, const BwdParams& p, hipStream_t s);
fb_status launch_attention_bwd_d128(fb_dtype dt, fb_dtype phi_dt, int RP, const BwdParams& p, hipStream_t s);
// Delta = rowsum(dO * O) into delta ([B][H][N] fp32).
fb_status launch_attention_bwd_delta(fb_dtype dt, const void* o, const int64_t so[3], const void* dout,
                                     const int64_t sdo[3], int B, int H, int N, int D, float* delta, hipStream_t s);
// out[b'][h'][n][r] = sum of part[b][h][n][r] ([B][H][N][R] dense fp32) over the batches /
// heads that an axis of out with stride 0 gathers, in (b, h) order.
fb_status launch_attention_bwd_reduce(const float* part, int B, int H, int N, int R, float* out,
                                      const int64_t sout[3], hipStream_t s);
// Factors with R not a multiple of 8: phi ([.][.][N][R] with strides sphi, 0 = broadcast, of
// element size es) -> out [B][H][N][R8] dense, columns R..R8-1 zero.
fb_status launch_attention_bwd_pad_factor(const void* phi, int es, const int64_t sphi[3], int B, int H, int N, int R,
                                          int R8, void* out, hipStream_t s);
// The summed / copied factor gradient of a padded run: out[b'][h'][n][r] (r < R, any 4-byte
// aligned strides) = sum of part[b][h][n][r] ([B][H][N][R8] dense fp32) over the batches / heads
// that an axis of out with stride 0 gathers, in (b, h) order.
fb_status launch_attention_bwd_unpad(const float* part, int B, int H, int N, int R8, int R, float* out,
                                     const int64_t sout[3], hipStream_t s);
// fp32 Q/K/V and factors (fb_attn_bwd_f32.hip): Delta, then the dK/dV and dQ kernels (head
// dims 16 / 32 / 64, any R up to 64, factors read in place with their strides).
fb_status launch_attention_bwd_delta_f32(const void* o, const int64_t so[3], const void* dout, const int64_t sdo[3],
                                         int B, int H, int N, int D, float* delta, hipStream_t s);
fb_status launch_attention_bwd_f32(const BwdParams& p, int D, hipStream_t s);
// Workspace layout of the backward: Delta, then the partial factor gradients that need a sum.
struct BwdWork {
  size_t delta_off, pq_off, pk_off, bytes;   // pq_off / pk_off = SIZE_MAX: no partial buffer
  // R not a multiple of 8: the factors are copied into [B][H][N][R8] buffers (zero columns
  // R..R8-1) at phq_off / phk_off and the kernels' per-(b, h) factor gradients go to
  // [B][H][N][R8] partials at pq_off / pk_off; R8 = 0 when no padding is needed
  size_t phq_off, phk_off;
  int R8;
};
BwdWork bwd_work_layout(int B, int H, int N, int R, const int64_t sdphi_q[3], const int64_t sdphi_k[3]);

void set_error(const char* fmt, ...);

// The backward pass behind fb_attn_bwd_lowrank (validation, then the launches); `fn` names
// the public entry point in error messages.  g->work must hold at least
// bwd_work_layout(...).bytes bytes.
fb_status attn_bwd_lowrank_impl(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt, int R,
                                const int64_t sphi_q[3], const int64_t sphi_k[3], const fb_attn_bwd_args* g,
                                hipStream_t stream, const char* fn, bool log2 = false);

}  // namespace fb
