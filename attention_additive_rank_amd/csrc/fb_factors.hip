// Exact factor generation and dense materialisation of the closed-form biases.
//
// ALiBi (FlashBias rebuttal, answer to Reviewer BRmd, Q2: the bias is built from
// #heads slopes; FlashBias generates Block_q x 2 and Block_k x 2 factor tiles):
//   b[h,i,j] = m_h (j - i),  phi_q(i) = [1, i],  phi_k(j) = [m_h j, -m_h].
// Sandwich (rebuttal, answer to Reviewer UJUf, Q1 (1)-(2)):
//   b[i,j] = sum_{k=1}^{C/2} cos((i-j) w_k),  w_k = 10000^(-2k/C),
//   phi(i) = [cos(i w_1), sin(i w_1), ..., cos(i w_{C/2}), sin(i w_{C/2})],
//   phi_q = phi_k = phi, so phi phi^T = b by cos(a-b) = cos a cos b + sin a sin b.
// All values are computed in fp64 and rounded once (round to nearest even) into
// the output type; the optional split writes each value as a sum of pieces.
#include <cmath>

#include "fb_internal.h"

namespace fb {
namespace {

// ALiBi: the caller's slopes (use_host set), or none; Sandwich: the frequencies w_1..w_{C/2}
// from the host's fp64 pow (use_host set when C / 2 <= kMaxSlopes), else computed here.
struct Slopes {
  double m[kMaxSlopes];
};

// Correctly rounded (nearest even) value of x in a binary format with `prec`
// significand bits and minimum normal exponent `emin`, returned as a double.
__device__ __forceinline__ double round_prec(double x, int prec, int emin) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  frexp(x, &e);              // x = f * 2^e, 0.5 <= |f| < 1
  int ex = e - 1;            // exponent of the leading bit
  if (ex < emin) ex = emin;  // subnormal range: fixed quantum
  // quantum q = 2^(ex - prec + 1); scaling by 1 / q (a power of two) is exact
  return rint(x * ldexp(1.0, prec - 1 - ex)) * ldexp(1.0, ex - prec + 1);
}

template <typename T> struct Fmt;
template <> struct Fmt<float>    { static constexpr int prec = 24, emin = -126; };
template <> struct Fmt<__bf16>   { static constexpr int prec = 8,  emin = -126; };
template <> struct Fmt<_Float16> { static constexpr int prec = 11, emin = -14; };

// Store a double that is exactly representable in T.
template <typename T> __device__ __forceinline__ T exact_to(double x) { return (T)(float)x; }

template <typename T> __device__ __forceinline__ double rn(double x) {
  return round_prec(x, Fmt<T>::prec, Fmt<T>::emin);
}

// Piece `a` of the split of x: x_0 = rn(x), x_1 = rn(x - x_0), x_2 = rn(x - x_0 - x_1).
template <typename T> __device__ __forceinline__ double piece(double x, int a) {
  double rest = x, p = 0.0;
  for (int i = 0; i <= a; ++i) {
    p = rn<T>(rest);
    rest -= p;
  }
  return p;
}

__device__ __forceinline__ double alibi_slope(const Slopes& s, int use_host, int h, int H) {
  return use_host ? s.m[h] : exp2(-8.0 * (double)(h + 1) / (double)H);
}

__device__ __forceinline__ double sandwich_freq(const Slopes& s, int use_host, int k, int C) {  // k = 1..C/2
  return use_host ? s.m[k - 1] : pow(10000.0, -2.0 * (double)k / (double)C);
}

// pair index -> (a, b) pieces, ordered (0,0), (0,1), (1,0), (0,2), (1,1), (2,0)
__device__ __forceinline__ void pair_of(int idx, int& a, int& b) {
  int s = 0;
  while (idx > s) { idx -= s + 1; ++s; }
  a = idx;
  b = s - idx;
}

// One thread per (head, row, output column): column c is piece c % npairs of natural column
// c / npairs (Sandwich's cos (even) or sin (odd) of one angle, ALiBi's two columns), with
// npairs = split (split + 1) / 2 pieces per natural column; columns at or beyond R_used are
// written as zero.  Every value is formed in fp64 and rounded once, as one chain per thread
// (short, so the launch is not bound by the latency of a long fp64 chain), and consecutive
// threads write consecutive columns of a row.  Index arithmetic is 32-bit (the host caps
// H N R_pad below 2^31).
template <typename T>
__global__ void make_factors_kernel(fb_bias_kind kind, int H, int N, int C, Slopes slopes, int use_host,
                                    int split, T* phq, T* phk, int R_pad, int R_nat, double qscale) {
  const int npairs = split * (split + 1) / 2;
  const int R_used = R_nat * npairs;
  const int total = H * N * R_pad;
  for (int64_t t64 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t64 < total;
       t64 += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)t64;
    const int col = t % R_pad;
    const int hn = t / R_pad;
    const int n = hn % N;
    const int h = hn / N;
    double vq = 0.0, vk = 0.0;
    if (col < R_used) {
      const int nat = col / npairs;      // natural column: 2 g + u
      const int g = nat >> 1, u = nat & 1;
      double fq, fk;
      if (kind == FB_ALIBI) {
        const double m = alibi_slope(slopes, use_host, h, H);
        fq = u ? (double)n : 1.0;
        fk = u ? -m : m * (double)n;
      } else {
        double sn, cs;
        sincos((double)n * sandwich_freq(slopes, use_host, g + 1, C), &sn, &cs);
        fq = fk = u ? sn : cs;
      }
      int a, b;
      pair_of(col % npairs, a, b);
      vq = piece<T>(fq * qscale, a);
      vk = piece<T>(fk, b);
    }
    phq[t] = exact_to<T>(vq);
    phk[t] = exact_to<T>(vk);
  }
}

template <typename T>
__global__ void make_dense_bias_kernel(fb_bias_kind kind, int H, int N, int C, Slopes slopes, int use_host,
                                       T* bias, int64_t head_stride, int64_t row_stride) {
  const int64_t total = (int64_t)H * N * N;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(t % N);
    const int64_t hi = t / N;
    const int i = (int)(hi % N);
    const int h = (int)(hi / N);
    double v;
    if (kind == FB_ALIBI) {
      v = alibi_slope(slopes, use_host, h, H) * (double)(j - i);
    } else {
      v = 0.0;
      const double d = (double)(i - j);
      for (int k = 1; k <= C / 2; ++k) v += cos(d * sandwich_freq(slopes, use_host, k, C));
    }
    bias[h * head_stride + (int64_t)i * row_stride + j] = exact_to<T>(rn<T>(v));
  }
}

// The kernel argument for `kind`; use_host says whether it holds the values (ALiBi: the
// caller's slopes, if any; Sandwich: the C / 2 frequencies, if they fit).
Slopes pack_slopes(fb_bias_kind kind, const double* host, int H, int C, int& use_host) {
  Slopes s{};
  use_host = 0;
  if (kind == FB_ALIBI && host) {
    for (int h = 0; h < H; ++h) s.m[h] = host[h];
    use_host = 1;
  } else if (kind == FB_SANDWICH && C / 2 <= kMaxSlopes) {
    for (int k = 1; k <= C / 2; ++k) s.m[k - 1] = std::pow(10000.0, -2.0 * k / C);
    use_host = 1;
  }
  return s;
}

int grid_for(int64_t total) {
  const int64_t g = (total + 255) / 256;
  return (int)(g > 65536 ? 65536 : (g < 1 ? 1 : g));
}

}  // namespace

fb_status launch_make_factors(fb_bias_kind kind, int H, int N, int C, const double* slopes_host,
                              fb_dtype out_dt, int split, void* phq, void* phk, int R_pad, int R_nat,
                              double qscale, hipStream_t stream) {
  int use_host;
  const Slopes s = pack_slopes(kind, slopes_host, H, C, use_host);
  const int grid = grid_for((int64_t)H * N * R_pad);
  switch (out_dt) {
    case FB_F32:
      hipLaunchKernelGGL(make_factors_kernel<float>, dim3(grid), dim3(256), 0, stream, kind, H, N, C, s,
                         use_host, split, (float*)phq, (float*)phk, R_pad, R_nat, qscale);
      break;
    case FB_BF16:
      hipLaunchKernelGGL(make_factors_kernel<__bf16>, dim3(grid), dim3(256), 0, stream, kind, H, N, C, s,
                         use_host, split, (__bf16*)phq, (__bf16*)phk, R_pad, R_nat, qscale);
      break;
    case FB_F16:
      hipLaunchKernelGGL(make_factors_kernel<_Float16>, dim3(grid), dim3(256), 0, stream, kind, H, N, C, s,
                         use_host, split, (_Float16*)phq, (_Float16*)phk, R_pad, R_nat, qscale);
      break;
    default:
      return FB_EUNSUPPORTED;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("fb_make_factors: launch failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

fb_status launch_make_dense_bias(fb_bias_kind kind, int H, int N, int C, const double* slopes_host,
                                 fb_dtype out_dt, void* bias, int64_t head_stride, int64_t row_stride,
                                 hipStream_t stream) {
  int use_host;
  const Slopes s = pack_slopes(kind, slopes_host, H, C, use_host);
  const int grid = grid_for((int64_t)H * N * N);
  switch (out_dt) {
    case FB_F32:
      hipLaunchKernelGGL(make_dense_bias_kernel<float>, dim3(grid), dim3(256), 0, stream, kind, H, N, C, s,
                         use_host, (float*)bias, head_stride, row_stride);
      break;
    case FB_BF16:
      hipLaunchKernelGGL(make_dense_bias_kernel<__bf16>, dim3(grid), dim3(256), 0, stream, kind, H, N, C, s,
                         use_host, (__bf16*)bias, head_stride, row_stride);
      break;
    case FB_F16:
      hipLaunchKernelGGL(make_dense_bias_kernel<_Float16>, dim3(grid), dim3(256), 0, stream, kind, H, N, C, s,
                         use_host, (_Float16*)bias, head_stride, row_stride);
      break;
    default:
      return FB_EUNSUPPORTED;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("fb_make_dense_bias: launch failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

}  // namespace fb
