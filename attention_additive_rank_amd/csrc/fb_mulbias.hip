// Operand expansion for attention with a multiplicative low-rank bias (FlashBias
// rebuttal, answer to Reviewer BRmd, Q1 (2), Eq. (1) and Eq. (3)).  With b = phi_q phi_k^T
// of rank R, the biased score s (q_i . k_j) b_ij equals q'_i . k'_j for
//   q' = s [q phi_q,1, ..., q phi_q,R],   k' = [k phi_k,1, ..., k phi_k,R]   (width D R),
// so the fused low-rank kernel runs it unchanged: the first D columns of q' / k' are its
// Q / K operands (with scale 1) and the other (R - 1) D columns its factor columns.
// Each output element is formed in fp32 and rounded once to the operand type.
#include <algorithm>

#include "fb_internal.h"

namespace fb {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec8 { typedef T type __attribute__((ext_vector_type(8))); };

template <typename P> __device__ __forceinline__ float to_f(P x) { return (float)x; }

// One thread per 16-byte chunk (8 columns) of one (b, h, n) row of x: the chunk is read
// once and written R times, scaled by each factor of the row.  Bytes per row: D es read,
// R D es written, R factor values read.
template <typename T, typename P>
__global__ __launch_bounds__(256) void mulbias_expand_kernel(const T* __restrict__ x, int64_t sx0, int64_t sx1,
                                                             int64_t sx2, const P* __restrict__ phi, int64_t sp0,
                                                             int64_t sp1, int64_t sp2, int B, int H, int N, int D,
                                                             int R, float scale, T* __restrict__ first,
                                                             T* __restrict__ rest) {
  typedef typename Vec8<T>::type T8;
  const int cpr = D / 8;                                   // 8-column chunks per row of x
  const int64_t total = (int64_t)B * H * N * cpr;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / cpr;
    const int c = (int)(t - row * cpr) * 8;
    const int n = (int)(row % N);
    const int64_t bh = row / N;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const T8 xv = __builtin_bit_cast(T8, *(const u32x4*)(x + b * sx0 + h * sx1 + n * sx2 + c));
    const P* pr = phi + b * sp0 + h * sp1 + n * sp2;
    for (int r = 0; r < R; ++r) {
      const float f = to_f(pr[r]) * scale;
      T8 y;
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = (T)((float)xv[j] * f);
      T* dst = r == 0 ? first + row * D + c : rest + row * (int64_t)(R - 1) * D + (int64_t)(r - 1) * D + c;
      *(u32x4*)dst = __builtin_bit_cast(u32x4, y);
    }
  }
}

template <typename T, typename P>
fb_status launch_t(const void* x, const int64_t sx[3], const void* phi, const int64_t sp[3], int B, int H, int N,
                   int D, int R, float scale, void* first, void* rest, hipStream_t stream) {
  const int64_t total = (int64_t)B * H * N * (D / 8);
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 16384);
  hipLaunchKernelGGL((mulbias_expand_kernel<T, P>), dim3(grid), dim3(256), 0, stream, (const T*)x, sx[0], sx[1],
                     sx[2], (const P*)phi, sp[0], sp[1], sp[2], B, H, N, D, R, scale, (T*)first, (T*)rest);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("multiplicative-bias expansion launch failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

template <typename T>
fb_status launch_phi(fb_dtype phi_dt, const void* x, const int64_t sx[3], const void* phi, const int64_t sp[3],
                     int B, int H, int N, int D, int R, float scale, void* first, void* rest, hipStream_t s) {
  switch (phi_dt) {
    case FB_F32: return launch_t<T, float>(x, sx, phi, sp, B, H, N, D, R, scale, first, rest, s);
    case FB_BF16: return launch_t<T, __bf16>(x, sx, phi, sp, B, H, N, D, R, scale, first, rest, s);
    case FB_F16: return launch_t<T, _Float16>(x, sx, phi, sp, B, H, N, D, R, scale, first, rest, s);
  }
  return FB_EUNSUPPORTED;
}

}  // namespace

fb_status launch_mulbias_expand(fb_dtype dt, fb_dtype phi_dt, const void* x, const int64_t sx[3], const void* phi,
                                const int64_t sphi[3], int B, int H, int N, int D, int R, float scale, void* first,
                                void* rest, hipStream_t stream) {
  if (dt == FB_BF16) return launch_phi<__bf16>(phi_dt, x, sx, phi, sphi, B, H, N, D, R, scale, first, rest, stream);
  if (dt == FB_F16) return launch_phi<_Float16>(phi_dt, x, sx, phi, sphi, B, H, N, D, R, scale, first, rest, stream);
  return FB_EUNSUPPORTED;
}

}  // namespace fb
