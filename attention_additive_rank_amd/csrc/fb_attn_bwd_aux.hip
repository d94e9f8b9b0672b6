// Small kernels around the attention backward: Delta_i = sum_d dO_id O_id (fp32) before the
// fused kernels, and the sum of per-(b, h) factor gradients for a factor shared by several
// batches or heads after them (fixed order, no atomics).
#include <algorithm>

#include "fb_attn_bwd.h"

namespace fb {
namespace {

// One thread per (b, h, n) row: D / 8 chunks of dO and O, fp32 products summed in order.
template <typename T>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ o, int64_t so0, int64_t so1, int64_t so2,
                                                    const T* __restrict__ d, int64_t sd0, int64_t sd1, int64_t sd2,
                                                    int B, int H, int N, int D, float* __restrict__ delta) {
  typedef T T8 __attribute__((ext_vector_type(8)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t rows = (int64_t)B * H * N;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows; r += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(r % N);
    const int64_t bh = r / N;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const T* orow = o + b * so0 + h * so1 + n * so2;
    const T* drow = d + b * sd0 + h * sd1 + n * sd2;
    float acc = 0.f;
    for (int c = 0; c < D; c += 8) {
      const T8 a = __builtin_bit_cast(T8, *(const u32x4*)(orow + c));
      const T8 g = __builtin_bit_cast(T8, *(const u32x4*)(drow + c));
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += (float)a[j] * (float)g[j];
    }
    delta[r] = acc;
  }
}

// One thread per output element: the partials of the (b, h) pairs it gathers, b outer.
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, int B, int H, int N, int R,
                                                     int Bo, int Ho, float* __restrict__ out, int64_t s0, int64_t s1,
                                                     int64_t s2) {
  const int64_t total = (int64_t)Bo * Ho * N * R;
  const int64_t hstride = (int64_t)N * R, bstride = (int64_t)H * hstride;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t nr = t % hstride;
    const int64_t bh = t / hstride;
    const int ho = (int)(bh % Ho), bo = (int)(bh / Ho);
    const int b0 = Bo == 1 ? 0 : bo, b1 = Bo == 1 ? B : bo + 1;
    const int h0 = Ho == 1 ? 0 : ho, h1 = Ho == 1 ? H : ho + 1;
    float acc = 0.f;
    for (int b = b0; b < b1; ++b)
      for (int h = h0; h < h1; ++h) acc += part[b * bstride + h * hstride + nr];
    out[bo * s0 + ho * s1 + (nr / R) * s2 + nr % R] = acc;
  }
}

int grid_for(int64_t work) { return (int)std::min<int64_t>((work + 255) / 256, 8192); }

}  // namespace

fb_status launch_attention_bwd_delta(fb_dtype dt, const void* o, const int64_t so[3], const void* dout,
                                     const int64_t sdo[3], int B, int H, int N, int D, float* delta, hipStream_t s) {
  const int64_t rows = (int64_t)B * H * N;
  if (dt == FB_BF16)
    hipLaunchKernelGGL((delta_kernel<__bf16>), dim3(grid_for(rows)), dim3(256), 0, s, (const __bf16*)o, so[0], so[1],
                       so[2], (const __bf16*)dout, sdo[0], sdo[1], sdo[2], B, H, N, D, delta);
  else
    hipLaunchKernelGGL((delta_kernel<_Float16>), dim3(grid_for(rows)), dim3(256), 0, s, (const _Float16*)o, so[0],
                       so[1], so[2], (const _Float16*)dout, sdo[0], sdo[1], sdo[2], B, H, N, D, delta);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention backward preparation failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

fb_status launch_attention_bwd_reduce(const float* part, int B, int H, int N, int R, float* out,
                                      const int64_t sout[3], hipStream_t s) {
  // an axis of the output with stride 0 has one position and gathers all of that axis
  const int Bo = sout[0] ? B : 1, Ho = sout[1] ? H : 1;
  hipLaunchKernelGGL(reduce_kernel, dim3(grid_for((int64_t)Bo * Ho * N * R)), dim3(256), 0, s, part, B, H, N, R, Bo,
                     Ho, out, sout[0], sout[1], sout[2]);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("factor-gradient reduction failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

}  // namespace fb
