// Small kernels around the attention backward: Delta_i = sum_d dO_id O_id (fp32) before the
// fused kernels, and the sum of per-(b, h) factor gradients for a factor shared by several
// batches or heads after them (fixed order, no atomics).
#include <algorithm>

#include "fb_attn_bwd.h"

namespace fb {
namespace {

// D / 8 threads per (b, h, n) row, one 16-byte chunk of dO and O each: fp32 products of the
// chunk, then a butterfly over the row's threads (fixed order); whole waves read whole rows.
template <typename T, int TPR>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ o, int64_t so0, int64_t so1, int64_t so2,
                                                    const T* __restrict__ d, int64_t sd0, int64_t sd1, int64_t sd2,
                                                    int B, int H, int N, float* __restrict__ delta) {
  typedef T T8 __attribute__((ext_vector_type(8)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t rows = (int64_t)B * H * N;
  const int sub = threadIdx.x % TPR;
  const int64_t step = (int64_t)gridDim.x * (blockDim.x / TPR);
  // the row loop is uniform over a row's TPR threads, so each butterfly sees its whole row
  for (int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / TPR; r < rows; r += step) {
    const int n = (int)(r % N);
    const int64_t bh = r / N;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const T8 a = __builtin_bit_cast(T8, *(const u32x4*)(o + b * so0 + h * so1 + n * so2 + 8 * sub));
    const T8 g = __builtin_bit_cast(T8, *(const u32x4*)(d + b * sd0 + h * sd1 + n * sd2 + 8 * sub));
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += (float)a[j] * (float)g[j];
#pragma unroll
    for (int m = TPR / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m, TPR);
    if (sub == 0) delta[r] = acc;
  }
}

// One thread per four consecutive output columns: the partials of the (b, h) pairs it
// gathers, b outer, h inner (16-byte loads and stores; R and the output strides are
// multiples of 4).
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, int B, int H, int N, int R,
                                                     int Bo, int Ho, float* __restrict__ out, int64_t s0, int64_t s1,
                                                     int64_t s2) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int R4 = R / 4;
  const int64_t plane = (int64_t)N * R4;            // float4s per (b, h)
  const int64_t total = (int64_t)Bo * Ho * plane;
  const f32x4* p4 = (const f32x4*)part;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t nr = t % plane;
    const int64_t bh = t / plane;
    const int ho = (int)(bh % Ho), bo = (int)(bh / Ho);
    const int b0 = Bo == 1 ? 0 : bo, b1 = Bo == 1 ? B : bo + 1;
    const int h0 = Ho == 1 ? 0 : ho, h1 = Ho == 1 ? H : ho + 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int b = b0; b < b1; ++b) {
#pragma unroll 4
      for (int h = h0; h < h1; ++h) acc += p4[((int64_t)b * H + h) * plane + nr];
    }
    const int n = (int)(nr / R4), c = (int)(nr % R4) * 4;
    *(f32x4*)(out + bo * s0 + ho * s1 + n * s2 + c) = acc;
  }
}

// One thread per 8 output columns of a padded factor row: the row's elements below R (element
// loads, any alignment), zeros above.
template <typename T>
__global__ __launch_bounds__(256) void pad_factor_kernel(const T* __restrict__ phi, int64_t s0, int64_t s1, int64_t s2,
                                                         int B, int H, int N, int R, int R8, T* __restrict__ out) {
  typedef T T8 __attribute__((ext_vector_type(8)));
  const int C8 = R8 / 8;
  const int64_t total = (int64_t)B * H * N * C8;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int c0 = (int)(t % C8) * 8;
    const int64_t row = t / C8;
    const int n = (int)(row % N);
    const int64_t bh = row / N;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const T* src = phi + b * s0 + h * s1 + n * s2;
    T8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = c0 + j < R ? src[c0 + j] : (T)0.f;
    *(T8*)(out + row * R8 + c0) = v;
  }
}

// One thread per output element of a padded run's factor gradient: the partials of the (b, h)
// pairs it gathers, b outer, h inner.
__global__ __launch_bounds__(256) void unpad_kernel(const float* __restrict__ part, int B, int H, int N, int R8, int R,
                                                    int Bo, int Ho, float* __restrict__ out, int64_t s0, int64_t s1,
                                                    int64_t s2) {
  const int64_t plane = (int64_t)N * R;
  const int64_t total = (int64_t)Bo * Ho * plane;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t nr = t % plane;
    const int64_t bh = t / plane;
    const int ho = (int)(bh % Ho), bo = (int)(bh / Ho);
    const int n = (int)(nr / R), c = (int)(nr % R);
    const int b0 = Bo == 1 ? 0 : bo, b1 = Bo == 1 ? B : bo + 1;
    const int h0 = Ho == 1 ? 0 : ho, h1 = Ho == 1 ? H : ho + 1;
    float acc = 0.f;
    for (int b = b0; b < b1; ++b)
      for (int h = h0; h < h1; ++h) acc += part[(((int64_t)b * H + h) * N + n) * R8 + c];
    out[bo * s0 + ho * s1 + n * s2 + c] = acc;
  }
}

int grid_for(int64_t work) { return (int)std::min<int64_t>((work + 255) / 256, 8192); }

template <typename T, int TPR>
void launch_delta(const void* o, const int64_t so[3], const void* dout, const int64_t sdo[3], int B, int H, int N,
                  float* delta, hipStream_t s) {
  const dim3 grid(grid_for((int64_t)B * H * N * TPR));
  hipLaunchKernelGGL((delta_kernel<T, TPR>), grid, dim3(256), 0, s, (const T*)o, so[0], so[1], so[2], (const T*)dout,
                     sdo[0], sdo[1], sdo[2], B, H, N, delta);
}

template <typename T>
void launch_delta_d(int D, const void* o, const int64_t so[3], const void* dout, const int64_t sdo[3], int B, int H,
                    int N, float* delta, hipStream_t s) {
  // D in {16, 32, 64, 128} (checked by the caller): D / 8 threads per row
  if (D == 16) launch_delta<T, 2>(o, so, dout, sdo, B, H, N, delta, s);
  else if (D == 32) launch_delta<T, 4>(o, so, dout, sdo, B, H, N, delta, s);
  else if (D == 64) launch_delta<T, 8>(o, so, dout, sdo, B, H, N, delta, s);
  else launch_delta<T, 16>(o, so, dout, sdo, B, H, N, delta, s);
}

}  // namespace

fb_status launch_attention_bwd_delta(fb_dtype dt, const void* o, const int64_t so[3], const void* dout,
                                     const int64_t sdo[3], int B, int H, int N, int D, float* delta, hipStream_t s) {
  if (dt == FB_BF16)
    launch_delta_d<__bf16>(D, o, so, dout, sdo, B, H, N, delta, s);
  else
    launch_delta_d<_Float16>(D, o, so, dout, sdo, B, H, N, delta, s);
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
  hipLaunchKernelGGL(reduce_kernel, dim3(grid_for((int64_t)Bo * Ho * N * (R / 4))), dim3(256), 0, s, part, B, H, N,
                     R, Bo, Ho, out, sout[0], sout[1], sout[2]);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("factor-gradient reduction failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

fb_status launch_attention_bwd_pad_factor(const void* phi, int es, const int64_t sphi[3], int B, int H, int N, int R,
                                          int R8, void* out, hipStream_t s) {
  const dim3 grid(grid_for((int64_t)B * H * N * (R8 / 8)));
  if (es == 2)
    hipLaunchKernelGGL(pad_factor_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)phi, sphi[0], sphi[1],
                       sphi[2], B, H, N, R, R8, (uint16_t*)out);
  else
    return FB_EUNSUPPORTED;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("factor padding failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

fb_status launch_attention_bwd_unpad(const float* part, int B, int H, int N, int R8, int R, float* out,
                                     const int64_t sout[3], hipStream_t s) {
  // an axis of the output with stride 0 has one position and gathers all of that axis
  const int Bo = sout[0] ? B : 1, Ho = sout[1] ? H : 1;
  hipLaunchKernelGGL(unpad_kernel, dim3(grid_for((int64_t)Bo * Ho * N * R)), dim3(256), 0, s, part, B, H, N, R8, R, Bo,
                     Ho, out, sout[0], sout[1], sout[2]);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("factor-gradient unpadding failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

}  // namespace fb
