// Small kernels around the attention backward: Delta_i = sum_d dO_id O_id (fp32), and
// clearing the fp32 factor-gradient outputs before the backward kernels accumulate into
// them (atomically, so that factors broadcast over batch or heads get summed gradients).
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

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ x, int64_t s0, int64_t s1, int64_t s2, int B,
                                                   int H, int N, int R) {
  const int64_t total = (int64_t)B * H * N * R;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(t % R);
    const int64_t row = t / R;
    const int n = (int)(row % N);
    const int64_t bh = row / N;
    const int h = (int)(bh % H), b = (int)(bh / H);
    x[b * s0 + h * s1 + n * s2 + r] = 0.f;
  }
}

int grid_for(int64_t work) { return (int)std::min<int64_t>((work + 255) / 256, 8192); }

}  // namespace

fb_status launch_attention_bwd_aux(fb_dtype dt, const void* o, const int64_t so[3], const void* dout,
                                   const int64_t sdo[3], int B, int H, int N, int D, float* delta, float* dphq,
                                   const int64_t sdpq[3], float* dphk, const int64_t sdpk[3], int R, hipStream_t s) {
  const int64_t rows = (int64_t)B * H * N;
  if (dt == FB_BF16)
    hipLaunchKernelGGL((delta_kernel<__bf16>), dim3(grid_for(rows)), dim3(256), 0, s, (const __bf16*)o, so[0], so[1],
                       so[2], (const __bf16*)dout, sdo[0], sdo[1], sdo[2], B, H, N, D, delta);
  else
    hipLaunchKernelGGL((delta_kernel<_Float16>), dim3(grid_for(rows)), dim3(256), 0, s, (const _Float16*)o, so[0],
                       so[1], so[2], (const _Float16*)dout, sdo[0], sdo[1], sdo[2], B, H, N, D, delta);
  if (R > 0) {
    // clear each distinct element once: an axis with stride 0 has one position
    const int Bq = sdpq[0] ? B : 1, Hq = sdpq[1] ? H : 1, Bk = sdpk[0] ? B : 1, Hk = sdpk[1] ? H : 1;
    hipLaunchKernelGGL(zero_kernel, dim3(grid_for((int64_t)Bq * Hq * N * R)), dim3(256), 0, s, dphq, sdpq[0], sdpq[1],
                       sdpq[2], Bq, Hq, N, R);
    hipLaunchKernelGGL(zero_kernel, dim3(grid_for((int64_t)Bk * Hk * N * R)), dim3(256), 0, s, dphk, sdpk[0], sdpk[1],
                       sdpk[2], Bk, Hk, N, R);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention backward preparation failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

}  // namespace fb
