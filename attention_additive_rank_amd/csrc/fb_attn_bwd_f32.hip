// Backward of attention with an additive low-rank bias for fp32 Q/K/V and fp32 factors.
//
// The gradients are those of the 16-bit kernels (fb_attn_bwd.h): with Q' = [Q s, phi_q],
// K' = [K, phi_k] (FlashBias rebuttal, answer to Reviewer UJUf, Q2), S = Q' K'^T, the
// forward's row log-sum-exp L, P = exp(S - L), Delta_i = sum_d dO_id O_id,
//   dV = P^T dO,  dP = dO V^T,  dS = P .* (dP - Delta),
//   dK' = dS^T Q' = [dK, dphi_k],  dQ' = dS K' = [dQ / s, dphi_q],
// recomputing S and P block by block (nothing N x N is stored).
//
// The fp32 matrix core (v_mfma_f32_32x32x2f32) takes one k element per lane: lane l of A
// holds A[l % 32][l / 32], lane l of B holds B[l / 32][l % 32], and lane l of the 32 x 32
// result holds column l % 32, rows crow(r, l / 32) = 8 (r / 4) + 4 (l / 32) + r % 4 in its
// registers r = 0..15.  Each kernel computes the scores in the orientation that puts the
// next product's B operand in those registers as they are:
//   attn_bwd_f32_dkv_kernel (a wavefront owns 32 keys, streams 32-query blocks): S and dP
//     with queries as rows, so register u of P / dS is B[k = query crow(u, h)][n = key] of
//     dV^T += dO^T P and dK'^T += Q'^T dS, whose A operands read the rows crow(u, h);
//   attn_bwd_f32_dq_kernel (a wavefront owns 32 queries, streams 32-key blocks): S^T and
//     dP^T with keys as rows, so register u of dS^T is B of dQ'^T += K'^T dS^T.
// Operands are read from global memory per lane (zero past N and past the D + R columns);
// this path serves fp32 models at modest sizes, the 16-bit kernels are the fast path.
#include <algorithm>

#include "fb_internal.h"

namespace fb {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Rows of one (b, h): Q' = [Q s, phi_q] and K' = [K, phi_k] by column, V and dO.
struct Rows {
  const float *q, *k, *v, *dout, *pq, *pk;
  int sq, sk, sv, sdo, spq, spk;
  int D, R, N;
  float scale;
  __device__ float qp(int n, int c) const {
    if (n >= N) return 0.f;
    if (c < D) return q[(int64_t)n * sq + c] * scale;
    c -= D;
    return c < R ? pq[(int64_t)n * spq + c] : 0.f;
  }
  __device__ float kp(int n, int c) const {
    if (n >= N) return 0.f;
    if (c < D) return k[(int64_t)n * sk + c];
    c -= D;
    return c < R ? pk[(int64_t)n * spk + c] : 0.f;
  }
  __device__ float vr(int n, int c) const { return n < N && c < D ? v[(int64_t)n * sv + c] : 0.f; }
  __device__ float dor(int n, int c) const { return n < N && c < D ? dout[(int64_t)n * sdo + c] : 0.f; }
};

__device__ __forceinline__ Rows rows_of(const BwdParams& p, int b, int h, int D) {
  Rows w;
  w.q = (const float*)p.q + ((int64_t)b * p.sq[0] + (int64_t)h * p.sq[1]);
  w.k = (const float*)p.k + ((int64_t)b * p.sk[0] + (int64_t)h * p.sk[1]);
  w.v = (const float*)p.v + ((int64_t)b * p.sv[0] + (int64_t)h * p.sv[1]);
  w.dout = (const float*)p.dout + ((int64_t)b * p.sdo[0] + (int64_t)h * p.sdo[1]);
  w.pq = p.R > 0 ? (const float*)p.phq + ((int64_t)b * p.spq[0] + (int64_t)h * p.spq[1]) : nullptr;
  w.pk = p.R > 0 ? (const float*)p.phk + ((int64_t)b * p.spk[0] + (int64_t)h * p.spk[1]) : nullptr;
  w.sq = p.sq[2];
  w.sk = p.sk[2];
  w.sv = p.sv[2];
  w.sdo = p.sdo[2];
  w.spq = p.spq[2];
  w.spk = p.spk[2];
  w.D = D;
  w.R = p.R;
  w.N = p.N;
  w.scale = p.scale;
  return w;
}

// DB: 32-wide blocks of the head dim, CB: of the K' / Q' width D + R.
template <int DB, int CB, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_bwd_f32_dkv_kernel(BwdParams p, int D) {
  const int lane = threadIdx.x & 63, ln = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int blk = blockIdx.x % p.nblk, bh = blockIdx.x / p.nblk;
  const int hh = bh % p.H, bb = bh / p.H;
  const int k0 = blk * kBwdRows + wave * 32;   // this wavefront's keys k0 .. k0 + 31
  if (k0 >= p.N) return;                       // (no workgroup barriers in this kernel)
  const Rows w = rows_of(p, bb, hh, D);
  const float* L = p.lse + ((int64_t)bb * p.H + hh) * p.N;
  const float* Dl = p.delta + ((int64_t)bb * p.H + hh) * p.N;
  const int W = D + p.R;
  const int key = k0 + ln;
  f32x16 dvt[DB], dkt[CB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dvt[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < CB; ++i) dkt[i] = f32x16{};
  // causal: queries before k0 see none of these keys
  for (int q0 = CAUSAL ? k0 : 0; q0 < p.N; q0 += 32) {
    f32x16 s = f32x16{}, dp = f32x16{};
    for (int c = 0; c < W; c += 2) s = mma(w.qp(q0 + ln, c + hf), w.kp(key, c + hf), s);
    for (int c = 0; c < D; c += 2) dp = mma(w.dor(q0 + ln, c + hf), w.vr(key, c + hf), dp);
    float pr[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = q0 + crow(r, hf);
      const bool ok = q < p.N && key < p.N && (!CAUSAL || key <= q);
      const float lq = ok ? L[q] : 0.f, dq = ok ? Dl[q] : 0.f;
      pr[r] = ok ? __builtin_amdgcn_exp2f((s[r] - lq) * kLog2e) : 0.f;
      ds[r] = pr[r] * (dp[r] - dq);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int q = q0 + crow(u, hf);
#pragma unroll
      for (int db = 0; db < DB; ++db) dvt[db] = mma(w.dor(q, 32 * db + ln), pr[u], dvt[db]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) dkt[cb] = mma(w.qp(q, 32 * cb + ln), ds[u], dkt[cb]);
    }
  }
  if (key >= p.N) return;
  float* dV = (float*)p.dv + ((int64_t)bb * p.sdv[0] + (int64_t)hh * p.sdv[1] + (int64_t)key * p.sdv[2]);
  float* dK = (float*)p.dk + ((int64_t)bb * p.sdk[0] + (int64_t)hh * p.sdk[1] + (int64_t)key * p.sdk[2]);
  float* dPk = p.R > 0 ? p.dphk + ((int64_t)bb * p.sdpk[0] + (int64_t)hh * p.sdpk[1] + (int64_t)key * p.sdpk[2])
                       : nullptr;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 32 * db + crow(r, hf);
      if (d < D) dV[d] = dvt[db][r];
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = 32 * cb + crow(r, hf);
      if (c < D) dK[c] = dkt[cb][r];
      else if (c < W) dPk[c - D] = dkt[cb][r];
    }
  }
}

template <int CB, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_bwd_f32_dq_kernel(BwdParams p, int D) {
  const int lane = threadIdx.x & 63, ln = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int blk = blockIdx.x % p.nblk, bh = blockIdx.x / p.nblk;
  const int hh = bh % p.H, bb = bh / p.H;
  const int q0 = blk * kBwdRows + wave * 32;   // this wavefront's queries q0 .. q0 + 31
  if (q0 >= p.N) return;
  const Rows w = rows_of(p, bb, hh, D);
  const int W = D + p.R;
  const int qq = q0 + ln;
  const bool qok = qq < p.N;
  const float lq = qok ? p.lse[((int64_t)bb * p.H + hh) * p.N + qq] : 0.f;
  const float dl = qok ? p.delta[((int64_t)bb * p.H + hh) * p.N + qq] : 0.f;
  f32x16 dqt[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) dqt[i] = f32x16{};
  const int kend = CAUSAL ? min(p.N, q0 + 32) : p.N;
  for (int kb0 = 0; kb0 < kend; kb0 += 32) {
    f32x16 st = f32x16{}, dpt = f32x16{};
    for (int c = 0; c < W; c += 2) st = mma(w.kp(kb0 + ln, c + hf), w.qp(qq, c + hf), st);
    for (int c = 0; c < D; c += 2) dpt = mma(w.vr(kb0 + ln, c + hf), w.dor(qq, c + hf), dpt);
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = kb0 + crow(r, hf);
      const bool ok = qok && kk < p.N && (!CAUSAL || kk <= qq);
      const float pv = ok ? __builtin_amdgcn_exp2f((st[r] - lq) * kLog2e) : 0.f;
      ds[r] = pv * (dpt[r] - dl);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int kk = kb0 + crow(u, hf);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) dqt[cb] = mma(w.kp(kk, 32 * cb + ln), ds[u], dqt[cb]);
    }
  }
  if (!qok) return;
  float* dQ = (float*)p.dq + ((int64_t)bb * p.sdq[0] + (int64_t)hh * p.sdq[1] + (int64_t)qq * p.sdq[2]);
  float* dPq = p.R > 0 ? p.dphq + ((int64_t)bb * p.sdpq[0] + (int64_t)hh * p.sdpq[1] + (int64_t)qq * p.sdpq[2])
                       : nullptr;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = 32 * cb + crow(r, hf);
      if (c < D) dQ[c] = p.scale * dqt[cb][r];
      else if (c < W) dPq[c - D] = dqt[cb][r];
    }
  }
}

// Delta = rowsum(dO * O), one thread per row.
__global__ __launch_bounds__(256) void delta_f32_kernel(const float* __restrict__ o, int64_t so0, int64_t so1,
                                                        int64_t so2, const float* __restrict__ d, int64_t sd0,
                                                        int64_t sd1, int64_t sd2, int B, int H, int N, int D,
                                                        float* __restrict__ delta) {
  const int64_t rows = (int64_t)B * H * N;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows; r += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(r % N);
    const int64_t bh = r / N;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const float* orow = o + b * so0 + h * so1 + n * so2;
    const float* drow = d + b * sd0 + h * sd1 + n * sd2;
    float acc = 0.f;
    for (int c = 0; c < D; ++c) acc += orow[c] * drow[c];
    delta[r] = acc;
  }
}

template <int DB, int CB>
void launch_pair(const BwdParams& p, int D, bool causal, dim3 grid, hipStream_t s) {
  if (causal) {
    hipLaunchKernelGGL((attn_bwd_f32_dkv_kernel<DB, CB, true>), grid, dim3(256), 0, s, p, D);
    hipLaunchKernelGGL((attn_bwd_f32_dq_kernel<CB, true>), grid, dim3(256), 0, s, p, D);
  } else {
    hipLaunchKernelGGL((attn_bwd_f32_dkv_kernel<DB, CB, false>), grid, dim3(256), 0, s, p, D);
    hipLaunchKernelGGL((attn_bwd_f32_dq_kernel<CB, false>), grid, dim3(256), 0, s, p, D);
  }
}

template <int DB>
fb_status launch_cb(const BwdParams& p, int D, int CB, bool causal, dim3 grid, hipStream_t s) {
  switch (CB) {
    case 1: launch_pair<DB, 1>(p, D, causal, grid, s); return FB_OK;
    case 2: launch_pair<DB, 2>(p, D, causal, grid, s); return FB_OK;
    case 3: launch_pair<DB, 3>(p, D, causal, grid, s); return FB_OK;
    case 4: launch_pair<DB, 4>(p, D, causal, grid, s); return FB_OK;
  }
  return FB_EUNSUPPORTED;
}

}  // namespace

fb_status launch_attention_bwd_delta_f32(const void* o, const int64_t so[3], const void* dout, const int64_t sdo[3],
                                         int B, int H, int N, int D, float* delta, hipStream_t s) {
  const int64_t rows = (int64_t)B * H * N;
  const int grid = (int)std::min<int64_t>((rows + 255) / 256, 8192);
  hipLaunchKernelGGL(delta_f32_kernel, dim3(grid), dim3(256), 0, s, (const float*)o, so[0], so[1], so[2],
                     (const float*)dout, sdo[0], sdo[1], sdo[2], B, H, N, D, delta);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention backward preparation failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

fb_status launch_attention_bwd_f32(const BwdParams& p, int D, hipStream_t s) {
  if (D != 16 && D != 32 && D != 64) return FB_EUNSUPPORTED;
  const int CB = (D + p.R + 31) / 32;
  const bool causal = (p.flags & FLAG_CAUSAL) != 0;
  const dim3 grid((unsigned)(p.nblk * p.H * p.B));
  const fb_status st = D <= 32 ? launch_cb<1>(p, D, CB, causal, grid, s) : launch_cb<2>(p, D, CB, causal, grid, s);
  if (st != FB_OK) return st;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("attention backward launch failed: %s", hipGetErrorString(e));
    return FB_EHIP;
  }
  return FB_OK;
}

}  // namespace fb
