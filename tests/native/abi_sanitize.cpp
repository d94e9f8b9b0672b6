// Driver for the host sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer) of the
// C-ABI layer and the host SVD: argument validation of every entry point, workspace sizes, and
// the truncated SVD on small matrices with known structure.  Exits non-zero on a failed check;
// the sanitizers abort on a memory or UB error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "fb.h"

static int g_fail = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::printf("FAILED line %d: %s (%s)\n", __LINE__, #c, fb_last_error()); \
      ++g_fail;                                                               \
    }                                                                         \
  } while (0)

static void* const FAKE = (void*)(uintptr_t)0x10000;   // aligned, never dereferenced

static fb_attn_args args(int B, int H, int N, int D, fb_dtype dt) {
  fb_attn_args a{};
  a.B = B;
  a.H = H;
  a.N = N;
  a.D = D;
  a.dt = dt;
  a.scale = 0.125f;
  a.q = a.k = a.v = FAKE;
  a.o = FAKE;
  const int64_t st[3] = {(int64_t)H * N * D, (int64_t)N * D, D};
  for (int i = 0; i < 3; ++i) a.sq[i] = a.sk[i] = a.sv[i] = a.so[i] = st[i];
  return a;
}

static void validation() {
  for (int s = 0; s <= 4; ++s) CHECK(fb_status_str((fb_status)s) != nullptr);
  const int64_t sp[3] = {0, 0, 64};
  fb_attn_args a = args(2, 3, 100, 64, FB_BF16);
  CHECK(fb_attn_fwd_lowrank(nullptr, nullptr, nullptr, FB_BF16, 0, nullptr, nullptr, nullptr) == FB_EINVAL);
  fb_attn_args b = a;
  b.D = 48;
  CHECK(fb_attn_fwd_lowrank(&b, nullptr, nullptr, FB_BF16, 0, nullptr, nullptr, nullptr) == FB_EUNSUPPORTED);
  b = a;
  b.q = (void*)((uintptr_t)FAKE + 8);
  CHECK(fb_attn_fwd_lowrank(&b, nullptr, nullptr, FB_BF16, 0, nullptr, nullptr, nullptr) == FB_EINVAL);
  b = a;
  b.N = -1;
  CHECK(fb_attn_fwd_lowrank_log2(&b, nullptr, nullptr, FB_BF16, 0, nullptr, nullptr, nullptr) == FB_EINVAL);
  CHECK(fb_attn_fwd_lowrank(&a, FAKE, FAKE, FB_F16, 200, sp, sp, nullptr) == FB_EUNSUPPORTED);   // R above 128
  CHECK(fb_attn_fwd_densebias(&a, nullptr, FB_BF16, sp, nullptr) == FB_EINVAL);
  b = a;
  b.dt = FB_F32;
  CHECK(fb_attn_fwd_alibi(&b, nullptr, nullptr) == FB_EUNSUPPORTED);
  // a valid request reaches the (stubbed) launcher
  CHECK(fb_attn_fwd_lowrank(&a, nullptr, nullptr, FB_BF16, 0, nullptr, nullptr, nullptr) == FB_EUNSUPPORTED);
  b = a;
  b.N = 0;
  CHECK(fb_attn_fwd_lowrank(&b, nullptr, nullptr, FB_BF16, 0, nullptr, nullptr, nullptr) == FB_OK);

  CHECK(fb_make_factors(FB_SANDWICH, 1, 64, 3, nullptr, FB_F16, 1, FAKE, FAKE, 16, nullptr, nullptr) == FB_EINVAL);
  CHECK(fb_make_factors(FB_ALIBI, 4, 64, 0, nullptr, FB_F16, 4, FAKE, FAKE, 16, nullptr, nullptr) == FB_EINVAL);
  int used = -1;
  CHECK(fb_make_factors_log2(FB_ALIBI, 4, 64, 0, nullptr, FB_F16, 2, FAKE, FAKE, 4, &used, nullptr) == FB_EINVAL);
  CHECK(fb_make_dense_bias(FB_ALIBI, 4, 64, 0, nullptr, FB_BF16, nullptr, 64 * 64, 64, nullptr) == FB_EINVAL);

  // multiplicative bias: workspace sizes, validation
  CHECK(fb_mulbias_workspace_bytes(&a, 0) == 0);
  const size_t ws = fb_mulbias_workspace_bytes(&a, 2);
  CHECK(ws >= (size_t)2 * 2 * 3 * 100 * 64 * 2 * 2);
  CHECK(fb_attn_fwd_mulbias(&a, FAKE, FAKE, FB_F32, 4, sp, sp, FAKE, ws, nullptr) == FB_EUNSUPPORTED);   // 3 D > 128
  CHECK(fb_attn_fwd_mulbias(&a, FAKE, FAKE, FB_F32, 2, sp, sp, nullptr, ws, nullptr) == FB_EINVAL);

  // backward: workspace sizes and validation
  const int64_t shared[3] = {0, 0, 8};
  const int64_t full[3] = {3 * 100 * 8, 100 * 8, 8};
  CHECK(fb_attn_bwd_workspace_bytes(2, 3, 100, 8, shared, full) == 2560 + 19200);
  CHECK(fb_attn_bwd_workspace_bytes(-1, 3, 100, 8, shared, full) == 0);
  fb_attn_bwd_args g{};
  g.dout = g.dq = g.dk = g.dv = FAKE;
  g.dphi_q = g.dphi_k = (float*)FAKE;
  for (int i = 0; i < 3; ++i) {
    g.sdo[i] = g.sdq[i] = g.sdk[i] = g.sdv[i] = a.sq[i];
    g.sdphi_q[i] = g.sdphi_k[i] = shared[i];
  }
  g.work = FAKE;
  g.work_bytes = 1 << 20;
  CHECK(fb_attn_bwd_lowrank(&a, FAKE, FAKE, FB_F16, 8, sp, sp, &g, nullptr) == FB_EINVAL);   // no LSE
  b = a;
  b.lse = (float*)FAKE;
  CHECK(fb_attn_bwd_lowrank(&b, FAKE, FAKE, FB_F16, 72, sp, sp, &g, nullptr) == FB_EUNSUPPORTED);   // R > 64
  CHECK(fb_attn_bwd_lowrank(&b, FAKE, FAKE, FB_F16, 12, sp, sp, &g, nullptr) == FB_EINVAL);   // row stride < R
  // R = 12: Delta, two padded 16-bit factor copies and two padded fp32 gradient buffers
  CHECK(fb_attn_bwd_workspace_bytes(2, 3, 100, 12, shared, full) == 2560 + 2 * 19200 + 2 * 38400);
  g.work_bytes = 64;
  CHECK(fb_attn_bwd_lowrank(&b, FAKE, FAKE, FB_F16, 8, sp, sp, &g, nullptr) == FB_EINVAL);
}

// b = U diag(s) V^T with random orthonormal U, V (Gram-Schmidt on Gaussian columns)
static std::vector<double> with_singular_values(int N, const std::vector<double>& s, unsigned seed) {
  std::mt19937_64 rng(seed);
  std::normal_distribution<double> nd;
  const int r = (int)s.size();
  std::vector<double> U((size_t)N * r), V((size_t)N * r);
  for (auto* M : {&U, &V}) {
    for (auto& x : *M) x = nd(rng);
    for (int c = 0; c < r; ++c) {
      for (int p = 0; p < c; ++p) {
        double d = 0;
        for (int i = 0; i < N; ++i) d += (*M)[(size_t)i * r + c] * (*M)[(size_t)i * r + p];
        for (int i = 0; i < N; ++i) (*M)[(size_t)i * r + c] -= d * (*M)[(size_t)i * r + p];
      }
      double n = 0;
      for (int i = 0; i < N; ++i) n += (*M)[(size_t)i * r + c] * (*M)[(size_t)i * r + c];
      n = std::sqrt(n);
      for (int i = 0; i < N; ++i) (*M)[(size_t)i * r + c] /= n;
    }
  }
  std::vector<double> b((size_t)N * N, 0.0);
  for (int i = 0; i < N; ++i)
    for (int j = 0; j < N; ++j) {
      double acc = 0;
      for (int c = 0; c < r; ++c) acc += U[(size_t)i * r + c] * s[c] * V[(size_t)j * r + c];
      b[(size_t)i * N + j] = acc;
    }
  return b;
}

static void svd() {
  const int N = 96;
  const std::vector<double> s = {5.0, 3.0, 2.0, 1.0, 0.5, 0.25};
  const std::vector<double> b = with_singular_values(N, s, 7);
  const double total = 5 * 5 + 3 * 3 + 2 * 2 + 1 + 0.25 + 0.0625;
  for (int R : {1, 3, 6}) {
    std::vector<double> pq((size_t)N * R), pk((size_t)N * R), sig(R), pq2((size_t)N * R);
    double en = -1, en2 = -1;
    CHECK(fb_svd_factors(b.data(), N, R, 11, pq.data(), pk.data(), sig.data(), &en) == FB_OK);
    CHECK(fb_svd_factors_log2(b.data(), N, R, 11, pq2.data(), nullptr, nullptr, &en2) == FB_EINVAL);   // null phi_k
    double kept = 0;
    for (int r = 0; r < R; ++r) {
      CHECK(std::fabs(sig[r] - s[r]) < 1e-9);
      kept += s[r] * s[r];
    }
    CHECK(std::fabs(en - kept / total) < 1e-12);
    // residual^2 = total - kept (Eckart-Young for the exact singular values chosen here)
    double res = 0;
    for (int i = 0; i < N; ++i)
      for (int j = 0; j < N; ++j) {
        double x = b[(size_t)i * N + j];
        for (int r = 0; r < R; ++r) x -= pq[(size_t)i * R + r] * pk[(size_t)j * R + r];
        res += x * x;
      }
    CHECK(std::fabs(res - (total - kept)) < 1e-9);
    std::vector<double> pk2((size_t)N * R);
    CHECK(fb_svd_factors_log2(b.data(), N, R, 11, pq2.data(), pk2.data(), nullptr, nullptr) == FB_OK);
    for (size_t t = 0; t < pq.size(); ++t) CHECK(std::fabs(pq2[t] - 1.4426950408889634 * pq[t]) <= 1e-15 * std::fabs(pq2[t]) + 1e-300);
  }
  int R = 0, hit = -1;
  double e = 0;
  CHECK(fb_svd_rank_for_energy(b.data(), N, 6, 0.95, 3, &R, &e, &hit) == FB_OK);
  CHECK(R == 3 && hit == 1);   // energies 25, 9, 4, ... of 39.3125: 34 < 95%, 38 >= 95%
  CHECK(fb_svd_factors(b.data(), N, N + 1, 0, nullptr, nullptr, nullptr, nullptr) == FB_EINVAL);
}

int main() {
  validation();
  svd();
  std::printf("%s: %d failed checks\n", g_fail ? "FAIL" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
