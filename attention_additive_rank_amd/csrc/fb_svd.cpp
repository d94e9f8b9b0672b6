// Host truncated SVD of a general bias matrix: the "SVD decomposition" path of
// FlashBias for static (e.g. learned) biases, done offline once per layer/head
// (FlashBias rebuttal, answer to Reviewer xU4x, Q6), which yields the factors
// phi_q = U_R sqrt(S_R), phi_k = V_R sqrt(S_R) of the best rank-R approximation.
//
// Method (randomized subspace iteration, Halko, Martinsson & Tropp, SIAM Review
// 2011, Algorithms 4.4 / 5.1):
//   1. Omega: N x l Gaussian test matrix, l = R + oversampling.
//   2. Q = orth(A Omega); repeat  Z = orth(A^T Q), Q = orth(A Z)  until the top-R
//      Ritz values settle (relative change <= 1e-13) or an iteration cap.
//   3. Bt = A^T Q (N x l) = B^T with B = Q^T A; a one-sided (Hestenes) Jacobi SVD
//      of Bt gives Bt = Ut S J^T, so A ~ Q B = (Q J) S Ut^T: U = Q J, V = Ut.
// Orthonormalisation uses Householder QR.  Dense products run on all host cores.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include <sched.h>

#include "fb_internal.h"

namespace fb {
namespace {

int host_threads() {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    const int n = CPU_COUNT(&set);
    if (n > 0) return std::min(n, 64);
  }
  const unsigned n = std::thread::hardware_concurrency();
  return n ? (int)std::min(n, 64u) : 1;
}

template <typename F>
void parallel_for(int n, F&& f) {
  const int nt = std::min(host_threads(), std::max(1, n / 16));
  if (nt <= 1) {
    f(0, n);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(nt);
  for (int t = 0; t < nt; ++t) {
    const int lo = (int)((int64_t)n * t / nt), hi = (int)((int64_t)n * (t + 1) / nt);
    th.emplace_back([&f, lo, hi] { f(lo, hi); });
  }
  for (auto& x : th) x.join();
}

// Y (N x l) = A (N x N, row-major) X (N x l)
void mul_AX(const double* A, int N, const double* X, int l, double* Y) {
  parallel_for(N, [&](int lo, int hi) {
    for (int i = lo; i < hi; ++i) {
      double* y = Y + (int64_t)i * l;
      std::fill(y, y + l, 0.0);
      const double* a = A + (int64_t)i * N;
      for (int r = 0; r < N; ++r) {
        const double ar = a[r];
        const double* x = X + (int64_t)r * l;
        for (int c = 0; c < l; ++c) y[c] += ar * x[c];
      }
    }
  });
}

// Y (N x l) = A^T X, accumulated row by row of A so that A is read contiguously
void mul_AtX(const double* A, int N, const double* X, int l, double* Y) {
  parallel_for(N, [&](int lo, int hi) {
    for (int i = lo; i < hi; ++i) std::fill(Y + (int64_t)i * l, Y + (int64_t)(i + 1) * l, 0.0);
    for (int r = 0; r < N; ++r) {
      const double* a = A + (int64_t)r * N;
      const double* x = X + (int64_t)r * l;
      for (int i = lo; i < hi; ++i) {
        const double ari = a[i];
        double* y = Y + (int64_t)i * l;
        for (int c = 0; c < l; ++c) y[c] += ari * x[c];
      }
    }
  });
}

// In place: M (N x l, row-major, N >= l) <- Q, the thin orthonormal factor of M = Q R
// (Householder reflections, then Q = H_1 ... H_l [I; 0]).
void orthonormalize(double* M, int N, int l) {
  std::vector<double> V((size_t)N * l, 0.0);  // Householder vectors (column k in V[:, k])
  std::vector<double> beta(l, 0.0);
  for (int k = 0; k < l; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < N; ++i) norm2 += M[(int64_t)i * l + k] * M[(int64_t)i * l + k];
    const double norm = std::sqrt(norm2);
    const double x0 = M[(int64_t)k * l + k];
    const double alpha = (x0 >= 0.0) ? -norm : norm;
    // v = x - alpha e_1
    double vnorm2 = 0.0;
    for (int i = k; i < N; ++i) {
      const double vi = M[(int64_t)i * l + k] - (i == k ? alpha : 0.0);
      V[(int64_t)i * l + k] = vi;
      vnorm2 += vi * vi;
    }
    beta[k] = vnorm2 > 0.0 ? 2.0 / vnorm2 : 0.0;
    // apply H_k = I - beta v v^T to the remaining columns
    for (int c = k; c < l; ++c) {
      double dot = 0.0;
      for (int i = k; i < N; ++i) dot += V[(int64_t)i * l + k] * M[(int64_t)i * l + c];
      const double f = beta[k] * dot;
      for (int i = k; i < N; ++i) M[(int64_t)i * l + c] -= f * V[(int64_t)i * l + k];
    }
  }
  // form Q: start from [I; 0] and apply H_l ... H_1 from the left
  std::fill(M, M + (int64_t)N * l, 0.0);
  for (int k = 0; k < l; ++k) M[(int64_t)k * l + k] = 1.0;
  for (int k = l - 1; k >= 0; --k) {
    for (int c = 0; c < l; ++c) {
      double dot = 0.0;
      for (int i = k; i < N; ++i) dot += V[(int64_t)i * l + k] * M[(int64_t)i * l + c];
      const double f = beta[k] * dot;
      if (f != 0.0)
        for (int i = k; i < N; ++i) M[(int64_t)i * l + c] -= f * V[(int64_t)i * l + k];
    }
  }
}

// One-sided Jacobi on G (N x l, row-major): rotates column pairs until they are
// mutually orthogonal; J (l x l) accumulates the rotations.  On return the
// columns of G are S_c * u_c and G_in = G_out J^T.
void hestenes(double* G, int N, int l, double* J) {
  std::fill(J, J + (int64_t)l * l, 0.0);
  for (int i = 0; i < l; ++i) J[(int64_t)i * l + i] = 1.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < l - 1; ++p) {
      for (int q = p + 1; q < l; ++q) {
        double a = 0.0, b = 0.0, g = 0.0;
        for (int i = 0; i < N; ++i) {
          const double x = G[(int64_t)i * l + p], y = G[(int64_t)i * l + q];
          a += x * x;
          b += y * y;
          g += x * y;
        }
        if (a == 0.0 || b == 0.0) continue;
        const double rel = std::fabs(g) / std::sqrt(a * b);
        off = std::max(off, rel);
        if (rel < 1e-14) continue;
        const double zeta = (b - a) / (2.0 * g);
        const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = c * t;
        for (int i = 0; i < N; ++i) {
          const double x = G[(int64_t)i * l + p], y = G[(int64_t)i * l + q];
          G[(int64_t)i * l + p] = c * x - s * y;
          G[(int64_t)i * l + q] = s * x + c * y;
        }
        for (int i = 0; i < l; ++i) {
          const double x = J[(int64_t)i * l + p], y = J[(int64_t)i * l + q];
          J[(int64_t)i * l + p] = c * x - s * y;
          J[(int64_t)i * l + q] = s * x + c * y;
        }
      }
    }
    if (off < 1e-12) break;  // one more sweep already ran below this level
  }
}

struct Rng {  // splitmix64 + Box-Muller
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
  double normal() {
    const double u = uniform(), v = uniform();
    return std::sqrt(-2.0 * std::log(u)) * std::cos(6.283185307179586 * v);
  }
};

// Ritz values and vectors of A restricted to span(Q): sigma (l), U = Q J (N x l), V (N x l), sorted.
void ritz(const double* A, int N, const double* Q, int l, std::vector<double>& sigma, std::vector<double>* U,
          std::vector<double>* V) {
  std::vector<double> Bt((size_t)N * l), J((size_t)l * l);
  mul_AtX(A, N, Q, l, Bt.data());  // Bt = A^T Q = (Q^T A)^T
  hestenes(Bt.data(), N, l, J.data());
  std::vector<double> s(l);
  for (int c = 0; c < l; ++c) {
    double n2 = 0.0;
    for (int i = 0; i < N; ++i) n2 += Bt[(int64_t)i * l + c] * Bt[(int64_t)i * l + c];
    s[c] = std::sqrt(n2);
  }
  std::vector<int> ord(l);
  for (int c = 0; c < l; ++c) ord[c] = c;
  std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return s[x] > s[y]; });
  sigma.resize(l);
  for (int c = 0; c < l; ++c) sigma[c] = s[ord[c]];
  if (U && V) {
    U->assign((size_t)N * l, 0.0);
    V->assign((size_t)N * l, 0.0);
    for (int c = 0; c < l; ++c) {
      const int oc = ord[c];
      const double inv = s[oc] > 0.0 ? 1.0 / s[oc] : 0.0;
      for (int i = 0; i < N; ++i) (*V)[(int64_t)i * l + c] = Bt[(int64_t)i * l + oc] * inv;
      for (int i = 0; i < N; ++i) {
        double acc = 0.0;
        for (int r = 0; r < l; ++r) acc += Q[(int64_t)i * l + r] * J[(int64_t)r * l + oc];
        (*U)[(int64_t)i * l + c] = acc;
      }
    }
  }
}

}  // namespace

fb_status svd_factors(const double* A, int N, int R, uint64_t seed, double* phq, double* phk, double* sigma_out,
                      double* energy_out) {
  const int l = std::min(N, R + std::max(R, 10));
  std::vector<double> Q((size_t)N * l), Z((size_t)N * l);
  Rng rng{seed ^ 0x243F6A8885A308D3ull};
  for (auto& x : Z) x = rng.normal();
  mul_AX(A, N, Z.data(), l, Q.data());
  orthonormalize(Q.data(), N, l);
  std::vector<double> sig, prev;
  const int max_iter = 300;
  for (int it = 0; it < max_iter; ++it) {
    mul_AtX(A, N, Q.data(), l, Z.data());
    orthonormalize(Z.data(), N, l);
    mul_AX(A, N, Z.data(), l, Q.data());
    orthonormalize(Q.data(), N, l);
    if (it % 2 == 1) {
      ritz(A, N, Q.data(), l, sig, nullptr, nullptr);
      if (!prev.empty()) {
        double change = 0.0;
        for (int r = 0; r < R; ++r) change = std::max(change, std::fabs(sig[r] - prev[r]));
        if (change <= 1e-13 * std::max(sig[0], 1e-300)) break;
      }
      prev = sig;
    }
  }
  std::vector<double> U, V;
  ritz(A, N, Q.data(), l, sig, &U, &V);
  for (int i = 0; i < N; ++i)
    for (int r = 0; r < R; ++r) {
      const double root = std::sqrt(sig[r]);
      phq[(int64_t)i * R + r] = U[(int64_t)i * l + r] * root;
      phk[(int64_t)i * R + r] = V[(int64_t)i * l + r] * root;
    }
  if (sigma_out)
    for (int r = 0; r < R; ++r) sigma_out[r] = sig[r];
  if (energy_out) {
    double tot = 0.0;
    for (int64_t t = 0; t < (int64_t)N * N; ++t) tot += A[t] * A[t];
    double kept = 0.0;
    for (int r = 0; r < R; ++r) kept += sig[r] * sig[r];
    *energy_out = tot > 0.0 ? kept / tot : 1.0;
  }
  return FB_OK;
}

}  // namespace fb
