// C ABI of libflashbias: argument validation and dispatch.  Every check runs
// before any launch; nothing here allocates device memory.
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <new>
#include <vector>
#include <algorithm>

#include "fb_internal.h"

namespace fb {

fb_status svd_factors(const double* A, int N, int R, uint64_t seed, double* phq, double* phk, double* sigma,
                      double* energy);

namespace {
thread_local char g_err[512] = "";

int esize(fb_dtype t) { return t == FB_F32 ? 4 : 2; }
bool known_dtype(fb_dtype t) { return t == FB_F32 || t == FB_BF16 || t == FB_F16; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define FB_FAIL(code, ...)      \
  do {                          \
    set_error(__VA_ARGS__);     \
    return code;                \
  } while (0)

// Strides of a [B][H][N][X] tensor whose rows start on 16-byte boundaries.
bool rows_aligned(const int64_t s[3], int es) {
  const int64_t ce = 16 / es;
  return s[0] % ce == 0 && s[1] % ce == 0 && s[2] % ce == 0;
}

// Element strides and the extent of one (b, h) slice must fit in 32-bit offsets.
bool strides_fit32(const int64_t s[3], int N) {
  const int64_t lim = 0x7fffffffLL;
  return s[0] <= lim && s[1] <= lim && s[2] <= lim && (int64_t)N * s[2] <= lim;
}

// A key tile of rows with this element stride spans fewer than 2^31 bytes.
bool tile_fits32(int64_t row_stride, int es) { return (int64_t)kAttnKeyTile * row_stride * es <= 0x7fffffffLL; }

fb_status check_common(const fb_attn_args* a, const char* fn) {
  if (!a) FB_FAIL(FB_EINVAL, "%s: null argument struct", fn);
  if (a->B < 0 || a->H < 0 || a->N < 0) FB_FAIL(FB_EINVAL, "%s: negative size", fn);
  if (!known_dtype(a->dt)) FB_FAIL(FB_EUNSUPPORTED, "%s: unknown dtype %d", fn, (int)a->dt);
  if (a->D != 16 && a->D != 32 && a->D != 64 && a->D != 128)
    FB_FAIL(FB_EUNSUPPORTED, "%s: head dim %d not in {16,32,64,128}", fn, a->D);
  if (a->dt == FB_F32 && a->D > 64) FB_FAIL(FB_EUNSUPPORTED, "%s: fp32 supports head dims <= 64", fn);
  if ((int64_t)a->B * a->H * a->N == 0) return FB_OK;
  if (!a->q || !a->k || !a->v || !a->o) FB_FAIL(FB_EINVAL, "%s: null q/k/v/o", fn);
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    FB_FAIL(FB_EINVAL, "%s: q/k/v/o must be 16-byte aligned", fn);
  const int es = esize(a->dt);
  const int64_t* st[4] = {a->sq, a->sk, a->sv, a->so};
  const char* nm[4] = {"q", "k", "v", "o"};
  for (int i = 0; i < 4; ++i) {
    if (st[i][0] < 0 || st[i][1] < 0 || st[i][2] < 0) FB_FAIL(FB_EINVAL, "%s: negative %s stride", fn, nm[i]);
    if (!rows_aligned(st[i], es)) FB_FAIL(FB_EINVAL, "%s: %s strides must be multiples of %d elements", fn, nm[i], 16 / es);
    if (a->N > 1 && st[i][2] < a->D) FB_FAIL(FB_EINVAL, "%s: %s row stride < D", fn, nm[i]);
  }
  if (a->lse && ((uintptr_t)a->lse & 3u)) FB_FAIL(FB_EINVAL, "%s: lse must be 4-byte aligned", fn);
  if (!std::isfinite(a->scale)) FB_FAIL(FB_EINVAL, "%s: scale must be finite", fn);
  const int64_t nqb = (a->N + kAttnBlockM - 1) / kAttnBlockM;
  if (nqb * a->H * a->B > 0x7fffffffLL) FB_FAIL(FB_EUNSUPPORTED, "%s: grid too large", fn);
  for (int i = 0; i < 4; ++i)
    if (!strides_fit32(st[i], a->N)) FB_FAIL(FB_EUNSUPPORTED, "%s: %s strides exceed 32 bits", fn, nm[i]);
  // key rows are addressed by 32-bit byte offsets within one key tile
  if (!tile_fits32(a->sk[2], es) || !tile_fits32(a->sv[2], es))
    FB_FAIL(FB_EUNSUPPORTED, "%s: k/v row strides too large", fn);
  return FB_OK;
}

fb_status dispatch_attention(int mode, fb_dtype dt, fb_dtype aux, int D, int RP, const AttnParams& p,
                             hipStream_t s) {
#define FB_DISPATCH_D(d)                                                   \
  case d:                                                                  \
    if (dt == FB_BF16) return launch_attention_d##d##_bf16(mode, aux, RP, p, s); \
    if (dt == FB_F16) return launch_attention_d##d##_f16(mode, aux, RP, p, s);   \
    return launch_attention_d##d##_f32(mode, aux, RP, p, s);
  switch (D) {
    FB_DISPATCH_D(16)
    FB_DISPATCH_D(32)
    FB_DISPATCH_D(64)
    FB_DISPATCH_D(128)
  }
#undef FB_DISPATCH_D
  return FB_EUNSUPPORTED;
}

AttnParams base_params(const fb_attn_args* a) {
  AttnParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  for (int i = 0; i < 3; ++i) {
    p.sq[i] = (int)a->sq[i];
    p.sk[i] = (int)a->sk[i];
    p.sv[i] = (int)a->sv[i];
    p.so[i] = (int)a->so[i];
  }
  p.B = a->B;
  p.H = a->H;
  p.N = a->N;
  p.flags = a->causal ? FLAG_CAUSAL : 0;
  p.scale = a->scale;
  p.nqb = (a->N + kAttnBlockM - 1) / kAttnBlockM;
  return p;
}

}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

BwdWork bwd_work_layout(int B, int H, int N, int R, const int64_t sdphi_q[3], const int64_t sdphi_k[3]) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  // a factor gradient needs per-(b, h) partials when an axis of size > 1 has stride 0
  auto summed = [&](const int64_t* sd) { return R > 0 && ((sd[0] == 0 && B > 1) || (sd[1] == 0 && H > 1)); };
  const size_t rows = (size_t)B * H * N;
  BwdWork w{0, SIZE_MAX, SIZE_MAX, up(rows * 4), SIZE_MAX, SIZE_MAX, 0};
  if (R > 0 && R % 8 != 0) {
    // padded factors (16-bit) and per-(b, h) padded factor gradients (fp32)
    w.R8 = (R + 7) / 8 * 8;
    const size_t fb16 = up(rows * (size_t)w.R8 * 2), fb32 = up(rows * (size_t)w.R8 * 4);
    w.phq_off = w.bytes;
    w.phk_off = w.phq_off + fb16;
    w.pq_off = w.phk_off + fb16;
    w.pk_off = w.pq_off + fb32;
    w.bytes = w.pk_off + fb32;
    if (rows == 0) w.bytes = 0;
    return w;
  }
  if (summed(sdphi_q)) {
    w.pq_off = w.bytes;
    w.bytes += up(rows * (size_t)R * 4);
  }
  if (summed(sdphi_k)) {
    w.pk_off = w.bytes;
    w.bytes += up(rows * (size_t)R * 4);
  }
  if (rows == 0) w.bytes = 0;
  return w;
}

}  // namespace fb

using namespace fb;

extern "C" {

const char* fb_status_str(fb_status st) {
  switch (st) {
    case FB_OK: return "FB_OK";
    case FB_EINVAL: return "FB_EINVAL: invalid argument";
    case FB_EUNSUPPORTED: return "FB_EUNSUPPORTED: unsupported configuration";
    case FB_EHIP: return "FB_EHIP: HIP runtime error";
    case FB_ENOMEM: return "FB_ENOMEM: out of host memory";
  }
  return "unknown fb_status";
}

const char* fb_last_error(void) { return g_err; }

}  // extern "C"

namespace {

fb_status make_factors(const char* fn, double qscale, fb_bias_kind kind, int H, int N, int C,
                       const double* slopes_host, fb_dtype out_dt, int split, void* phi_q, void* phi_k, int R_pad,
                       int* R_used, hipStream_t stream) {
  if (kind != FB_ALIBI && kind != FB_SANDWICH) FB_FAIL(FB_EINVAL, "%s: unknown bias kind", fn);
  if (!known_dtype(out_dt)) FB_FAIL(FB_EINVAL, "%s: unknown dtype", fn);
  if (H < 1 || N < 1) FB_FAIL(FB_EINVAL, "%s: H and N must be >= 1", fn);
  if (kind == FB_SANDWICH && (C < 2 || C % 2)) FB_FAIL(FB_EINVAL, "%s: Sandwich needs an even C >= 2", fn);
  if (split < 1 || split > 3) FB_FAIL(FB_EINVAL, "%s: split must be 1, 2 or 3", fn);
  if (kind == FB_ALIBI && slopes_host && H > kMaxSlopes)
    FB_FAIL(FB_EUNSUPPORTED, "%s: explicit slopes limited to %d heads", fn, kMaxSlopes);
  const int r_nat = kind == FB_ALIBI ? 2 : C;
  const int used = r_nat * split * (split + 1) / 2;
  if (R_used) *R_used = used;
  if (R_pad < used) FB_FAIL(FB_EINVAL, "%s: R_pad %d < %d columns needed", fn, R_pad, used);
  if (!phi_q || !phi_k) FB_FAIL(FB_EINVAL, "%s: null factor pointer", fn);
  if (!aligned16(phi_q) || !aligned16(phi_k)) FB_FAIL(FB_EINVAL, "%s: factor pointers must be 16-byte aligned", fn);
  if ((int64_t)H * N * R_pad > 0x7fffffffLL) FB_FAIL(FB_EUNSUPPORTED, "%s: H N R_pad must stay below 2^31", fn);
  return launch_make_factors(kind, H, N, C, kind == FB_ALIBI ? slopes_host : nullptr, out_dt, split, phi_q,
                             phi_k, R_pad, r_nat, qscale, stream);
}

}  // namespace

extern "C" {

fb_status fb_make_factors(fb_bias_kind kind, int H, int N, int C, const double* slopes_host, fb_dtype out_dt,
                          int split, void* phi_q, void* phi_k, int R_pad, int* R_used, hipStream_t stream) {
  return make_factors("fb_make_factors", 1.0, kind, H, N, C, slopes_host, out_dt, split, phi_q, phi_k, R_pad,
                      R_used, stream);
}

fb_status fb_make_factors_log2(fb_bias_kind kind, int H, int N, int C, const double* slopes_host, fb_dtype out_dt,
                               int split, void* phi_q, void* phi_k, int R_pad, int* R_used, hipStream_t stream) {
  // log2(e) = 1 / ln 2 in double
  return make_factors("fb_make_factors_log2", 1.4426950408889634074, kind, H, N, C, slopes_host, out_dt, split,
                      phi_q, phi_k, R_pad, R_used, stream);
}

fb_status fb_make_dense_bias(fb_bias_kind kind, int H, int N, int C, const double* slopes_host, fb_dtype out_dt,
                             void* bias, int64_t head_stride, int64_t row_stride, hipStream_t stream) {
  const char* fn = "fb_make_dense_bias";
  if (kind != FB_ALIBI && kind != FB_SANDWICH) FB_FAIL(FB_EINVAL, "%s: unknown bias kind", fn);
  if (!known_dtype(out_dt)) FB_FAIL(FB_EINVAL, "%s: unknown dtype", fn);
  if (H < 1 || N < 1) FB_FAIL(FB_EINVAL, "%s: H and N must be >= 1", fn);
  if (kind == FB_SANDWICH && (C < 2 || C % 2)) FB_FAIL(FB_EINVAL, "%s: Sandwich needs an even C >= 2", fn);
  if (!bias) FB_FAIL(FB_EINVAL, "%s: null bias", fn);
  if (((uintptr_t)bias % esize(out_dt)) != 0) FB_FAIL(FB_EINVAL, "%s: misaligned bias", fn);
  if (row_stride < N) FB_FAIL(FB_EINVAL, "%s: row_stride < N", fn);
  if (H > 1 && head_stride < (int64_t)N * row_stride) FB_FAIL(FB_EINVAL, "%s: head_stride too small", fn);
  if (kind == FB_ALIBI && slopes_host && H > kMaxSlopes)
    FB_FAIL(FB_EUNSUPPORTED, "%s: explicit slopes limited to %d heads", fn, kMaxSlopes);
  return launch_make_dense_bias(kind, H, N, C, kind == FB_ALIBI ? slopes_host : nullptr, out_dt, bias,
                                head_stride, row_stride, stream);
}

fb_status fb_svd_factors(const double* bias, int N, int R, uint64_t seed, double* phi_q, double* phi_k,
                         double* sigma, double* energy) {
  const char* fn = "fb_svd_factors";
  if (!bias || !phi_q || !phi_k) FB_FAIL(FB_EINVAL, "%s: null pointer", fn);
  if (N < 1 || R < 1 || R > N) FB_FAIL(FB_EINVAL, "%s: need 1 <= R <= N", fn);
  try {
    return svd_factors(bias, N, R, seed, phi_q, phi_k, sigma, energy);
  } catch (const std::bad_alloc&) {
    FB_FAIL(FB_ENOMEM, "%s: out of host memory", fn);
  } catch (...) {
    FB_FAIL(FB_EINVAL, "%s: internal error", fn);
  }
}

fb_status fb_svd_factors_log2(const double* bias, int N, int R, uint64_t seed, double* phi_q, double* phi_k,
                              double* sigma, double* energy) {
  const fb_status st = fb_svd_factors(bias, N, R, seed, phi_q, phi_k, sigma, energy);
  if (st != FB_OK) return st;
  // phi_q in exp2 units, scaled in fp64 before the caller rounds it
  const double log2e = 1.4426950408889634074;
  for (int64_t t = 0; t < (int64_t)N * R; ++t) phi_q[t] *= log2e;
  return FB_OK;
}

fb_status fb_svd_rank_for_energy(const double* bias, int N, int R_max, double target, uint64_t seed,
                                 int* R_out, double* energy_out, int* reached) {
  const char* fn = "fb_svd_rank_for_energy";
  if (!bias || !R_out) FB_FAIL(FB_EINVAL, "%s: null pointer", fn);
  if (N < 1 || R_max < 1 || R_max > N) FB_FAIL(FB_EINVAL, "%s: need 1 <= R_max <= N", fn);
  if (!(target > 0.0 && target <= 1.0)) FB_FAIL(FB_EINVAL, "%s: need 0 < target <= 1", fn);
  try {
    std::vector<double> phq((size_t)N * R_max), phk((size_t)N * R_max), sig(R_max);
    const fb_status st = svd_factors(bias, N, R_max, seed, phq.data(), phk.data(), sig.data(), nullptr);
    if (st != FB_OK) return st;
    double total = 0.0;
    for (int64_t t = 0; t < (int64_t)N * N; ++t) total += bias[t] * bias[t];
    int R = R_max;
    double kept = 0.0, kept_at_R = 0.0;
    bool ok = false;
    for (int r = 0; r < R_max; ++r) {
      kept += sig[r] * sig[r];
      if (total <= 0.0 || kept >= target * total) {
        R = r + 1;
        kept_at_R = kept;
        ok = true;
        break;
      }
    }
    if (!ok) kept_at_R = kept;
    if (energy_out) *energy_out = total > 0.0 ? std::min(1.0, kept_at_R / total) : 1.0;
    if (reached) *reached = ok ? 1 : 0;
    *R_out = R;
    return FB_OK;
  } catch (const std::bad_alloc&) {
    FB_FAIL(FB_ENOMEM, "%s: out of host memory", fn);
  } catch (...) {
    FB_FAIL(FB_EINVAL, "%s: internal error", fn);
  }
}

}  // extern "C"

namespace {

// Both low-rank forward entry points; log2 != 0: phi_q comes in exp2 units (mode 3).
fb_status lowrank_forward(const char* fn, int log2, const fb_attn_args* a, const void* phi_q, const void* phi_k,
                          fb_dtype phi_dt, int R, const int64_t sphi_q[3], const int64_t sphi_k[3],
                          hipStream_t stream) {
  fb_status st = check_common(a, fn);
  if (st != FB_OK) return st;
  if (log2 && a->dt == FB_F32) FB_FAIL(FB_EUNSUPPORTED, "%s: q/k/v must be bf16 or f16", fn);
  if (R < 0) FB_FAIL(FB_EINVAL, "%s: negative R", fn);
  const int maxR = a->dt == FB_F32 ? 32 : 128;
  if (R > maxR) FB_FAIL(FB_EUNSUPPORTED, "%s: R = %d above the limit %d", fn, R, maxR);
  if (R > 0) {
    if (!known_dtype(phi_dt)) FB_FAIL(FB_EUNSUPPORTED, "%s: unknown factor dtype", fn);
    if ((a->dt == FB_F32) != (phi_dt == FB_F32) || (a->dt == FB_F16 && phi_dt != FB_F16))
      FB_FAIL(FB_EUNSUPPORTED, "%s: factor dtype does not match the q/k/v dtype", fn);
  }
  if ((int64_t)a->B * a->H * a->N == 0) return FB_OK;
  AttnParams p = base_params(a);
  int RP = 0;
  if (R > 0) {
    if (!phi_q || !phi_k || !sphi_q || !sphi_k) FB_FAIL(FB_EINVAL, "%s: null factor pointer or strides", fn);
    for (int i = 0; i < 3; ++i)
      if (sphi_q[i] < 0 || sphi_k[i] < 0) FB_FAIL(FB_EINVAL, "%s: negative factor stride", fn);
    if (!strides_fit32(sphi_q, a->N) || !strides_fit32(sphi_k, a->N) || !tile_fits32(sphi_k[2], esize(phi_dt)))
      FB_FAIL(FB_EUNSUPPORTED, "%s: factor strides exceed 32 bits", fn);
    if (a->N > 1 && (sphi_q[2] < R || sphi_k[2] < R)) FB_FAIL(FB_EINVAL, "%s: factor row stride < R", fn);
    const int es = esize(phi_dt);
    if (((uintptr_t)phi_q % es) || ((uintptr_t)phi_k % es)) FB_FAIL(FB_EINVAL, "%s: misaligned factors", fn);
    p.phq = phi_q;
    p.phk = phi_k;
    for (int i = 0; i < 3; ++i) {
      p.spq[i] = (int)sphi_q[i];
      p.spk[i] = (int)sphi_k[i];
    }
    p.R = R;
    if (aligned16(phi_q) && rows_aligned(sphi_q, es)) p.flags |= FLAG_PHQ_VEC;
    if (aligned16(phi_k) && rows_aligned(sphi_k, es)) p.flags |= FLAG_PHK_VEC;
    const int step = a->dt == FB_F32 ? 8 : 16;
    RP = (R + step - 1) / step * step;
    if (a->dt == FB_F32) { if (RP == 24) RP = 32; }
    else { if (RP == 48) RP = 64; else if (RP > 64) RP = 128; }
  }
  const fb_dtype aux = R > 0 ? phi_dt : a->dt;
  st = dispatch_attention(log2 ? 3 : 0, a->dt, aux, a->D, RP, p, stream);
  if (st == FB_EUNSUPPORTED) set_error("%s: no kernel for this dtype / rank combination", fn);
  return st;
}

}  // namespace

extern "C" {

fb_status fb_attn_fwd_lowrank(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt,
                              int R, const int64_t sphi_q[3], const int64_t sphi_k[3], hipStream_t stream) {
  return lowrank_forward("fb_attn_fwd_lowrank", 0, a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, stream);
}

fb_status fb_attn_fwd_lowrank_log2(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt,
                                   int R, const int64_t sphi_q[3], const int64_t sphi_k[3], hipStream_t stream) {
  return lowrank_forward("fb_attn_fwd_lowrank_log2", 1, a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, stream);
}

size_t fb_mulbias_workspace_bytes(const fb_attn_args* a, int R) {
  if (!a || R < 1 || a->B < 0 || a->H < 0 || a->N < 0 || a->D < 1) return 0;
  const size_t rows = (size_t)a->B * a->H * a->N;
  const size_t es = esize(a->dt);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t first = up(rows * a->D * es), rest = up(rows * (size_t)(R - 1) * a->D * es);
  return rows == 0 ? 0 : 2 * first + 2 * rest;
}

size_t fb_attn_bwd_workspace_bytes(int B, int H, int N, int R, const int64_t sdphi_q[3], const int64_t sdphi_k[3]) {
  if (B < 0 || H < 0 || N < 0 || R < 0 || (R > 0 && (!sdphi_q || !sdphi_k))) return 0;
  return bwd_work_layout(B, H, N, R, sdphi_q, sdphi_k).bytes;
}

}  // extern "C"

namespace {

struct MulbiasParts {
  void *q1, *k1, *pq, *pk;
};

// Validation shared by both multiplicative-bias entry points; on success, *parts locates
// the expanded operands in the workspace (nothing to do when the inputs are empty).
fb_status mulbias_check(const char* fn, const fb_attn_args* a, const void* phi_q, const void* phi_k,
                        fb_dtype phi_dt, int R, const int64_t sphi_q[3], const int64_t sphi_k[3],
                        void* workspace, size_t workspace_bytes, MulbiasParts* parts) {
  fb_status st = check_common(a, fn);
  if (st != FB_OK) return st;
  if (a->dt != FB_BF16 && a->dt != FB_F16) FB_FAIL(FB_EUNSUPPORTED, "%s: q/k/v must be bf16 or f16", fn);
  if (R < 1) FB_FAIL(FB_EINVAL, "%s: need R >= 1", fn);
  if ((int64_t)(R - 1) * a->D > 128) FB_FAIL(FB_EUNSUPPORTED, "%s: (R - 1) * D = %d above 128", fn, (R - 1) * a->D);
  if (!known_dtype(phi_dt)) FB_FAIL(FB_EUNSUPPORTED, "%s: unknown factor dtype", fn);
  parts->q1 = parts->k1 = parts->pq = parts->pk = nullptr;
  if ((int64_t)a->B * a->H * a->N == 0) return FB_OK;
  if (!phi_q || !phi_k || !sphi_q || !sphi_k) FB_FAIL(FB_EINVAL, "%s: null factor pointer or strides", fn);
  for (int i = 0; i < 3; ++i)
    if (sphi_q[i] < 0 || sphi_k[i] < 0) FB_FAIL(FB_EINVAL, "%s: negative factor stride", fn);
  if (a->N > 1 && (sphi_q[2] < R || sphi_k[2] < R)) FB_FAIL(FB_EINVAL, "%s: factor row stride < R", fn);
  if (((uintptr_t)phi_q % esize(phi_dt)) || ((uintptr_t)phi_k % esize(phi_dt)))
    FB_FAIL(FB_EINVAL, "%s: misaligned factors", fn);
  const size_t need = fb_mulbias_workspace_bytes(a, R);
  if (!workspace) FB_FAIL(FB_EINVAL, "%s: null workspace", fn);
  if ((uintptr_t)workspace & 255u) FB_FAIL(FB_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if (workspace_bytes < need) FB_FAIL(FB_EINVAL, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  const size_t rows = (size_t)a->B * a->H * a->N, es = esize(a->dt);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* w = (char*)workspace;
  parts->q1 = w;
  parts->k1 = w + up(rows * a->D * es);
  parts->pq = w + 2 * up(rows * a->D * es);
  parts->pk = (char*)parts->pq + up(rows * (size_t)(R - 1) * a->D * es);
  return FB_OK;
}

fb_status mulbias_expand(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt, int R,
                         const int64_t sphi_q[3], const int64_t sphi_k[3], const MulbiasParts& w, hipStream_t s) {
  fb_status st = launch_mulbias_expand(a->dt, phi_dt, a->q, a->sq, phi_q, sphi_q, a->B, a->H, a->N, a->D, R,
                                       a->scale, w.q1, R > 1 ? w.pq : nullptr, s);
  if (st != FB_OK) return st;
  return launch_mulbias_expand(a->dt, phi_dt, a->k, a->sk, phi_k, sphi_k, a->B, a->H, a->N, a->D, R, 1.0f, w.k1,
                               R > 1 ? w.pk : nullptr, s);
}

}  // namespace

extern "C" {

fb_status fb_mulbias_expand(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt, int R,
                            const int64_t sphi_q[3], const int64_t sphi_k[3], void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  MulbiasParts w;
  fb_status st = mulbias_check("fb_mulbias_expand", a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, workspace,
                               workspace_bytes, &w);
  if (st != FB_OK || (int64_t)a->B * a->H * a->N == 0) return st;
  return mulbias_expand(a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, w, stream);
}

fb_status fb_attn_fwd_mulbias(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt, int R,
                              const int64_t sphi_q[3], const int64_t sphi_k[3], void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "fb_attn_fwd_mulbias";
  MulbiasParts w;
  fb_status st = mulbias_check(fn, a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, workspace, workspace_bytes, &w);
  if (st != FB_OK || (int64_t)a->B * a->H * a->N == 0) return st;
  st = mulbias_expand(a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, w, stream);
  if (st != FB_OK) return st;
  fb_attn_args e = *a;
  e.q = w.q1;
  e.k = w.k1;
  e.scale = 1.0f;
  const int64_t sx[3] = {(int64_t)a->H * a->N * a->D, (int64_t)a->N * a->D, a->D};
  for (int i = 0; i < 3; ++i) {
    e.sq[i] = sx[i];
    e.sk[i] = sx[i];
  }
  const int64_t W = (int64_t)(R - 1) * a->D;
  const int64_t sf[3] = {(int64_t)a->H * a->N * W, (int64_t)a->N * W, W};
  st = fb_attn_fwd_lowrank(&e, R > 1 ? w.pq : nullptr, R > 1 ? w.pk : nullptr, a->dt, (int)W, sf, sf, stream);
  if (st != FB_OK) {
    char msg[512];
    snprintf(msg, sizeof(msg), "%s", g_err);
    set_error("%s: %s", fn, msg);
  }
  return st;
}

fb_status fb_attn_bwd_lowrank(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt, int R,
                              const int64_t sphi_q[3], const int64_t sphi_k[3], const fb_attn_bwd_args* g,
                              hipStream_t stream) {
  return fb::attn_bwd_lowrank_impl(a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, g, stream, "fb_attn_bwd_lowrank");
}

fb_status fb_attn_bwd_lowrank_log2(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt,
                                   int R, const int64_t sphi_q[3], const int64_t sphi_k[3],
                                   const fb_attn_bwd_args* g, hipStream_t stream) {
  return fb::attn_bwd_lowrank_impl(a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, g, stream, "fb_attn_bwd_lowrank_log2",
                                   true);
}
}  // extern "C"

namespace fb {
fb_status attn_bwd_lowrank_impl(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt, int R,
                                const int64_t sphi_q[3], const int64_t sphi_k[3], const fb_attn_bwd_args* g,
                                hipStream_t stream, const char* fn, bool log2) {
  fb_status st = check_common(a, fn);
  if (st != FB_OK) return st;
  if (!g) FB_FAIL(FB_EINVAL, "%s: null gradient arguments", fn);
  const bool f32 = a->dt == FB_F32;
  if (a->dt != FB_BF16 && a->dt != FB_F16 && !f32) FB_FAIL(FB_EUNSUPPORTED, "%s: q/k/v must be bf16, f16 or fp32", fn);
  if (a->D != 16 && a->D != 32 && a->D != 64 && a->D != 128)
    FB_FAIL(FB_EUNSUPPORTED, "%s: head dim %d not in {16, 32, 64, 128}", fn, a->D);
  if (f32 && a->D > 64) FB_FAIL(FB_EUNSUPPORTED, "%s: fp32 q/k/v with head dims up to 64", fn);
  if (f32 && log2) FB_FAIL(FB_EUNSUPPORTED, "%s: exp2-unit factors need bf16 or f16 q/k/v", fn);
  if (R < 0) FB_FAIL(FB_EINVAL, "%s: negative R", fn);
  if (R > 64) FB_FAIL(FB_EUNSUPPORTED, "%s: R = %d (at most 64)", fn, R);
  if (R > 0) {
    if (!known_dtype(phi_dt) || (f32 ? phi_dt != FB_F32 : phi_dt == FB_F32) || (a->dt == FB_F16 && phi_dt != FB_F16))
      FB_FAIL(FB_EUNSUPPORTED, "%s: factor dtype does not match the q/k/v dtype", fn);
  }
  if ((int64_t)a->B * a->H * a->N == 0) return FB_OK;
  if (!a->lse) FB_FAIL(FB_EINVAL, "%s: the forward LSE is required", fn);
  if (!g->dout || !g->dq || !g->dk || !g->dv || !g->work) FB_FAIL(FB_EINVAL, "%s: null dO, output or workspace", fn);
  const int es = esize(a->dt);
  const int64_t* st6[4] = {g->sdo, g->sdq, g->sdk, g->sdv};
  const void* pt[4] = {g->dout, g->dq, g->dk, g->dv};
  for (int i = 0; i < 4; ++i) {
    if (!aligned16(pt[i])) FB_FAIL(FB_EINVAL, "%s: dO/dq/dk/dv must be 16-byte aligned", fn);
    if (st6[i][0] < 0 || st6[i][1] < 0 || st6[i][2] < 0 || !rows_aligned(st6[i], es))
      FB_FAIL(FB_EINVAL, "%s: dO/dq/dk/dv strides must be non-negative multiples of %d elements", fn, 16 / es);
    if (a->N > 1 && st6[i][2] < a->D) FB_FAIL(FB_EINVAL, "%s: gradient row stride < D", fn);
    if (!strides_fit32(st6[i], a->N)) FB_FAIL(FB_EUNSUPPORTED, "%s: gradient strides exceed 32 bits", fn);
  }
  // the streamed tiles (Q and dO; K and V) address 64 rows with 32-bit offsets
  if (!tile_fits32(a->sq[2], es) || !tile_fits32(g->sdo[2], es))
    FB_FAIL(FB_EUNSUPPORTED, "%s: a 64-row tile of Q or dO spans 2^31 bytes or more", fn);
  if ((uintptr_t)g->work & 255u) FB_FAIL(FB_EINVAL, "%s: workspace not 256-byte aligned", fn);
  const BwdWork wl = bwd_work_layout(a->B, a->H, a->N, R, g->sdphi_q, g->sdphi_k);
  if (g->work_bytes < wl.bytes)
    FB_FAIL(FB_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn, g->work_bytes, wl.bytes);
  if ((wl.pq_off != SIZE_MAX || wl.pk_off != SIZE_MAX) && (int64_t)a->H * a->N * R > 0x7fffffffLL)
    FB_FAIL(FB_EUNSUPPORTED, "%s: per-(b, h) factor gradients exceed 32-bit strides", fn);
  BwdParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.dout = g->dout;
  p.lse = a->lse;
  float* const delta = (float*)g->work;
  p.delta = delta;
  p.dq = g->dq;
  p.dk = g->dk;
  p.dv = g->dv;
  for (int i = 0; i < 3; ++i) {
    p.sq[i] = (int)a->sq[i];
    p.sk[i] = (int)a->sk[i];
    p.sv[i] = (int)a->sv[i];
    p.sdo[i] = (int)g->sdo[i];
    p.sdq[i] = (int)g->sdq[i];
    p.sdk[i] = (int)g->sdk[i];
    p.sdv[i] = (int)g->sdv[i];
  }
  p.R = R;
  p.flags = (a->causal ? FLAG_CAUSAL : 0) | (log2 && R > 0 ? FLAG_LOG2 : 0);
  p.B = a->B;
  p.H = a->H;
  p.N = a->N;
  p.scale = a->scale;
  p.nblk = (a->N + kBwdRows - 1) / kBwdRows;
  if (p.nblk * (int64_t)a->H * a->B > 0x7fffffffLL) FB_FAIL(FB_EUNSUPPORTED, "%s: grid too large", fn);
  int RP = 0, RW = 0;
  if (R > 0) {
    if (!phi_q || !phi_k || !sphi_q || !sphi_k || !g->dphi_q || !g->dphi_k)
      FB_FAIL(FB_EINVAL, "%s: null factor pointer, strides or factor gradient", fn);
    for (int i = 0; i < 3; ++i)
      if (sphi_q[i] < 0 || sphi_k[i] < 0 || g->sdphi_q[i] < 0 || g->sdphi_k[i] < 0)
        FB_FAIL(FB_EINVAL, "%s: negative factor stride", fn);
    // R not a multiple of 8: 16-bit factors are copied (zero-padded) into the workspace, and
    // the factor gradients go through [B][H][N][R8] partials; the fp32 kernels read the
    // factors in place, element by element
    const bool padded = wl.R8 > 0;
    if (!f32 && !padded && (!aligned16(phi_q) || !aligned16(phi_k) || !rows_aligned(sphi_q, esize(phi_dt)) ||
                            !rows_aligned(sphi_k, esize(phi_dt))))
      FB_FAIL(FB_EUNSUPPORTED, "%s: factor rows must be 16-byte aligned", fn);
    if ((padded || f32) && (((uintptr_t)phi_q | (uintptr_t)phi_k) & (uintptr_t)(esize(phi_dt) - 1)))
      FB_FAIL(FB_EINVAL, "%s: factors not aligned to their element size", fn);
    if (a->N > 1 && (sphi_q[2] < R || sphi_k[2] < R || g->sdphi_q[2] < R || g->sdphi_k[2] < R))
      FB_FAIL(FB_EINVAL, "%s: factor row stride < R", fn);
    if (!padded && (((uintptr_t)g->dphi_q & 15u) || ((uintptr_t)g->dphi_k & 15u) || g->sdphi_q[2] % 4 ||
                    g->sdphi_k[2] % 4 || g->sdphi_q[1] % 4 || g->sdphi_k[1] % 4 || g->sdphi_q[0] % 4 ||
                    g->sdphi_k[0] % 4))
      FB_FAIL(FB_EINVAL, "%s: dphi and its strides must be 16-byte aligned", fn);
    if (padded && (((uintptr_t)g->dphi_q | (uintptr_t)g->dphi_k) & 3u))
      FB_FAIL(FB_EINVAL, "%s: dphi must be 4-byte aligned", fn);
    if (!strides_fit32(sphi_q, a->N) || !strides_fit32(sphi_k, a->N) || !strides_fit32(g->sdphi_q, a->N) ||
        !strides_fit32(g->sdphi_k, a->N) || !tile_fits32(sphi_q[2], esize(phi_dt)) ||
        !tile_fits32(sphi_k[2], esize(phi_dt)))
      FB_FAIL(FB_EUNSUPPORTED, "%s: factor strides exceed 32 bits", fn);
    if (padded && (int64_t)a->H * a->N * wl.R8 > 0x7fffffffLL)
      FB_FAIL(FB_EUNSUPPORTED, "%s: padded per-(b, h) factors exceed 32-bit strides", fn);
    p.phq = phi_q;
    p.phk = phi_k;
    p.dphq = g->dphi_q;
    p.dphk = g->dphi_k;
    for (int i = 0; i < 3; ++i) {
      p.spq[i] = (int)sphi_q[i];
      p.spk[i] = (int)sphi_k[i];
      p.sdpq[i] = (int)g->sdphi_q[i];
      p.sdpk[i] = (int)g->sdphi_k[i];
    }
    RW = padded ? wl.R8 : R;
    if (padded && !f32) {
      // the factors go to [B][H][N][R8] copies with zero columns past R
      void* pq = (char*)g->work + wl.phq_off;
      void* pk = (char*)g->work + wl.phk_off;
      st = launch_attention_bwd_pad_factor(phi_q, esize(phi_dt), sphi_q, a->B, a->H, a->N, R, wl.R8, pq, stream);
      if (st == FB_OK)
        st = launch_attention_bwd_pad_factor(phi_k, esize(phi_dt), sphi_k, a->B, a->H, a->N, R, wl.R8, pk, stream);
      if (st != FB_OK) return st;
      p.phq = pq;
      p.phk = pk;
      const int sp[3] = {a->H * a->N * wl.R8, a->N * wl.R8, wl.R8};
      for (int i = 0; i < 3; ++i) p.spq[i] = p.spk[i] = sp[i];
      p.R = wl.R8;
    }
    // a gradient summed over batches or heads, and every factor gradient of a padded run,
    // goes to per-(b, h) partials first
    if (wl.pq_off != SIZE_MAX) {
      p.dphq = (float*)((char*)g->work + wl.pq_off);
      p.sdpq[0] = a->H * a->N * RW;
      p.sdpq[1] = a->N * RW;
      p.sdpq[2] = RW;
    }
    if (wl.pk_off != SIZE_MAX) {
      p.dphk = (float*)((char*)g->work + wl.pk_off);
      p.sdpk[0] = a->H * a->N * RW;
      p.sdpk[1] = a->N * RW;
      p.sdpk[2] = RW;
    }
    p.flags |= FLAG_PHQ_VEC | FLAG_PHK_VEC;
    RP = RW <= 16 ? 16 : RW <= 32 ? 32 : 64;
  }
  st = f32 ? launch_attention_bwd_delta_f32(a->o, a->so, g->dout, g->sdo, a->B, a->H, a->N, a->D, delta, stream)
          : launch_attention_bwd_delta(a->dt, a->o, a->so, g->dout, g->sdo, a->B, a->H, a->N, a->D, delta, stream);
  if (st != FB_OK) return st;
  const fb_dtype pdt = R > 0 ? phi_dt : a->dt;
  st = f32              ? launch_attention_bwd_f32(p, a->D, stream)
       : a->D == 16   ? launch_attention_bwd_d16(a->dt, pdt, RP, p, stream)
       : a->D == 32 ? launch_attention_bwd_d32(a->dt, pdt, RP, p, stream)
       : a->D == 64 ? launch_attention_bwd_d64(a->dt, pdt, RP, p, stream)
                    : launch_attention_bwd_d128(a->dt, pdt, RP, p, stream);
  if (st == FB_EUNSUPPORTED) set_error("%s: no kernel for this dtype / rank combination", fn);
  if (st != FB_OK) return st;
  if (R > 0 && wl.R8 > 0) {
    st = launch_attention_bwd_unpad(p.dphq, a->B, a->H, a->N, wl.R8, R, g->dphi_q, g->sdphi_q, stream);
    if (st == FB_OK) st = launch_attention_bwd_unpad(p.dphk, a->B, a->H, a->N, wl.R8, R, g->dphi_k, g->sdphi_k, stream);
    return st;
  }
  if (wl.pq_off != SIZE_MAX)
    st = launch_attention_bwd_reduce(p.dphq, a->B, a->H, a->N, R, g->dphi_q, g->sdphi_q, stream);
  if (st == FB_OK && wl.pk_off != SIZE_MAX)
    st = launch_attention_bwd_reduce(p.dphk, a->B, a->H, a->N, R, g->dphi_k, g->sdphi_k, stream);
  return st;
}
}  // namespace fb

extern "C" {

fb_status fb_attn_fwd_alibi(const fb_attn_args* a, const double* slopes_host, hipStream_t stream) {
  const char* fn = "fb_attn_fwd_alibi";
  fb_status st = check_common(a, fn);
  if (st != FB_OK) return st;
  if (a->dt != FB_BF16 && a->dt != FB_F16) FB_FAIL(FB_EUNSUPPORTED, "%s: q/k/v must be bf16 or f16", fn);
  if (a->H > kMaxJitHeads) FB_FAIL(FB_EUNSUPPORTED, "%s: at most %d heads", fn, kMaxJitHeads);
  if (a->N > 65536) FB_FAIL(FB_EUNSUPPORTED, "%s: N above 65536", fn);
  if ((int64_t)a->B * a->H * a->N == 0) return FB_OK;
  AttnParams p = base_params(a);
  for (int h = 0; h < a->H; ++h) {
    const double m = slopes_host ? slopes_host[h] : std::exp2(-8.0 * (h + 1) / a->H);
    if (!std::isfinite(m)) FB_FAIL(FB_EINVAL, "%s: non-finite slope", fn);
    // m = m_hi + m_lo, each rounded to nearest f16
    const _Float16 hi = (_Float16)m;
    const _Float16 lo = (_Float16)(m - (double)hi);
    p.alibi_m[h] = (uint32_t)__builtin_bit_cast(uint16_t, hi) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
  }
  p.R = 8;
  st = dispatch_attention(2, a->dt, FB_F16, a->D, 16, p, stream);
  if (st == FB_EUNSUPPORTED) set_error("%s: no kernel for this configuration", fn);
  return st;
}

fb_status fb_attn_fwd_sandwich(const fb_attn_args* a, int C, hipStream_t stream) {
  const char* fn = "fb_attn_fwd_sandwich";
  fb_status st = check_common(a, fn);
  if (st != FB_OK) return st;
  if (C < 2 || C % 2) FB_FAIL(FB_EINVAL, "%s: C must be even and >= 2", fn);
  if (a->dt != FB_BF16 && a->dt != FB_F16) FB_FAIL(FB_EUNSUPPORTED, "%s: q/k/v must be bf16 or f16", fn);
  if (a->D > 64) FB_FAIL(FB_EUNSUPPORTED, "%s: head dims up to 64", fn);
  if (C > 2 * kMaxSandwichPairs) FB_FAIL(FB_EUNSUPPORTED, "%s: C above %d", fn, 2 * kMaxSandwichPairs);
  if (a->N > 65536) FB_FAIL(FB_EUNSUPPORTED, "%s: N above 65536", fn);
  if ((int64_t)a->B * a->H * a->N == 0) return FB_OK;
  AttnParams p = base_params(a);
  const double two_pi = 6.283185307179586476925286766559;
  for (int f = 0; f < kMaxSandwichPairs; ++f) {
    if (f < C / 2) {
      // w_f = 10000^(-2(f+1)/C); nu_f = w_f / (2 pi) in revolutions, split so that an index
      // below 2^16 times either of the first two pieces is exact in fp32
      const double w = std::pow(10000.0, -2.0 * (f + 1) / C);
      double rest = w / two_pi;
      for (int i = 0; i < 2; ++i) {
        double piece = 0.0;
        if (rest != 0.0) {
          int e;
          std::frexp(rest, &e);
          const double q = std::ldexp(1.0, e - 8);    // 8 significant bits
          piece = std::nearbyint(rest / q) * q;
        }
        p.sw_nu[i][f] = (float)piece;
        rest -= piece;
      }
      p.sw_nu[2][f] = (float)rest;
      p.sw_rot[0][f] = std::cos(64.0 * w);
      p.sw_rot[1][f] = std::sin(64.0 * w);
    } else {
      p.sw_nu[0][f] = p.sw_nu[1][f] = p.sw_nu[2][f] = 0.f;
      p.sw_rot[0][f] = 1.0;
      p.sw_rot[1][f] = 0.0;
    }
  }
  p.sw_pairs = C / 2;
  p.R = C;
  const int RP = C <= 16 ? 16 : C <= 32 ? 32 : 64;   // a power-of-two number of 16-byte chunks per row
  st = dispatch_attention(4, a->dt, FB_F16, a->D, RP, p, stream);
  if (st == FB_EUNSUPPORTED) set_error("%s: no kernel for this configuration", fn);
  return st;
}

fb_status fb_attn_fwd_densebias(const fb_attn_args* a, const void* bias, fb_dtype bias_dt, const int64_t sbias[3],
                                hipStream_t stream) {
  const char* fn = "fb_attn_fwd_densebias";
  fb_status st = check_common(a, fn);
  if (st != FB_OK) return st;
  if (!known_dtype(bias_dt)) FB_FAIL(FB_EUNSUPPORTED, "%s: unknown bias dtype", fn);
  if (bias_dt != a->dt) FB_FAIL(FB_EUNSUPPORTED, "%s: bias dtype must equal the q/k/v dtype", fn);
  if ((int64_t)a->B * a->H * a->N == 0) return FB_OK;
  if (!bias || !sbias) FB_FAIL(FB_EINVAL, "%s: null bias or strides", fn);
  if (sbias[0] < 0 || sbias[1] < 0 || sbias[2] < 0) FB_FAIL(FB_EINVAL, "%s: negative bias stride", fn);
  if (a->N > 1 && sbias[2] < a->N) FB_FAIL(FB_EINVAL, "%s: bias row stride < N", fn);
  const int es = esize(bias_dt);
  if ((uintptr_t)bias % es) FB_FAIL(FB_EINVAL, "%s: misaligned bias", fn);
  if (!strides_fit32(sbias, a->N)) FB_FAIL(FB_EUNSUPPORTED, "%s: bias strides exceed 32 bits", fn);
  AttnParams p = base_params(a);
  p.bias = bias;
  for (int i = 0; i < 3; ++i) p.sb[i] = (int)sbias[i];
  if (aligned16(bias) && rows_aligned(sbias, es)) p.flags |= FLAG_BIAS_VEC;
  st = dispatch_attention(1, a->dt, bias_dt, a->D, 0, p, stream);
  if (st == FB_EUNSUPPORTED) set_error("%s: no kernel for this dtype combination", fn);
  return st;
}

}  // extern "C"
