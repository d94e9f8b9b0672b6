/*
 * fb.h -- C ABI of libflashbias: the forward pass of attention with an additive
 * bias on AMD Instinct MI355X (gfx950), with the bias given either as a
 * low-rank product b = phi_q phi_k^T (FlashBias) or as a dense N x N tensor.
 *
 * Source of the method: "FlashBias: Fast Computation of Attention with Bias"
 * (Wu et al.; abstract and the authors' OpenReview rebuttal).
 *
 *   O = softmax(s * Q K^T + b) V,  b[i,j] = sum_r phi_q[i,r] * phi_k[j,r]
 *
 * Attention with bias adds a bias matrix to the query-key scores (abstract).
 * When b has rank R, the factors are concatenated to the queries and keys,
 * Q' = [Q*s, phi_q], K' = [K, phi_k], and the attention runs on Q', K' with no
 * N x N bias read from HBM (rebuttal, answer to Reviewer UJUf, Q2: concatenate
 * the decomposed factor functions with queries and keys and run FlashAttention;
 * answer to Reviewer BRmd, Q3: factors of #heads x N x R instead of a
 * #heads x N x N bias).
 *
 * Conventions shared by every entry point
 *   - Every call returns fb_status; no C++ exception crosses the ABI.
 *   - Device pointers are caller-allocated (e.g. by PyTorch) and stay owned by
 *     the caller.  The library never allocates or frees device memory; its only
 *     device memory of its own is the fixed scratch array behind
 *     fb_attn_bwd_lowrank_noalloc.  Host buffers are read/written only during
 *     the call.
 *   - Argument validation is synchronous and happens before any launch; on a
 *     validation error nothing is launched and no output is touched.
 *   - Kernels are launched asynchronously on the caller's `stream`
 *     (NULL = the null stream); there is no implicit synchronisation.  A HIP
 *     launch error is reported as FB_EHIP.  Errors raised later by the kernel
 *     surface at the caller's next synchronisation.
 *   - Strides are in ELEMENTS.  For a tensor "[B][H][N][X] with strides
 *     s[3]", element (b,h,n,x) lives at base + b*s[0] + h*s[1] + n*s[2] + x: the
 *     last axis is contiguous.  A stride of 0 broadcasts along that axis.
 *   - NaN / Inf inputs are not checked; they propagate to the outputs.
 *   - fb_last_error() returns a short, thread-local description of the last
 *     non-FB_OK status raised in the calling thread.
 *   - The library is stateless and thread-safe.
 */
#ifndef FLASHBIAS_FB_H
#define FLASHBIAS_FB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

typedef enum {
  FB_OK = 0,
  FB_EINVAL = 1,        /* null pointer, bad size, misalignment, bad stride */
  FB_EUNSUPPORTED = 2,  /* valid request outside what the kernels implement */
  FB_EHIP = 3,          /* a HIP runtime call or launch failed */
  FB_ENOMEM = 4         /* host allocation failed (fb_svd_factors only) */
} fb_status;

typedef enum { FB_F32 = 0, FB_BF16 = 1, FB_F16 = 2 } fb_dtype;

typedef enum {
  FB_ALIBI = 0,     /* b[h,i,j] = m_h (j - i); rank 2 */
  FB_SANDWICH = 1   /* b[i,j] = sum_{k=1}^{C/2} cos((i-j) / 10000^(2k/C)); rank C */
} fb_bias_kind;

/* Human-readable name of a status code (static string). */
const char* fb_status_str(fb_status st);

/* Thread-local description of the last error raised in this thread ("" if none). */
const char* fb_last_error(void);

/*
 * fb_make_factors -- exact factors of a closed-form bias, generated on the GPU.
 *
 * ALiBi (rebuttal, answer to Reviewer BRmd, Q2: slopes of shape #heads; the
 * factor tiles are Block_q x 2 and Block_k x 2): phi_q(i) = [1, i],
 * phi_k(j) = [m_h * j, -m_h], so phi_q phi_k^T = m_h (j - i).
 * Sandwich (rebuttal, answer to Reviewer UJUf, Q1 (1)-(2)):
 * phi(i) = [cos(i w_1), sin(i w_1), ..., cos(i w_{C/2}), sin(i w_{C/2})],
 * w_k = 10000^(-2k/C), phi_q = phi_k = phi; phi phi^T is the Sandwich bias.
 *
 *   kind        FB_ALIBI or FB_SANDWICH
 *   H, N        heads and sequence length (>= 1)
 *   C           Sandwich channel count (even, >= 2); ignored for ALiBi
 *   slopes_host ALiBi: host array [H] of slopes, or NULL for m_h = 2^(-8(h+1)/H);
 *               ignored for Sandwich
 *   out_dt      element type of phi_q / phi_k
 *   split       1, 2 or 3: each factor value x is written as `split` pieces of
 *               out_dt, x ~ x_0 + x_1 + ..., x_0 = rn(x), x_1 = rn(x - x_0), ...
 *               Each natural column c becomes the columns of the piece pairs
 *               (a, b) with a + b < split (phi_q gets piece a, phi_k piece b),
 *               in the order (0,0), (0,1), (1,0), (0,2), (1,1), (2,0); so
 *               phi_q' phi_k'^T equals phi_q phi_k^T up to the dropped
 *               higher-order piece products.  split = 1 is plain rounding.
 *   phi_q,phi_k device, caller-allocated, [H][N][R_pad] of out_dt, contiguous
 *   R_pad       row length; must be >= R_used.  Columns R_used..R_pad-1 are
 *               written as zero.
 *   R_used      host out (may be NULL): natural rank x split(split+1)/2
 *               (ALiBi 2, Sandwich C, times 1, 3 or 6)
 * The values are computed in fp64 on the device and rounded to nearest even.
 * Errors: FB_EINVAL (null pointers, H or N < 1, odd or < 2 C for Sandwich,
 * split outside 1..3, R_pad < R_used, 16-byte-misaligned phi pointers);
 * FB_EUNSUPPORTED (H * N * R_pad of 2^31 or more; more than 256 explicit slopes);
 * FB_EHIP.
 */
fb_status fb_make_factors(fb_bias_kind kind, int H, int N, int C, const double* slopes_host,
                          fb_dtype out_dt, int split, void* phi_q, void* phi_k, int R_pad,
                          int* R_used, hipStream_t stream);

/*
 * fb_make_factors_log2 -- as fb_make_factors, with phi_q in exp2 units: every
 * phi_q value is multiplied by log2(e) in fp64 before it is split and rounded,
 * so phi_q phi_k^T = b log2(e) (split pieces stay exact products).  These are the
 * factors fb_attn_fwd_lowrank_log2 takes.  Arguments and errors as
 * fb_make_factors.
 */
fb_status fb_make_factors_log2(fb_bias_kind kind, int H, int N, int C, const double* slopes_host,
                               fb_dtype out_dt, int split, void* phi_q, void* phi_k, int R_pad,
                               int* R_used, hipStream_t stream);

/*
 * fb_make_dense_bias -- the same closed-form biases, materialised as a dense
 * [H][N][N] tensor (the input of the dense-bias baseline, fb_attn_fwd_densebias).
 * Computed in fp64 from the defining formula (ALiBi m_h (j - i); Sandwich the
 * sum of C/2 cosines), rounded to nearest even into out_dt.
 *   bias        device, [H][N][N] with element strides head_stride, row_stride
 *               (last axis contiguous)
 * Errors: FB_EINVAL (null bias, H or N < 1, C odd or < 2 for Sandwich,
 * row_stride < N, head_stride < N*row_stride when H > 1); FB_EHIP.
 */
fb_status fb_make_dense_bias(fb_bias_kind kind, int H, int N, int C, const double* slopes_host,
                             fb_dtype out_dt, void* bias, int64_t head_stride, int64_t row_stride,
                             hipStream_t stream);

/*
 * fb_svd_factors -- truncated SVD factors of one general (e.g. learned) bias,
 * computed on the host; the pages do this offline, once per layer and head
 * (rebuttal, answer to Reviewer xU4x, Q6; abstract: fast-accurate
 * approximation for general biases).
 *
 *   bias        host, [N][N] fp64, row-major (read only)
 *   N, R        1 <= R <= N
 *   seed        seed of the randomized range finder (results are deterministic
 *               for a given seed)
 *   phi_q,phi_k host out, [N][R] fp64: U_R sqrt(S_R) and V_R sqrt(S_R), so that
 *               phi_q phi_k^T is the best rank-R approximation of bias
 *   sigma       host out [R] or NULL: the R largest singular values, descending
 *   energy      host out or NULL: sum_{r<R} sigma_r^2 / ||bias||_F^2, the
 *               retained energy (rebuttal, answer to Reviewer Bp2x, Q2: heads
 *               are chosen to keep 95% energy)
 * Method: randomized subspace iteration (Halko, Martinsson, Tropp 2011) with
 * Householder QR re-orthonormalisation, iterated until the top-R singular
 * values settle, followed by a one-sided Jacobi SVD of the small projected
 * matrix.  Temporary host memory is freed before return.
 * Errors: FB_EINVAL (null pointers, N < 1, R < 1 or R > N); FB_ENOMEM.
 */
fb_status fb_svd_factors(const double* bias, int N, int R, uint64_t seed, double* phi_q,
                         double* phi_k, double* sigma, double* energy);

/*
 * fb_svd_factors_log2 -- as fb_svd_factors, with phi_q in exp2 units: every phi_q value is
 * multiplied by log2(e) in fp64 before it is returned, so phi_q phi_k^T = log2(e) times the
 * rank-R approximation.  These are the factors fb_attn_fwd_lowrank_log2 takes (after the
 * caller rounds them to the factor dtype).  sigma and energy are those of fb_svd_factors.
 * Arguments and errors as fb_svd_factors.
 */
fb_status fb_svd_factors_log2(const double* bias, int N, int R, uint64_t seed, double* phi_q,
                              double* phi_k, double* sigma, double* energy);

/*
 * fb_svd_rank_for_energy -- the smallest rank whose truncated SVD keeps a target share
 * of a bias's energy.  The pages apply the low-rank path only where a rank-R factorisation
 * keeps 95% of a head's bias energy (rebuttal, answer to Reviewer Bp2x, Q2, with the
 * SwinV2 study of different R); this is that test for one head.
 *
 *   bias        host, [N][N] fp64, row-major (read only)
 *   N, R_max    1 <= R_max <= N: the largest rank considered
 *   target      0 < target <= 1, e.g. 0.95
 *   seed        seed of the randomized range finder (as fb_svd_factors)
 *   R_out       host out: the smallest R <= R_max with
 *               sum_{r<R} sigma_r^2 >= target * ||bias||_F^2, or R_max when no R
 *               reaches the target (the caller then keeps the dense bias for the head)
 *   energy_out  host out or NULL: the energy kept by R_out
 *   reached     host out or NULL: 1 if R_out reaches the target, else 0
 * An all-zero bias needs rank 1 (energy 1).  The singular values come from the same
 * randomized subspace iteration as fb_svd_factors run at rank R_max; call fb_svd_factors
 * with R_out for the factors.
 * Errors: FB_EINVAL (null pointers, N < 1, R_max out of range, target out of range);
 * FB_ENOMEM.
 */
fb_status fb_svd_rank_for_energy(const double* bias, int N, int R_max, double target, uint64_t seed,
                                 int* R_out, double* energy_out, int* reached);

/* Arguments shared by both attention entry points. */
typedef struct {
  int B, H, N, D;      /* batch, heads, sequence length (queries = keys), head dim */
  fb_dtype dt;         /* element type of Q, K, V and O: FB_F32, FB_BF16 or FB_F16 */
  int causal;          /* nonzero: query i attends to keys j <= i */
  float scale;         /* s, the score scale (callers usually pass 1/sqrt(D)) */
  const void* q;       /* device [B][H][N][D], strides sq */
  const void* k;       /* device [B][H][N][D], strides sk */
  const void* v;       /* device [B][H][N][D], strides sv */
  void* o;             /* device [B][H][N][D], strides so (output) */
  int64_t sq[3], sk[3], sv[3], so[3];
  float* lse;          /* device [B][H][N] contiguous fp32, or NULL: m + ln(l), the
                          natural log-sum-exp of each row's biased scores */
} fb_attn_args;

/*
 * fb_attn_fwd_lowrank -- O = softmax(s Q K^T + phi_q phi_k^T) V in one fused
 * kernel: the augmented contraction [Q*s, phi_q] [K, phi_k]^T feeds an online
 * softmax and the P V product, tile by tile; the N x N bias is never formed.
 *
 *   a            shared arguments (see fb_attn_args)
 *   phi_q, phi_k device [B][H][N][R] (strides sphi_q / sphi_k; 0 broadcasts a
 *                factor over batch and/or heads).  May be NULL when R == 0.
 *   phi_dt       FB_F32 when a->dt is FB_F32; FB_BF16 or FB_F16 when a->dt is
 *                FB_BF16 or FB_F16 (the factor columns then run through their own
 *                matrix-core chain in phi_dt, accumulating into the same fp32 scores)
 *   R            number of factor columns, 0 <= R <= 128 (16-bit) or <= 32 (fp32);
 *                R == 0 is plain attention.  Columns are zero-padded internally to
 *                the matrix-core step (16 for 16-bit types, 8 for fp32).
 * Numerics: fp32 accumulation; Q*s is rounded once to dt; the probabilities P
 * are rounded to dt (RNE) before the P V product and their row sum is taken
 * from the same rounded values (fp32 accumulation; fp32 Q/K/V: unrounded);
 * O is written in dt.
 * Alignment: q, k, v, o 16-byte aligned and their strides multiples of
 * 16 bytes / element size.  phi rows may be unaligned; phi_k is fastest with
 * 16-byte aligned rows and R a multiple of 16 bytes / element size (it is then
 * copied straight into on-chip memory, otherwise staged through registers).
 * Errors: FB_EINVAL (null pointers, negative sizes, misalignment, row strides
 * too small); FB_EUNSUPPORTED (D not in {16,32,64,128}, or D = 128 with fp32
 * Q/K/V; R above the limit; a dtype pair not listed above; element strides or
 * N * row stride of any operand above 2^31 - 1; a k, v or phi_k row stride
 * whose 64 rows span 2^31 bytes or more); FB_EHIP.  B*H*N == 0 is a no-op
 * returning FB_OK.
 */
fb_status fb_attn_fwd_lowrank(const fb_attn_args* a, const void* phi_q, const void* phi_k,
                              fb_dtype phi_dt, int R, const int64_t sphi_q[3],
                              const int64_t sphi_k[3], hipStream_t stream);

/*
 * fb_attn_fwd_lowrank_log2 -- the same attention with phi_q given in exp2 units:
 *   O = softmax(s Q K^T + ln(2) phi_q phi_k^T) V,
 * i.e. phi_q = log2(e) phi_q' for the factors phi_q' of fb_attn_fwd_lowrank
 * (fb_make_factors_log2 writes them).  The kernel then works in exp2 units
 * throughout (Q s is rounded as Q s log2(e); every score chain starts from the
 * running max), which saves one vector operation per score in the softmax.
 * The pages' formulation is unchanged (FlashBias rebuttal, answer to Reviewer UJUf,
 * Q2: the factor columns are concatenated with queries and keys); only the unit of
 * phi_q differs.
 * Arguments, alignment and errors as fb_attn_fwd_lowrank, for bf16 / f16 Q/K/V
 * only (FB_EUNSUPPORTED for fp32).  Numerics differ in one rounding: Q s log2(e) is
 * rounded to dt (the row sum of P is taken from the rounded P, as in
 * fb_attn_fwd_lowrank).
 * R == 0 is plain attention in the same exp2 form.  LSE (when requested) is the
 * natural-log value as for fb_attn_fwd_lowrank; fb_attn_bwd_lowrank takes natural-unit
 * factors (phi_q ln(2) for the factors given here).
 * Kernel choice (results to the same bars either way): a non-causal launch with
 * D = 16 and R <= 32, or D = 32 and R <= 16, and N at most the keys whose K' and V
 * tiles fit in 80 KB of LDS (D = 32: 512 keys with R <= 16, 640 with R = 0; D = 16:
 * 512, 640 and 832 keys with R <= 32, R <= 16 and R = 0) runs one workgroup per
 * (b, h) with all its tiles resident in LDS; every other launch streams the tiles.  The environment
 * variable FB_ATTN_STREAMING=1 (read at each call) selects the streaming kernel
 * for every launch.
 */
fb_status fb_attn_fwd_lowrank_log2(const fb_attn_args* a, const void* phi_q, const void* phi_k,
                                   fb_dtype phi_dt, int R, const int64_t sphi_q[3],
                                   const int64_t sphi_k[3], hipStream_t stream);

/*
 * fb_attn_fwd_densebias -- O = softmax(s Q K^T + b) V with b read as a dense
 * tensor: each (query-tile, key-tile) pair streams its bias tile from HBM, the
 * quadratic IO of attention with bias (abstract; rebuttal, answer to Reviewer
 * BRmd, Q3).  The in-house baseline the low-rank kernel is measured against.
 *
 *   bias     device [B][H][N][N] with strides sbias (b, h, i); the last axis (j)
 *            contiguous; sbias[0] and/or sbias[1] may be 0 (shared bias)
 *   bias_dt  FB_F32 when a->dt is FB_F32; FB_BF16 or FB_F16 otherwise
 * Numerics and alignment as fb_attn_fwd_lowrank, except that the row sum of P
 * is taken in fp32 before P is rounded to dt; the bias is added in fp32.
 * Errors: as fb_attn_fwd_lowrank; FB_EINVAL for a null bias or sbias[2] < N.
 */
fb_status fb_attn_fwd_densebias(const fb_attn_args* a, const void* bias, fb_dtype bias_dt,
                                const int64_t sbias[3], hipStream_t stream);

/*
 * fb_attn_fwd_mulbias -- attention with a multiplicative low-rank bias,
 *   O = softmax((s Q K^T) .* (phi_q phi_k^T)) V
 * (FlashBias rebuttal, answer to Reviewer BRmd, Q1 (2): Eq. (1) defines the
 * multiplicative bias, Eq. (3) rewrites it as plain attention over the expanded
 * operands q' = [q phi_q,1, ..., q phi_q,R], k' = [k phi_k,1, ..., k phi_k,R] of
 * width D R).  One expansion kernel writes q' (scaled by s) and k' into the
 * caller's workspace, then the low-rank kernel runs with their first D columns as
 * Q / K and the remaining (R - 1) D as factor columns; the N x N bias is never formed.
 *
 *   a            shared arguments; a->dt must be FB_BF16 or FB_F16
 *   phi_q, phi_k device [B][H][N][R] in phi_dt (FB_F32, FB_BF16 or FB_F16), strides
 *                sphi_q / sphi_k (0 broadcasts over batch and/or heads)
 *   R            1 <= R and (R - 1) * D <= 128
 *   workspace    device, at least fb_mulbias_workspace_bytes(a, R) bytes, 256-byte
 *                aligned; owned by the caller and only used on `stream` during the
 *                call's work (it may be reused once that work has finished)
 * Numerics: every element of q' and k' is formed in fp32 and rounded once to dt;
 * then as fb_attn_fwd_lowrank (the scale is folded into q').
 * Errors: as fb_attn_fwd_lowrank; FB_EUNSUPPORTED for fp32 or (R - 1) D > 128;
 * FB_EINVAL for R < 1, null factors or workspace, a workspace that is too small
 * or misaligned.
 */
fb_status fb_attn_fwd_mulbias(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt, int R,
                              const int64_t sphi_q[3], const int64_t sphi_k[3], void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace fb_attn_fwd_mulbias needs for these arguments and rank:
 * q' and k' in a->dt, B H N D R elements each, plus alignment.  0 for empty inputs. */
size_t fb_mulbias_workspace_bytes(const fb_attn_args* a, int R);

/*
 * fb_mulbias_expand -- the first stage of fb_attn_fwd_mulbias alone: writes the
 * expanded operands into the workspace and returns; fb_attn_fwd_mulbias is this
 * followed by fb_attn_fwd_lowrank on them.  Arguments and errors as
 * fb_attn_fwd_mulbias (v and o are not touched).  Workspace layout, every part
 * contiguous row-major in a->dt and starting on a 256-byte boundary, with
 * E = B H N and up(x) = x rounded up to a multiple of 256:
 *   offset 0                       q1 = s q phi_q,1              [B][H][N][D]
 *   offset A = up(E D es)          k1 = k phi_k,1                [B][H][N][D]
 *   offset 2A                      s [q phi_q,2 .. q phi_q,R]    [B][H][N][(R-1) D]
 *   offset 2A + up(E (R-1) D es)   [k phi_k,2 .. k phi_k,R]      [B][H][N][(R-1) D]
 * (es = element size of a->dt); run fb_attn_fwd_lowrank with q1, k1, scale 1 and the
 * last two parts as phi_q / phi_k (R - 1) D columns wide.
 */
fb_status fb_mulbias_expand(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt, int R,
                            const int64_t sphi_q[3], const int64_t sphi_k[3], void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * fb_attn_fwd_alibi -- O = softmax(s Q K^T + b) V for the ALiBi bias
 * b[h,i,j] = m_h (j - i) with its rank-2 factors formed inside the kernel from the
 * slopes and the query / key indices, as the pages deploy ALiBi (FlashBias rebuttal,
 * answer to Reviewer BRmd, Q2: only the #heads slopes are loaded, the Block_q x 2 and
 * Block_k x 2 factor tiles are generated in the kernel).  No factor tensor exists: per
 * tile the kernel builds f16 factor columns whose products sum exactly (in fp32) to
 * m_h (j - i), with m_h held as two f16 values (22 bits) and i, j split at 2048.
 *
 *   a            shared arguments; a->dt FB_BF16 or FB_F16
 *   slopes_host  host [H] fp64 slopes, or NULL for m_h = 2^(-8(h+1)/H)
 * Limits: H <= 128 (the slopes travel in the kernel arguments), N <= 65536.
 * Numerics: as fb_attn_fwd_lowrank with an f16 factor chain.
 * Errors: as fb_attn_fwd_lowrank; FB_EUNSUPPORTED for fp32, H > 128 or N > 65536;
 * FB_EINVAL for a non-finite slope.
 */
fb_status fb_attn_fwd_alibi(const fb_attn_args* a, const double* slopes_host, hipStream_t stream);

/*
 * fb_attn_fwd_sandwich -- O = softmax(s Q K^T + b) V for the Sandwich bias
 * b[i,j] = sum_{k=1}^{C/2} cos((i - j) w_k), w_k = 10000^(-2k/C), with its cos / sin factor
 * columns formed inside the kernel (FlashBias rebuttal, answer to Reviewer UJUf, Q1 (1)-(2):
 * the factor functions phi(i) = [cos(i w_1), sin(i w_1), ...] with b = phi phi^T; answer to
 * Reviewer BRmd, Q2: the factor tiles are generated in the kernel instead of being loaded).
 * No factor tensor exists: phi_q of each query (in exp2 units, times log2(e)) is formed once
 * per query row and rounded to f16; each key tile's phi_k (f16) is written into on-chip memory
 * by the kernel, rotating exact per-offset values by the tile's first key in fp64.
 *
 *   a   shared arguments; a->dt FB_BF16 or FB_F16, a->D <= 64
 *   C   even, 2 <= C <= 64 (the Sandwich channel count; C/2 frequencies)
 * Limits: N <= 65536.
 * Numerics: as fb_attn_fwd_lowrank_log2 with f16 factor columns (C of them, zero-padded to
 * 16, 32 or 64, which sets R for the row-sum rule there); the factor values are within about 1e-6 of the exact cos / sin before
 * their f16 rounding.
 * Errors: as fb_attn_fwd_lowrank; FB_EINVAL for an odd C or C < 2; FB_EUNSUPPORTED for
 * fp32, D > 64, C > 64 or N > 65536.
 */
fb_status fb_attn_fwd_sandwich(const fb_attn_args* a, int C, hipStream_t stream);

/* Outputs and workspace of the attention backward. */
typedef struct {
  const void* dout;    /* device [B][H][N][D], strides sdo: the upstream gradient dO (a->dt) */
  int64_t sdo[3];
  void* dq;            /* device outputs [B][H][N][D] in a->dt, strides sdq / sdk / sdv */
  void* dk;
  void* dv;
  int64_t sdq[3], sdk[3], sdv[3];
  float* dphi_q;       /* device fp32 outputs [.][.][N][R] with strides sdphi_q / sdphi_k;
                          a 0 stride sums the gradient over that axis (a factor shared by
                          all batches or heads); NULL when R == 0 */
  float* dphi_k;
  int64_t sdphi_q[3], sdphi_k[3];
  void* work;          /* device workspace, 256-byte aligned, at least
                          fb_attn_bwd_workspace_bytes(...) bytes; caller-owned, contents
                          undefined on return */
  size_t work_bytes;
} fb_attn_bwd_args;

/*
 * fb_attn_bwd_workspace_bytes -- size of the workspace fb_attn_bwd_lowrank needs: the
 * fp32 row sums Delta = rowsum(dO * O) ([B][H][N]) and, for each factor gradient that is
 * summed over batches or heads (a 0 stride on an axis of size > 1), one fp32 partial
 * gradient per (b, h) ([B][H][N][R]), which a final pass adds up in a fixed order (no
 * atomics: the sums are deterministic).  When R is not a multiple of 8 it holds instead
 * zero-padded copies of both factors ([B][H][N][R8], R8 = R rounded up to 8, in the factor
 * dtype) and both factor gradients per (b, h) ([B][H][N][R8] fp32).  Each part starts on a
 * 256-byte boundary.
 * Returns 0 for negative sizes.
 */
size_t fb_attn_bwd_workspace_bytes(int B, int H, int N, int R, const int64_t sdphi_q[3], const int64_t sdphi_k[3]);

/*
 * fb_attn_bwd_lowrank -- gradients of O = softmax(s Q K^T + phi_q phi_k^T) V with
 * respect to Q, K, V and both factors, for an upstream gradient dO, without any N x N
 * tensor: the factor gradients are the last R columns of the gradients of the
 * augmented operands Q' = [Q*s, phi_q], K' = [K, phi_k] (the pages train with these
 * biases: FlashBias rebuttal, answer to Reviewer UJUf, Q1, GPT-2 with Sandwich bias):
 *   dV = P^T dO, dS = P .* (dO V^T - rowsum(dO .* O)), dQ = s dS K, dK = s dS^T Q,
 *   dphi_q = dS phi_k, dphi_k = dS^T phi_q,    P = exp(s Q K^T + phi_q phi_k^T - LSE).
 *
 *   a            the forward's arguments: q, k, v, o (the forward output) and lse (the
 *                forward's LSE output, required)
 *   phi_*, R ... the forward's factors (R == 0: plain attention)
 *   g            dO, the outputs and the workspace (see fb_attn_bwd_args)
 * Supported: a->dt FB_BF16 or FB_F16, D in {16, 32, 64, 128}, R <= 64; or a->dt FB_F32 with
 * FB_F32 factors, D in {16, 32, 64}, R <= 64 (fp32 matrix-core kernels that read the factors
 * in place with their strides, element-aligned; fp32 throughout).  16-bit, R % 8 == 0: the
 * factor rows and the factor-gradient rows must be 16-byte aligned (FB_EUNSUPPORTED /
 * FB_EINVAL); otherwise the library first copies the factors into zero-padded [B][H][N][R8]
 * buffers in the workspace, runs the kernels at width R8 and writes the first R columns of
 * the gradients (summed where a stride is 0) into dphi_*, which then need only 4-byte
 * alignment (the factors: element alignment).  The fused kernels recompute the
 * scores tile by tile; Q*s is rounded to dt as in the forward (for the key-major kernel
 * the scale is applied to K, identical when s is a power of two); P and dS are rounded to
 * dt for their MFMA products; accumulation is fp32.  dphi_* of one (b, h) are written by
 * the kernels; a factor shared over batches or heads gets the sum of the per-(b, h)
 * gradients, added in (b, h) order from the workspace (deterministic).
 * Errors: as the forward; FB_EINVAL for null outputs / lse, a null, misaligned or too
 * small workspace, negative or misaligned strides; FB_EUNSUPPORTED outside the
 * supported set.
 */
fb_status fb_attn_bwd_lowrank(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt, int R,
                              const int64_t sphi_q[3], const int64_t sphi_k[3], const fb_attn_bwd_args* g,
                              hipStream_t stream);

/*
 * fb_attn_bwd_lowrank_log2 -- the gradients of fb_attn_fwd_lowrank_log2's output:
 *   O = softmax(s Q K^T + ln(2) phi_q phi_k^T) V,   phi_q in exp2 units,
 * with respect to Q, K, V and the factors as given (dphi_q is the gradient with respect to
 * the exp2-unit phi_q: ln(2) dS phi_k; dphi_k = ln(2) dS^T phi_q).  The fused kernels form the
 * scores in exp2 units, as the forward does (K s log2(e) in the key-major kernel, Q s log2(e)
 * in the query-major one, L log2(e)); dS = P (dP - Delta) is in natural units.  a->lse is the
 * forward's natural-log LSE.  Arguments, workspace (fb_attn_bwd_workspace_bytes), support and
 * errors as fb_attn_bwd_lowrank; R == 0 is identical to fb_attn_bwd_lowrank.
 */
fb_status fb_attn_bwd_lowrank_log2(const fb_attn_args* a, const void* phi_q, const void* phi_k, fb_dtype phi_dt,
                                   int R, const int64_t sphi_q[3], const int64_t sphi_k[3],
                                   const fb_attn_bwd_args* g, hipStream_t stream);

/* Size of the device scratch array behind fb_attn_bwd_lowrank_noalloc (64 MiB per GPU). */
#define FB_BWD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * fb_attn_bwd_lowrank_noalloc -- fb_attn_bwd_lowrank for callers that cannot allocate
 * device memory: code under HIP graph capture, tight training loops, harnesses that forbid
 * hipMalloc.  It neither allocates nor frees anything; its workspace is a file-scope
 * device array of FB_BWD_NOALLOC_SCRATCH_BYTES bytes in the library, one copy per GPU,
 * which each GPU the library runs this on holds until the process ends.
 *
 *   Arguments as fb_attn_bwd_lowrank, except that g->work must be NULL and g->work_bytes 0.
 *   The stream (NULL = the null stream) must belong to the calling thread's current device.
 *   Results are those of fb_attn_bwd_lowrank on the same inputs (the same kernels).
 * Every call on one GPU shares that GPU's array and leaves the last call's contents in it
 * (nothing in it needs to start at zero: every byte the kernels read is written earlier in
 * the same call); calls that overlap on one GPU (other streams, other threads) race.
 * Errors: as fb_attn_bwd_lowrank; FB_EINVAL for a non-NULL g->work or nonzero
 * g->work_bytes, or a stream of another device; FB_EUNSUPPORTED when the sizes need more
 * workspace than the scratch holds (fb_attn_bwd_workspace_bytes above
 * FB_BWD_NOALLOC_SCRATCH_BYTES), checked before any HIP call; FB_EHIP when the scratch
 * address cannot be looked up.
 */
fb_status fb_attn_bwd_lowrank_noalloc(const fb_attn_args* a, const void* phi_q, const void* phi_k,
                                      fb_dtype phi_dt, int R, const int64_t sphi_q[3],
                                      const int64_t sphi_k[3], const fb_attn_bwd_args* g,
                                      hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FLASHBIAS_FB_H */
