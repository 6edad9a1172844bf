/*
 * disco_oracle.c — plain fp64 CPU oracle of the DISCO CSR contraction.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The HIP product path never calls it
 * and shares no code with it.
 *
 * What it computes (torch-harmonics "disco-kernel-dev" page, section
 * "Architecture snapshot": forward = CSR sparse contraction from the input grid
 * to the K-expanded (B,C,K,H,W) tensor; backward = the transpose contraction
 * back to the input grid; fused = contraction followed by the channel/basis
 * einsum).  The page gives the directions and the CSR layout but no formula;
 * the formula used is the plain one:
 *
 *   fwd:   out[p,k,ho,wo] = sum_{e in row(k,ho)} val_e * x[p, hi_e, (wi_e + s*wo) mod Wi]
 *   bwd:   gx = F^T gout, computed in the scatter form (each (e, wo) adds
 *          val_e * gout[p,k,ho,wo] to gx[p, hi_e, (wi_e + s*wo) mod Wi])
 *   fused: y[b,o,ho,wo] = sum_{c,k} W[o,c,k] * out[b,c,k,ho,wo]
 *
 * with s = Wi / Wo (the longitude subsampling factor) and p a flattened
 * (batch, channel) plane.  All inputs arrive as fp32 (bf16 data is widened to
 * fp32 exactly before the call) and are widened to double here; every sum is a
 * serial double accumulation in the order written.  With abs_mode = 1 every
 * operand is replaced by its absolute value, which yields the normaliser
 * sum |val * x| used to scale the parity error.
 *
 * fused_bwd: the gradients of <gy, y> for the fused convolution, the backward
 * the page pairs with its fused forward (same page, sections "Python dispatch
 * layer" and "Backward direction — gather vs scatter": the fused autograd
 * function runs the fused forward and the CSR transpose contraction backward;
 * section "Test coverage requirements": fused and unfused must agree in output
 * and gradient).  With the chain rule through y = einsum(W, F x):
 *
 *   g[b,c,k,ho,wo]  = sum_o W[o,c,k] * gy[b,o,ho,wo]
 *   gx[b,c]         = F^T g[b,c]                        (scatter form, as bwd)
 *   dW[o,c,k]       = sum_{b,ho,wo} gy[b,o,ho,wo] * out[b,c,k,ho,wo],  out = F x
 *
 * einsum: the fused convolution's second half alone, y[b,o,p] = sum_{c,k} W[o,c,k] * t[b,c,k,p]
 * for a contraction t given as input (p an output position).
 *
 * Parity status: fwd, bwd, fused, einsum and fused_bwd are each pinned by independent
 * checks in the CPU test suite (dense brute force, constant field,
 * equivariance, adjoint, FFT correlation, strided-subsample matmul, hand-worked
 * fixture; for fused_bwd: directional derivatives of the fused oracle and the
 * adjoint identities <gy, y> = <x, gx> = <W, dW>; for einsum: einsum of the forward oracle
 * reproduces the fused oracle bitwise, the hand-worked fixture, and K = 1 reduces to a numpy
 * matrix product).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline double opnd(double v, int abs_mode) { return abs_mode ? fabs(v) : v; }

/* Forward contraction over P planes.
 * x:   [P, Hi, Wi] fp32;  out: [P, K, Ho, Wo] double (overwritten). */
void oracle_fwd(int64_t P, int K, int Ho, int Wo, int Hi, int Wi,
                const int64_t *row_ptr, const int32_t *col_hi, const int32_t *col_wi,
                const float *val, const float *x, double *out, int abs_mode)
{
    const int s = Wi / Wo;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < P; ++p) {
        const float *xp = x + p * (int64_t)Hi * Wi;
        for (int k = 0; k < K; ++k) {
            for (int ho = 0; ho < Ho; ++ho) {
                const int64_t r = (int64_t)k * Ho + ho;
                double *o = out + ((p * K + k) * (int64_t)Ho + ho) * Wo;
                for (int wo = 0; wo < Wo; ++wo) o[wo] = 0.0;
                for (int64_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
                    const double v = opnd((double)val[e], abs_mode);
                    const float *xrow = xp + (int64_t)col_hi[e] * Wi;
                    for (int wo = 0; wo < Wo; ++wo) {
                        const int wi = (int)(((int64_t)col_wi[e] + (int64_t)s * wo) % Wi);
                        o[wo] += v * opnd((double)xrow[wi], abs_mode);
                    }
                }
            }
        }
    }
}

/* Transpose contraction (scatter form) over P planes.
 * gout: [P, K, Ho, Wo] fp32;  gx: [P, Hi, Wi] double (overwritten). */
void oracle_bwd(int64_t P, int K, int Ho, int Wo, int Hi, int Wi,
                const int64_t *row_ptr, const int32_t *col_hi, const int32_t *col_wi,
                const float *val, const float *gout, double *gx, int abs_mode)
{
    const int s = Wi / Wo;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < P; ++p) {
        double *g = gx + p * (int64_t)Hi * Wi;
        for (int64_t i = 0; i < (int64_t)Hi * Wi; ++i) g[i] = 0.0;
        for (int k = 0; k < K; ++k) {
            for (int ho = 0; ho < Ho; ++ho) {
                const int64_t r = (int64_t)k * Ho + ho;
                const float *go = gout + ((p * K + k) * (int64_t)Ho + ho) * Wo;
                for (int64_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
                    const double v = opnd((double)val[e], abs_mode);
                    double *grow = g + (int64_t)col_hi[e] * Wi;
                    for (int wo = 0; wo < Wo; ++wo) {
                        const int wi = (int)(((int64_t)col_wi[e] + (int64_t)s * wo) % Wi);
                        grow[wi] += v * opnd((double)go[wo], abs_mode);
                    }
                }
            }
        }
    }
}

/* Fused convolution for a list of output latitudes.
 * x: [B, C, Hi, Wi] fp32;  W: [Co, C, K] fp32;  ho_list: [nho];
 * y: [B, Co, nho, Wo] double (overwritten).
 * The contraction result for one (b, ho) is kept in double (no rounding)
 * before the einsum over (c, k). */
void oracle_fused(int B, int C, int Co, int K, int Ho, int Wo, int Hi, int Wi,
                  const int64_t *row_ptr, const int32_t *col_hi, const int32_t *col_wi,
                  const float *val, const float *x, const float *W,
                  int nho, const int32_t *ho_list, double *y, int abs_mode)
{
    const int s = Wi / Wo;
    double *t = (double *)malloc(sizeof(double) * (size_t)C * K * Wo);
    if (!t) abort();
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < nho; ++h) {
            const int ho = ho_list[h];
            /* t[c, k, wo] = contraction at (b, c, k, ho, wo) */
            #pragma omp parallel for schedule(dynamic, 1)
            for (int c = 0; c < C; ++c) {
                const float *xp = x + ((int64_t)b * C + c) * (int64_t)Hi * Wi;
                for (int k = 0; k < K; ++k) {
                    const int64_t r = (int64_t)k * Ho + ho;
                    double *o = t + ((int64_t)c * K + k) * Wo;
                    for (int wo = 0; wo < Wo; ++wo) o[wo] = 0.0;
                    for (int64_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
                        const double v = opnd((double)val[e], abs_mode);
                        const float *xrow = xp + (int64_t)col_hi[e] * Wi;
                        for (int wo = 0; wo < Wo; ++wo) {
                            const int wi = (int)(((int64_t)col_wi[e] + (int64_t)s * wo) % Wi);
                            o[wo] += v * opnd((double)xrow[wi], abs_mode);
                        }
                    }
                }
            }
            /* y[b, o, h, wo] = sum_{c,k} W[o,c,k] * t[c,k,wo] */
            #pragma omp parallel for schedule(dynamic, 1)
            for (int o = 0; o < Co; ++o) {
                double *yo = y + (((int64_t)b * Co + o) * nho + h) * Wo;
                for (int wo = 0; wo < Wo; ++wo) yo[wo] = 0.0;
                for (int c = 0; c < C; ++c) {
                    for (int k = 0; k < K; ++k) {
                        const double wv = opnd((double)W[((int64_t)o * C + c) * K + k], abs_mode);
                        const double *tk = t + ((int64_t)c * K + k) * Wo;
                        for (int wo = 0; wo < Wo; ++wo) yo[wo] += wv * tk[wo];
                    }
                }
            }
        }
    }
    free(t);
}

/* The einsum alone (the second half of the fused convolution, for a contraction given as input):
 * t: [B, C, K, P] double (P output positions), W: [Co, C, K] fp32 -> y: [B, Co, P] double.
 * Summed over c, then k, in the order oracle_fused uses, so that einsum(W, fwd(x)) reproduces
 * oracle_fused(x, W). */
void oracle_einsum(int B, int C, int Co, int K, int64_t P, const float *W, const double *t, double *y, int abs_mode)
{
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        for (int o = 0; o < Co; ++o) {
            double *yo = y + ((int64_t)b * Co + o) * P;
            for (int64_t p = 0; p < P; ++p) yo[p] = 0.0;
            for (int c = 0; c < C; ++c) {
                for (int k = 0; k < K; ++k) {
                    const double wv = opnd((double)W[((int64_t)o * C + c) * K + k], abs_mode);
                    const double *tk = t + (((int64_t)b * C + c) * K + k) * P;
                    for (int64_t p = 0; p < P; ++p) yo[p] += wv * opnd(tk[p], abs_mode);
                }
            }
        }
    }
}

/* Backward of the fused convolution over all output latitudes.
 * x: [B, C, Hi, Wi], W: [Co, C, K], gy: [B, Co, Ho, Wo] fp32;
 * gx: [B, C, Hi, Wi] and dW: [Co, C, K] double (overwritten).
 * abs_mode = 1 gives the normalisers (every operand by its absolute value). */
void oracle_fused_bwd(int B, int C, int Co, int K, int Ho, int Wo, int Hi, int Wi,
                      const int64_t *row_ptr, const int32_t *col_hi, const int32_t *col_wi,
                      const float *val, const float *x, const float *W, const float *gy,
                      double *gx, double *dW, int abs_mode)
{
    const int s = Wi / Wo;
    const int64_t HWo = (int64_t)Ho * Wo;
    double *g = (double *)malloc(sizeof(double) * (size_t)K * HWo);
    double *t = (double *)malloc(sizeof(double) * (size_t)K * HWo);
    if (!g || !t) abort();
    for (int64_t i = 0; i < (int64_t)Co * C * K; ++i) dW[i] = 0.0;
    for (int b = 0; b < B; ++b) {
        for (int c = 0; c < C; ++c) {
            /* g[k, ho, wo] = sum_o W[o,c,k] gy[b,o,ho,wo] */
            for (int64_t i = 0; i < (int64_t)K * HWo; ++i) g[i] = 0.0;
            for (int o = 0; o < Co; ++o) {
                const float *gyo = gy + ((int64_t)b * Co + o) * HWo;
                for (int k = 0; k < K; ++k) {
                    const double wv = opnd((double)W[((int64_t)o * C + c) * K + k], abs_mode);
                    double *gk = g + (int64_t)k * HWo;
                    for (int64_t i = 0; i < HWo; ++i) gk[i] += wv * opnd((double)gyo[i], abs_mode);
                }
            }
            /* gx[b, c] = F^T g (scatter) */
            double *gxp = gx + ((int64_t)b * C + c) * (int64_t)Hi * Wi;
            for (int64_t i = 0; i < (int64_t)Hi * Wi; ++i) gxp[i] = 0.0;
            for (int k = 0; k < K; ++k) {
                for (int ho = 0; ho < Ho; ++ho) {
                    const int64_t r = (int64_t)k * Ho + ho;
                    const double *gr = g + r * Wo;
                    for (int64_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
                        const double v = opnd((double)val[e], abs_mode);
                        double *grow = gxp + (int64_t)col_hi[e] * Wi;
                        for (int wo = 0; wo < Wo; ++wo) {
                            const int wi = (int)(((int64_t)col_wi[e] + (int64_t)s * wo) % Wi);
                            grow[wi] += v * gr[wo];
                        }
                    }
                }
            }
            /* t[k, ho, wo] = (F x)[b, c]; dW[o, c, k] += sum_{ho,wo} gy[b,o,ho,wo] t[k,ho,wo] */
            const float *xp = x + ((int64_t)b * C + c) * (int64_t)Hi * Wi;
            for (int k = 0; k < K; ++k) {
                for (int ho = 0; ho < Ho; ++ho) {
                    const int64_t r = (int64_t)k * Ho + ho;
                    double *tr = t + r * Wo;
                    for (int wo = 0; wo < Wo; ++wo) tr[wo] = 0.0;
                    for (int64_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
                        const double v = opnd((double)val[e], abs_mode);
                        const float *xrow = xp + (int64_t)col_hi[e] * Wi;
                        for (int wo = 0; wo < Wo; ++wo) {
                            const int wi = (int)(((int64_t)col_wi[e] + (int64_t)s * wo) % Wi);
                            tr[wo] += v * opnd((double)xrow[wi], abs_mode);
                        }
                    }
                }
            }
            #pragma omp parallel for schedule(dynamic, 1)
            for (int o = 0; o < Co; ++o) {
                const float *gyo = gy + ((int64_t)b * Co + o) * HWo;
                for (int k = 0; k < K; ++k) {
                    const double *tk = t + (int64_t)k * HWo;
                    double acc = 0.0;
                    for (int64_t i = 0; i < HWo; ++i) acc += opnd((double)gyo[i], abs_mode) * tk[i];
                    dW[((int64_t)o * C + c) * K + k] += acc;
                }
            }
        }
    }
    free(g);
    free(t);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
