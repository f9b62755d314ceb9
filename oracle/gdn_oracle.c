/*
 * gdn_oracle.c -- plain, slow fp64 CPU oracle of one Gated DeltaNet (GDN)
 * token-mixer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the HIP path is
 * checked against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load it.  It shares no code, header, table or helper with
 * the HIP library, and the product path never calls it.
 *
 * What it computes (sources):
 *   - The LinMorph project page ("Abstract", "Why learn the initialization?")
 *     replaces a video DiT's softmax attention with a Gated DeltaNet module
 *     whose parameter groups are update gates, decay terms, short
 *     convolutions and normalisation parameters.
 *   - The VMonarch page (section 2, "Efficient Attention Mechanisms", ref.
 *     [57] "Gated delta networks: Improving mamba2 with delta rule") places
 *     GDN among linear-attention mixers with a recurrent, expanded state and
 *     no KV cache.
 *   The pages print no equations, so this file takes the plainest reading of
 *   those parts, one function per part:
 *     1. short convolution: depthwise, causal, 4 taps, no bias, zero history,
 *        then SiLU, applied to q, k and v with separate weights;
 *     2. normalisation of q and k to unit L2 norm per token and head;
 *     3. the gated delta rule, token by token:
 *            S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *            o_t = S_t q_t,   S in R^{Dv x Dk};
 *     4. output normalisation: RMS over the Dv channels of o_t, times a
 *        per-channel weight, times SiLU(gate_t).
 *   Everything is fp64.  Inputs arrive as float32 arrays (every bf16 and
 *   fp32 input value is exactly representable there) and are widened once.
 *
 * Layouts (all row-major, contiguous):
 *   q, k [B,T,H,Dk]; v, gate [B,T,H,Dv]; log_a, beta [B,T,H];
 *   conv_q, conv_k [H*Dk,4]; conv_v [H*Dv,4]  (tap 3 multiplies x_t,
 *   tap j multiplies x_{t-3+j});  norm_w [H,Dv] or NULL (ones);
 *   S0, S_T [B,H,Dv,Dk];  y [B,T,H,Dv].
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Part 1: out[t][c] = SiLU( sum_{j=0..3} w[c][j] * x[t-3+j][c] ), x[<0] = 0. */
void oracle_short_conv_silu(long T, int D, const double *x, const double *w,
                            double *out)
{
    for (long t = 0; t < T; ++t) {
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int j = 0; j < 4; ++j) {
                long src = t - 3 + j;
                if (src >= 0)
                    acc += w[(long)c * 4 + j] * x[src * D + c];
            }
            out[t * D + c] = silu(acc);
        }
    }
}

/* Part 2: out[t] = x[t] / sqrt(|x[t]|^2 + eps). */
void oracle_l2_normalize(long T, int D, const double *x, double eps,
                         double *out)
{
    for (long t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int c = 0; c < D; ++c)
            ss += x[t * D + c] * x[t * D + c];
        double inv = 1.0 / sqrt(ss + eps);
        for (int c = 0; c < D; ++c)
            out[t * D + c] = x[t * D + c] * inv;
    }
}

/*
 * Part 3: the gated delta rule, one token at a time.
 *   S (Dv x Dk, row-major) holds S_0 on entry and S_T on return.
 *   For each t:  a = exp(log_a[t]),  b = beta[t],
 *       S <- a * S * (I - b k k^T) + b v k^T
 *   The product S (I - b k k^T) is expanded by distributivity into
 *   S - b (S k) k^T, which needs no Dk x Dk matrix; nothing else is
 *   rearranged.  Then o_t = S q_t.
 *   S_hist, when not NULL, receives the state after every token
 *   ([T][Dv][Dk]); it is meant for tiny T only.
 */
void oracle_delta_rule(long T, int Dk, int Dv, const double *q,
                       const double *k, const double *v, const double *log_a,
                       const double *beta, double *S, double *o,
                       double *S_hist)
{
    double *Sk = (double *)malloc(sizeof(double) * (size_t)Dv);
    for (long t = 0; t < T; ++t) {
        const double *kt = k + t * Dk, *qt = q + t * Dk, *vt = v + t * Dv;
        double a = exp(log_a[t]), b = beta[t];
        for (int i = 0; i < Dv; ++i) {
            double s = 0.0;
            for (int j = 0; j < Dk; ++j)
                s += S[(long)i * Dk + j] * kt[j];
            Sk[i] = s;
        }
        for (int i = 0; i < Dv; ++i)
            for (int j = 0; j < Dk; ++j) {
                double erased = S[(long)i * Dk + j] - b * Sk[i] * kt[j];
                S[(long)i * Dk + j] = a * erased + b * vt[i] * kt[j];
            }
        for (int i = 0; i < Dv; ++i) {
            double s = 0.0;
            for (int j = 0; j < Dk; ++j)
                s += S[(long)i * Dk + j] * qt[j];
            o[t * Dv + i] = s;
        }
        if (S_hist)
            memcpy(S_hist + t * (long)Dv * Dk, S,
                   sizeof(double) * (size_t)Dv * Dk);
    }
    free(Sk);
}

/* Part 4: y[t] = o[t] / sqrt(mean_c o[t][c]^2 + eps) * w * SiLU(gate[t]). */
void oracle_gated_rmsnorm(long T, int D, const double *o, const double *gate,
                          const double *w, double eps, double *y)
{
    for (long t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int c = 0; c < D; ++c)
            ss += o[t * D + c] * o[t * D + c];
        double inv = 1.0 / sqrt(ss / D + eps);
        for (int c = 0; c < D; ++c) {
            double wc = w ? w[c] : 1.0;
            y[t * D + c] = o[t * D + c] * inv * wc * silu(gate[t * D + c]);
        }
    }
}

/*
 * The whole layer for a set of (batch, head) pairs.  Each pair is an
 * independent task (the convolution is per channel, the recurrence and the
 * normalisation are per head), so tasks run on separate threads; inside a
 * task the steps run in the order above.
 *
 * reverse != 0 scans time backwards: token t of the scan is input token
 * T-1-t, and the scan's output for it is written back at T-1-t.
 * heads/n_heads select a subset of heads (NULL: all).  Output y entries of
 * unselected heads are left untouched.  n_threads <= 0 uses the OpenMP
 * default.  Returns the number of threads used, or -1 on allocation failure.
 */
int oracle_gdn_fwd(int B, long T, int H, int Dk, int Dv, const float *q,
                   const float *k, const float *v, const float *log_a,
                   const float *beta, const float *gate, const float *conv_q,
                   const float *conv_k, const float *conv_v,
                   const float *norm_w, double eps_l2, double eps_norm,
                   const float *S0, int reverse, double *y, double *S_T,
                   const int *heads, int n_heads, int n_threads)
{
    int nh = heads ? n_heads : H;
    long ntask = (long)B * nh;
    int used = 1;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long task = 0; task < ntask; ++task) {
#ifdef _OPENMP
        if (task == 0)
            used = omp_get_num_threads();
#endif
        int b = (int)(task / nh);
        int h = heads ? heads[task % nh] : (int)(task % nh);
        int D = Dk > Dv ? Dk : Dv;
        size_t n = (size_t)T * D;
        double *raw = (double *)malloc(sizeof(double) * n);
        double *tmp = (double *)malloc(sizeof(double) * n);
        double *qh = (double *)malloc(sizeof(double) * n);
        double *kh = (double *)malloc(sizeof(double) * n);
        double *vh = (double *)malloc(sizeof(double) * n);
        double *g = (double *)malloc(sizeof(double) * n);
        double *la = (double *)malloc(sizeof(double) * (size_t)T);
        double *be = (double *)malloc(sizeof(double) * (size_t)T);
        double *S = (double *)malloc(sizeof(double) * (size_t)Dv * Dk);
        double *w4 = (double *)malloc(sizeof(double) * (size_t)D * 4);
        double *nw = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (!raw || !tmp || !qh || !kh || !vh || !g || !la || !be || !S ||
            !w4 || !nw) {
            failed = 1;
        } else {
            /* the scan's token t is input token src(t) */
#define SRC(t) (reverse ? (T - 1 - (t)) : (t))
            /* q: gather, convolve + SiLU, normalise */
            for (long t = 0; t < T; ++t)
                for (int c = 0; c < Dk; ++c)
                    raw[t * Dk + c] =
                        q[(((long)b * T + SRC(t)) * H + h) * Dk + c];
            for (int c = 0; c < Dk; ++c)
                for (int j = 0; j < 4; ++j)
                    w4[c * 4 + j] = conv_q[((long)h * Dk + c) * 4 + j];
            oracle_short_conv_silu(T, Dk, raw, w4, tmp);
            oracle_l2_normalize(T, Dk, tmp, eps_l2, qh);
            /* k: the same with its own weights */
            for (long t = 0; t < T; ++t)
                for (int c = 0; c < Dk; ++c)
                    raw[t * Dk + c] =
                        k[(((long)b * T + SRC(t)) * H + h) * Dk + c];
            for (int c = 0; c < Dk; ++c)
                for (int j = 0; j < 4; ++j)
                    w4[c * 4 + j] = conv_k[((long)h * Dk + c) * 4 + j];
            oracle_short_conv_silu(T, Dk, raw, w4, tmp);
            oracle_l2_normalize(T, Dk, tmp, eps_l2, kh);
            /* v: convolution + SiLU only */
            for (long t = 0; t < T; ++t)
                for (int c = 0; c < Dv; ++c)
                    raw[t * Dv + c] =
                        v[(((long)b * T + SRC(t)) * H + h) * Dv + c];
            for (int c = 0; c < Dv; ++c)
                for (int j = 0; j < 4; ++j)
                    w4[c * 4 + j] = conv_v[((long)h * Dv + c) * 4 + j];
            oracle_short_conv_silu(T, Dv, raw, w4, vh);
            /* gates and initial state */
            for (long t = 0; t < T; ++t) {
                la[t] = log_a[((long)b * T + SRC(t)) * H + h];
                be[t] = beta[((long)b * T + SRC(t)) * H + h];
            }
            for (long i = 0; i < (long)Dv * Dk; ++i)
                S[i] = S0 ? S0[((long)b * H + h) * Dv * Dk + i] : 0.0;
            /* recurrence: o -> tmp */
            oracle_delta_rule(T, Dk, Dv, qh, kh, vh, la, be, S, tmp, NULL);
            /* output normalisation */
            for (long t = 0; t < T; ++t)
                for (int c = 0; c < Dv; ++c)
                    g[t * Dv + c] =
                        gate[(((long)b * T + SRC(t)) * H + h) * Dv + c];
            for (int c = 0; c < Dv; ++c)
                nw[c] = norm_w ? norm_w[(long)h * Dv + c] : 1.0;
            oracle_gated_rmsnorm(T, Dv, tmp, g, nw, eps_norm, raw);
            for (long t = 0; t < T; ++t)
                for (int c = 0; c < Dv; ++c)
                    y[(((long)b * T + SRC(t)) * H + h) * Dv + c] =
                        raw[t * Dv + c];
            if (S_T)
                memcpy(S_T + ((long)b * H + h) * Dv * Dk, S,
                       sizeof(double) * (size_t)Dv * Dk);
#undef SRC
        }
        free(raw); free(tmp); free(qh); free(kh); free(vh); free(g);
        free(la); free(be); free(S); free(w4); free(nw);
    }
    if (used > ntask)
        used = (int)ntask; /* threads beyond the task count stay idle */
    return failed ? -1 : used;
}
