/*
 * lla_oracle.c -- plain fp64 CPU oracle for the Looped Latent Attention (LLA) decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load this file;
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark use it.  It shares
 * no code, header, constant or helper with the HIP library.
 *
 * What it follows (all citations are to the pages on "Looped Latent Attention: Cross-Loop KV
 * Compression for Looped Transformers", O'Neill & Reid, arXiv 2607.15456):
 *   - the codec, pith.science paper page, section "What carries the argument": per layer, head
 *     and axis (K or V) a token's T loop-step vectors form one vector x of length T d; removing
 *     the mean mu and multiplying by W_down gives the rank-r latent c = (x - mu) W_down, and
 *     loop t reads back x_hat_t = c W_up,t + mu_t;
 *     attention itself is left unchanged; compression is rho = 2 T d_head / (r_k + r_v)
 *     (the referee report on the same page calls this Eq. 4 and says it is exact);
 *   - the read path, arXiv abstract: loop-specific K/V vectors are reconstructed only when
 *     attention reads them; the default codec is per head, LLA-2D folds all heads into one
 *     latent per layer and axis;
 *   - the loop-indexed baseline cache, Figure 1 caption: each recurrent step t contributes its
 *     own (K_t, V_t), so loop t's attention reads the loop-t keys and values.
 *
 * Readings where the pages are silent (each is listed in the design doc):
 *   - the current token attends to its own loop-t key/value (the optional "self" term);
 *   - LLA-2D stacks the vector in (t, h, i) order: index (t*H + h)*d + i;
 *   - mu has length X = T*D_g per (layer, group, axis) and mu_t is its block t;
 *   - softmax is the usual max-subtracted one, computed here in two passes;
 *   - an empty context with no self term yields a zero output.
 *
 * Every array is a dense row-major fp64 copy of exactly the values the device receives.
 *   G  = H (per-head, mode 0) or 1 (LLA-2D, mode 1);  D_g = d (mode 0) or H*d (mode 1);
 *   X  = T * D_g.
 *   W_down [G][X][r]        W_up [T][G][r][D_g]        mu [G][X]
 *   latent pools [n_pages][G][P][r]   block_table [B][max_pages]   seq_lens [B]
 *   q, out [B][H][d];  self k/v rows at k_self[b*self_stride + h*d + i]
 *   flat (uncompressed, loop-t) pools [n_pages][H][P][d]
 *   staging trajectories x [B][T][H][d]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Eq. 4 (pith.science paper page, "What carries the argument"): rho = 2 T d_head / (r_k + r_v)
 * per head and layer.  For LLA-2D the stored latent covers all H heads, so the uncompressed
 * side is 2 T H d_head per layer (abstract: LLA-2D folds heads into one latent). */
double oracle_compression_ratio(int mode, int T, int H, int d, int r_k, int r_v) {
    double flat = 2.0 * (double)T * (double)d * (mode == 1 ? (double)H : 1.0);
    return flat / (double)(r_k + r_v);
}

/* Page resolve: logical token j of sequence b lives in page block_table[b][j / P] at slot
 * j % P.  Returns a pointer to that token's latent for group g. */
static const double *latent_at(const double *pool, const int32_t *block_table, int max_pages,
                               int G, int P, int r, int b, int j, int g) {
    int page = block_table[(size_t)b * max_pages + j / P];
    int slot = j % P;
    return pool + (((size_t)page * G + g) * P + slot) * r;
}

/* x_hat_t = c W_up,t + mu_t  (pith.science paper page, "What carries the argument").
 * out has D_g entries. */
static void reconstruct(const double *c, int r, const double *W_up_tg, const double *mu_t,
                        int Dg, double *out) {
    /* out[i] = mu_t[i] + c[0] W[0][i] + c[1] W[1][i] + ... (summed in that order for every i) */
    for (int i = 0; i < Dg; ++i) out[i] = mu_t[i];
    for (int k = 0; k < r; ++k) {
        const double *row = W_up_tg + (size_t)k * Dg;
        for (int i = 0; i < Dg; ++i) out[i] += c[k] * row[i];
    }
}

/*
 * Decode attention for loop t (0-based) over the latent cache, all b and h.
 * For each (b, group g) every cached token's K and V are first reconstructed explicitly for
 * loop t; each head of the group then runs ordinary softmax attention over its d-slice
 * (attention unchanged: "What carries the argument").  Two-pass softmax.
 * k_self / v_self may both be NULL (cache only).  Returns 0, or -1 on bad arguments.
 */
int oracle_decode(int mode, int T, int H, int d, int r_k, int r_v, int t,
                  const double *W_up_k, const double *W_up_v,
                  const double *mu_k, const double *mu_v,
                  const double *k_pool, const double *v_pool,
                  const int32_t *block_table, const int32_t *seq_lens,
                  int B, int P, int max_pages,
                  const double *q, const double *k_self, const double *v_self,
                  long self_stride, double scale, double *out) {
    if (t < 0 || t >= T || (k_self == NULL) != (v_self == NULL)) return -1;
    const int G = (mode == 1) ? 1 : H;
    const int Dg = (mode == 1) ? H * d : d;
    const int hpg = H / G; /* heads per group */
    const size_t X = (size_t)T * Dg;
    if (self_stride <= 0) self_stride = (long)H * d;

    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < G; ++g) {
            const int len = seq_lens[b];
            const int n_scores = len + (k_self ? 1 : 0);
            double *xk = (double *)malloc(sizeof(double) * Dg);
            double *xv = (double *)malloc(sizeof(double) * Dg);
            double *s = (double *)malloc(sizeof(double) * ((size_t)n_scores * hpg + 1));
            double *acc = (double *)calloc((size_t)hpg * d, sizeof(double));
            if (!xk || !xv || !s || !acc) {
#pragma omp atomic write
                failed = 1;
                free(xk); free(xv); free(s); free(acc);
                continue;
            }
            const double *Wk = W_up_k + ((size_t)t * G + g) * r_k * Dg;
            const double *Wv = W_up_v + ((size_t)t * G + g) * r_v * Dg;
            const double *mk = mu_k + (size_t)g * X + (size_t)t * Dg;
            const double *mv = mu_v + (size_t)g * X + (size_t)t * Dg;

            /* pass 1: scores s_j = scale * <q_h, K_hat_j[h-slice]> */
            for (int j = 0; j < len; ++j) {
                const double *ck = latent_at(k_pool, block_table, max_pages, G, P, r_k, b, j, g);
                reconstruct(ck, r_k, Wk, mk, Dg, xk);
                for (int hl = 0; hl < hpg; ++hl) {
                    const int h = g * hpg + hl;
                    const double *qh = q + ((size_t)b * H + h) * d;
                    double dot = 0.0;
                    for (int i = 0; i < d; ++i) dot += qh[i] * xk[hl * d + i];
                    s[(size_t)j * hpg + hl] = scale * dot;
                }
            }
            if (k_self) {
                for (int hl = 0; hl < hpg; ++hl) {
                    const int h = g * hpg + hl;
                    const double *qh = q + ((size_t)b * H + h) * d;
                    const double *kh = k_self + (size_t)b * self_stride + (size_t)h * d;
                    double dot = 0.0;
                    for (int i = 0; i < d; ++i) dot += qh[i] * kh[i];
                    s[(size_t)len * hpg + hl] = scale * dot;
                }
            }
            /* pass 2: w_j = exp(s_j - max s), out = sum_j w_j V_hat_j / sum_j w_j */
            for (int hl = 0; hl < hpg; ++hl) {
                double m = -INFINITY, Z = 0.0;
                for (int j = 0; j < n_scores; ++j) m = fmax(m, s[(size_t)j * hpg + hl]);
                for (int j = 0; j < n_scores; ++j) {
                    double w = exp(s[(size_t)j * hpg + hl] - m);
                    s[(size_t)j * hpg + hl] = w;
                    Z += w;
                }
                for (int j = 0; j < n_scores; ++j) s[(size_t)j * hpg + hl] /= (Z > 0 ? Z : 1.0);
            }
            for (int j = 0; j < len; ++j) {
                const double *cv = latent_at(v_pool, block_table, max_pages, G, P, r_v, b, j, g);
                reconstruct(cv, r_v, Wv, mv, Dg, xv);
                for (int hl = 0; hl < hpg; ++hl)
                    for (int i = 0; i < d; ++i)
                        acc[hl * d + i] += s[(size_t)j * hpg + hl] * xv[hl * d + i];
            }
            if (v_self) {
                for (int hl = 0; hl < hpg; ++hl) {
                    const int h = g * hpg + hl;
                    const double *vh = v_self + (size_t)b * self_stride + (size_t)h * d;
                    for (int i = 0; i < d; ++i)
                        acc[hl * d + i] += s[(size_t)len * hpg + hl] * vh[i];
                }
            }
            for (int hl = 0; hl < hpg; ++hl) {
                const int h = g * hpg + hl;
                for (int i = 0; i < d; ++i) out[((size_t)b * H + h) * d + i] = acc[hl * d + i];
            }
            free(xk); free(xv); free(s); free(acc);
        }
    }
    return failed ? -2 : 0;
}

/*
 * Rotary position embedding (the rotation of RoFormer, which the pages cite; their free-parameter
 * ledger records the assumption that a token keeps one position at every recurrence step, so the
 * rotation can be applied after reconstruction to the pre-rotation K the codec stores).
 * Rotates the first rot_dims entries of x (length >= rot_dims, rot_dims even) to position pos:
 * pair m (0 <= m < rot_dims/2) has frequency f_m = theta^(-2m/rot_dims) and angle a = pos f_m,
 *   style 0 (half split):  pair (m, m + rot_dims/2)
 *   style 1 (interleaved): pair (2m, 2m + 1)
 * and (x_a, x_b) -> (x_a cos a - x_b sin a, x_a sin a + x_b cos a).  Entries past rot_dims are
 * left unchanged.  Returns 0, or -1 on bad arguments.
 */
int oracle_rope_rotate(double *x, int rot_dims, int style, double theta, double pos) {
    if (rot_dims < 0 || (rot_dims & 1) || theta <= 0.0 || (style != 0 && style != 1)) return -1;
    const int half = rot_dims / 2;
    for (int m = 0; m < half; ++m) {
        const double f = pow(theta, -2.0 * m / (double)rot_dims);
        const double a = pos * f;
        const double c = cos(a), s = sin(a);
        const int ia = style == 0 ? m : 2 * m;
        const int ib = style == 0 ? m + half : 2 * m + 1;
        const double xa = x[ia], xb = x[ib];
        x[ia] = xa * c - xb * s;
        x[ib] = xa * s + xb * c;
    }
    return 0;
}

/*
 * Decode attention for loop t with the rotation applied after reconstruction: every cached
 * token j's K_hat_t(j) (mu_t included) is rotated to position j, the current token's own key
 * k_self to position seq_lens[b] (its position in the sequence); q is taken as given (already
 * rotated by the caller to that same position); V is not rotated.  Otherwise identical to
 * oracle_decode (explicit reconstruction, two-pass softmax, same self-term convention).
 * rot_dims in [0, d] and even; rot_dims = 0 reproduces oracle_decode exactly.
 */
int oracle_decode_rope(int mode, int T, int H, int d, int r_k, int r_v, int t,
                       const double *W_up_k, const double *W_up_v,
                       const double *mu_k, const double *mu_v,
                       const double *k_pool, const double *v_pool,
                       const int32_t *block_table, const int32_t *seq_lens,
                       int B, int P, int max_pages,
                       const double *q, const double *k_self, const double *v_self,
                       long self_stride, double scale, double theta, int rot_dims, int style,
                       double *out) {
    if (t < 0 || t >= T || (k_self == NULL) != (v_self == NULL)) return -1;
    if (rot_dims < 0 || rot_dims > d || (rot_dims & 1) || theta <= 0.0 ||
        (style != 0 && style != 1))
        return -1;
    const int G = (mode == 1) ? 1 : H;
    const int Dg = (mode == 1) ? H * d : d;
    const int hpg = H / G;
    const size_t X = (size_t)T * Dg;
    if (self_stride <= 0) self_stride = (long)H * d;

    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < G; ++g) {
            const int len = seq_lens[b];
            const int n_scores = len + (k_self ? 1 : 0);
            double *xk = (double *)malloc(sizeof(double) * Dg);
            double *xv = (double *)malloc(sizeof(double) * Dg);
            double *ks = (double *)malloc(sizeof(double) * d);
            double *s = (double *)malloc(sizeof(double) * ((size_t)n_scores * hpg + 1));
            double *acc = (double *)calloc((size_t)hpg * d, sizeof(double));
            if (!xk || !xv || !ks || !s || !acc) {
#pragma omp atomic write
                failed = 1;
                free(xk); free(xv); free(ks); free(s); free(acc);
                continue;
            }
            const double *Wk = W_up_k + ((size_t)t * G + g) * r_k * Dg;
            const double *Wv = W_up_v + ((size_t)t * G + g) * r_v * Dg;
            const double *mk = mu_k + (size_t)g * X + (size_t)t * Dg;
            const double *mv = mu_v + (size_t)g * X + (size_t)t * Dg;

            for (int j = 0; j < len; ++j) {
                const double *ck = latent_at(k_pool, block_table, max_pages, G, P, r_k, b, j, g);
                reconstruct(ck, r_k, Wk, mk, Dg, xk);
                for (int hl = 0; hl < hpg; ++hl) {
                    double *kh = xk + (size_t)hl * d;
                    oracle_rope_rotate(kh, rot_dims, style, theta, (double)j);
                    const int h = g * hpg + hl;
                    const double *qh = q + ((size_t)b * H + h) * d;
                    double dot = 0.0;
                    for (int i = 0; i < d; ++i) dot += qh[i] * kh[i];
                    s[(size_t)j * hpg + hl] = scale * dot;
                }
            }
            if (k_self) {
                for (int hl = 0; hl < hpg; ++hl) {
                    const int h = g * hpg + hl;
                    const double *qh = q + ((size_t)b * H + h) * d;
                    memcpy(ks, k_self + (size_t)b * self_stride + (size_t)h * d,
                           sizeof(double) * d);
                    oracle_rope_rotate(ks, rot_dims, style, theta, (double)len);
                    double dot = 0.0;
                    for (int i = 0; i < d; ++i) dot += qh[i] * ks[i];
                    s[(size_t)len * hpg + hl] = scale * dot;
                }
            }
            for (int hl = 0; hl < hpg; ++hl) {
                double m = -INFINITY, Z = 0.0;
                for (int j = 0; j < n_scores; ++j) m = fmax(m, s[(size_t)j * hpg + hl]);
                for (int j = 0; j < n_scores; ++j) {
                    double w = exp(s[(size_t)j * hpg + hl] - m);
                    s[(size_t)j * hpg + hl] = w;
                    Z += w;
                }
                for (int j = 0; j < n_scores; ++j) s[(size_t)j * hpg + hl] /= (Z > 0 ? Z : 1.0);
            }
            for (int j = 0; j < len; ++j) {
                const double *cv = latent_at(v_pool, block_table, max_pages, G, P, r_v, b, j, g);
                reconstruct(cv, r_v, Wv, mv, Dg, xv);
                for (int hl = 0; hl < hpg; ++hl)
                    for (int i = 0; i < d; ++i)
                        acc[hl * d + i] += s[(size_t)j * hpg + hl] * xv[hl * d + i];
            }
            if (v_self) {
                for (int hl = 0; hl < hpg; ++hl) {
                    const int h = g * hpg + hl;
                    const double *vh = v_self + (size_t)b * self_stride + (size_t)h * d;
                    for (int i = 0; i < d; ++i)
                        acc[hl * d + i] += s[(size_t)len * hpg + hl] * vh[i];
                }
            }
            for (int hl = 0; hl < hpg; ++hl) {
                const int h = g * hpg + hl;
                for (int i = 0; i < d; ++i) out[((size_t)b * H + h) * d + i] = acc[hl * d + i];
            }
            free(xk); free(xv); free(ks); free(s); free(acc);
        }
    }
    return failed ? -2 : 0;
}

/*
 * Encode: c = (x - mu) W_down for one axis (pith.science paper page, "What carries the
 * argument": the loop-step vectors joined into one, the mean removed, the rest projected).
 * x is the staging buffer [B][T][H][d].  The stacked vector of group g is
 *   per-head: xs[t*d + i]         = x[b][t][g][i]
 *   LLA-2D:   xs[(t*H + h)*d + i] = x[b][t][h][i]
 * c_out is [B][G][r].
 */
int oracle_encode(int mode, int T, int H, int d, int r, const double *W_down, const double *mu,
                  const double *x, int B, double *c_out) {
    const int G = (mode == 1) ? 1 : H;
    const int Dg = (mode == 1) ? H * d : d;
    const size_t X = (size_t)T * Dg;
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < G; ++g) {
            double *c = c_out + ((size_t)b * G + g) * r;
            for (int k = 0; k < r; ++k) c[k] = 0.0;
            for (int tt = 0; tt < T; ++tt) {
                for (int hl = 0; hl < H / G; ++hl) {
                    const int h = (mode == 1) ? hl : g;
                    for (int i = 0; i < d; ++i) {
                        const size_t xi = ((size_t)tt * (H / G) + hl) * d + i; /* stacked index */
                        const double centred =
                            x[(((size_t)b * T + tt) * H + h) * d + i] - mu[(size_t)g * X + xi];
                        const double *wrow = W_down + ((size_t)g * X + xi) * r;
                        for (int k = 0; k < r; ++k) c[k] += centred * wrow[k];
                    }
                }
            }
        }
    }
    return 0;
}

/* Append: write c[b][g][:] to the cache slot of logical position write_pos[b]
 * (page block_table[b][pos / P], slot pos % P).  pool is an fp64 copy of the latent pool. */
int oracle_append(int G, int r, const double *c, int B, const int32_t *write_pos,
                  const int32_t *block_table, int P, int max_pages, double *pool) {
    for (int b = 0; b < B; ++b) {
        const int pos = write_pos[b];
        if (pos < 0 || pos / P >= max_pages) return -1;
        const int page = block_table[(size_t)b * max_pages + pos / P];
        for (int g = 0; g < G; ++g)
            for (int k = 0; k < r; ++k)
                pool[(((size_t)page * G + g) * P + pos % P) * r + k] = c[((size_t)b * G + g) * r + k];
    }
    return 0;
}

/*
 * Flat comparator: ordinary softmax attention of loop t's query over an uncompressed
 * loop-t cache (Figure 1 caption: each recurrent step contributes its own K_t, V_t).
 * Pools [n_pages][H][P][d].  Same self-term convention as oracle_decode.
 */
int oracle_flat_attn(int H, int d, const double *k_pool, const double *v_pool,
                     const int32_t *block_table, const int32_t *seq_lens, int B, int P,
                     int max_pages, const double *q, const double *k_self, const double *v_self,
                     long self_stride, double scale, double *out) {
    if ((k_self == NULL) != (v_self == NULL)) return -1;
    if (self_stride <= 0) self_stride = (long)H * d;
    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            const int len = seq_lens[b];
            const int n = len + (k_self ? 1 : 0);
            double *w = (double *)malloc(sizeof(double) * ((size_t)n + 1));
            if (!w) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            const double *qh = q + ((size_t)b * H + h) * d;
            double m = -INFINITY, Z = 0.0;
            for (int j = 0; j < n; ++j) {
                const double *kj;
                if (j < len) {
                    const int page = block_table[(size_t)b * max_pages + j / P];
                    kj = k_pool + (((size_t)page * H + h) * P + j % P) * d;
                } else {
                    kj = k_self + (size_t)b * self_stride + (size_t)h * d;
                }
                double dot = 0.0;
                for (int i = 0; i < d; ++i) dot += qh[i] * kj[i];
                w[j] = scale * dot;
                m = fmax(m, w[j]);
            }
            for (int j = 0; j < n; ++j) { w[j] = exp(w[j] - m); Z += w[j]; }
            double *o = out + ((size_t)b * H + h) * d;
            for (int i = 0; i < d; ++i) o[i] = 0.0;
            for (int j = 0; j < n; ++j) {
                const double *vj;
                if (j < len) {
                    const int page = block_table[(size_t)b * max_pages + j / P];
                    vj = v_pool + (((size_t)page * H + h) * P + j % P) * d;
                } else {
                    vj = v_self + (size_t)b * self_stride + (size_t)h * d;
                }
                for (int i = 0; i < d; ++i) o[i] += (w[j] / Z) * vj[i];
            }
            free(w);
        }
    }
    return failed ? -2 : 0;
}

/*
 * Chunked prefill attention for loop t (0-based).  The pages say nothing of prefill; the reading
 * taken is the decode rule above applied to a chunk of new tokens at once: new token i of
 * sequence b (0 <= i < n_new[b], logical position seq_lens[b] + i) attends to every cached token
 * j < seq_lens[b] through the codec (K_hat_t(j), V_hat_t(j) reconstructed explicitly, as in
 * oracle_decode) and, causally, to the chunk's own loop-t keys/values i' <= i, taken as given
 * (their latents are written only after the last loop, like the decode self term).
 *   q, out        [B][Pn][H][d]
 *   k_new, v_new  rows at k_new[(b*Pn + i)*new_stride + h*d]  (new_stride <= 0 means H*d)
 *   n_new         [B], values clamped to [0, Pn]
 * Rows i >= n_new[b] of out are not written.  Two-pass softmax per (b, i, h).
 * Returns 0, -1 on bad arguments, -2 when memory runs out.
 */
int oracle_prefill(int mode, int T, int H, int d, int r_k, int r_v, int t,
                   const double *W_up_k, const double *W_up_v,
                   const double *mu_k, const double *mu_v,
                   const double *k_pool, const double *v_pool,
                   const int32_t *block_table, const int32_t *seq_lens,
                   int B, int P, int max_pages, int Pn, const int32_t *n_new,
                   const double *q, const double *k_new, const double *v_new,
                   long new_stride, double scale, double *out) {
    if (t < 0 || t >= T || Pn < 0 || !k_new || !v_new || !n_new) return -1;
    const int G = (mode == 1) ? 1 : H;
    const int Dg = (mode == 1) ? H * d : d;
    const int hpg = H / G;
    const size_t X = (size_t)T * Dg;
    if (new_stride <= 0) new_stride = (long)H * d;

    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < G; ++g) {
            const int len = seq_lens[b];
            const int nn = n_new[b] < 0 ? 0 : (n_new[b] > Pn ? Pn : n_new[b]);
            /* every cached token reconstructed once for loop t: Kc, Vc [len][Dg] */
            double *Kc = (double *)malloc(sizeof(double) * ((size_t)len * Dg + 1));
            double *Vc = (double *)malloc(sizeof(double) * ((size_t)len * Dg + 1));
            double *s = (double *)malloc(sizeof(double) * ((size_t)len + nn + 1));
            if (!Kc || !Vc || !s) {
#pragma omp atomic write
                failed = 1;
                free(Kc); free(Vc); free(s);
                continue;
            }
            const double *Wk = W_up_k + ((size_t)t * G + g) * r_k * Dg;
            const double *Wv = W_up_v + ((size_t)t * G + g) * r_v * Dg;
            const double *mk = mu_k + (size_t)g * X + (size_t)t * Dg;
            const double *mv = mu_v + (size_t)g * X + (size_t)t * Dg;
            for (int j = 0; j < len; ++j) {
                reconstruct(latent_at(k_pool, block_table, max_pages, G, P, r_k, b, j, g), r_k,
                            Wk, mk, Dg, Kc + (size_t)j * Dg);
                reconstruct(latent_at(v_pool, block_table, max_pages, G, P, r_v, b, j, g), r_v,
                            Wv, mv, Dg, Vc + (size_t)j * Dg);
            }
            for (int i = 0; i < nn; ++i) {
                for (int hl = 0; hl < hpg; ++hl) {
                    const int h = g * hpg + hl;
                    const double *qh = q + (((size_t)b * Pn + i) * H + h) * d;
                    const int n = len + i + 1;          /* cached tokens, then new 0..i */
                    for (int j = 0; j < n; ++j) {
                        const double *kj = j < len
                            ? Kc + (size_t)j * Dg + (size_t)hl * d
                            : k_new + ((size_t)b * Pn + (j - len)) * new_stride + (size_t)h * d;
                        double dot = 0.0;
                        for (int e = 0; e < d; ++e) dot += qh[e] * kj[e];
                        s[j] = scale * dot;
                    }
                    double m = -INFINITY, Z = 0.0;
                    for (int j = 0; j < n; ++j) m = fmax(m, s[j]);
                    for (int j = 0; j < n; ++j) {
                        s[j] = exp(s[j] - m);
                        Z += s[j];
                    }
                    double *o = out + (((size_t)b * Pn + i) * H + h) * d;
                    for (int e = 0; e < d; ++e) o[e] = 0.0;
                    for (int j = 0; j < n; ++j) {
                        const double *vj = j < len
                            ? Vc + (size_t)j * Dg + (size_t)hl * d
                            : v_new + ((size_t)b * Pn + (j - len)) * new_stride + (size_t)h * d;
                        const double w = s[j] / Z;
                        for (int e = 0; e < d; ++e) o[e] += w * vj[e];
                    }
                }
            }
            free(Kc); free(Vc); free(s);
        }
    }
    return failed ? -2 : 0;
}
