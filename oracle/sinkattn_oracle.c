/*
 * sinkattn_oracle.c -- plain fp64 CPU oracle for sink attention and partial RoPE.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only the
 * test suite, the package smoke check and the CPU-baseline leg of the benchmark
 * may load it.  It shares no code, header, table or helper with the HIP library.
 *
 * Everything here is the plain definition written out as loops, in double
 * precision, from the exact input values.  Sources (MiMo-V2-Flash Technical
 * Report, full translation, page "garden.houmin.site/digest/mimo-v2-flash"):
 *
 *   - Section 2.2, first equation: the logit between query i and key j of one
 *     head is a_ij = (q_i . k_j) / sqrt(d), d the per-head dimension.
 *   - Section 2.2, second and third equations: the weight of key j is
 *     s_ij = exp(a_ij - m_i) / ( exp(sink - m_i) + sum_j' exp(a_ij' - m_i) )
 *     with m_i = max( max_j a_ij , sink ), one learnable scalar sink per head.
 *   - Section 2.2, fourth equation: o_i = sum_j s_ij v_j (the sink has no value).
 *   - Section 2.1 and Table 1: GQA (64 query heads over 8 KV heads for SWA,
 *     over 4 for GA), QK head dim 192, V head dim 128, W = 128; RoPE only on the
 *     first 64 dims of q and k.
 *   - Section 3.2 ("long-context extension"): RoPE base 10,000 for SWA and
 *     640,000 then 5,000,000 for GA.
 *
 * Readings where the pages leave a step open (each one is also listed with its
 * reason in the design notes of the repository):
 *   - d in 1/sqrt(d) is the QK dim (the contracted one); scale is a parameter.
 *   - A window W holds W keys including the query itself: p_q - W < p_k <= p_q.
 *   - The denominator sum runs over the same visible keys as the numerator.
 *   - One sink per query head; sink is a raw logit (not divided by sqrt(d));
 *     it carries no value.
 *   - Query head h reads KV head h / (Hq / Hkv) (contiguous groups).
 *   - Empty visible set (cannot happen for a causal self-inclusive window but
 *     defined anyway): o = 0 and lse = sink.
 *   - RoPE (RoFormer, cited by Section 2.1): interleaved pairs (2c, 2c+1),
 *     angle p * base^(-2c/rope_dim) for c < rope_dim/2, computed in fp64;
 *     style 1 pairs (c, c + rope_dim/2) instead.  Dims >= rope_dim unchanged.
 *
 * Parity pins for these functions live in tests/test_oracle_pins.py.
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

/*
 * Sink attention for ONE sequence, every (query row, query head) pair.
 *
 *   q    [nq, hq, dqk]     k [nk, hkv, dqk]     v [nk, hkv, dv]
 *   qpos [nq]  absolute position of each query row
 *   kpos [nk]  absolute position of each key row (a negative position marks an
 *              empty slot that no query can see)
 *   sink [hq]  one logit per query head (-INFINITY disables it)
 *   window     > 0: key visible iff qpos - W < kpos <= qpos; <= 0: kpos <= qpos
 *   o    [nq, hq, dv]  out;  lse [nq, hq] out (may be NULL): m + ln Z
 *
 * Returns 0, or -1 on a bad argument.
 */
int oracle_sink_attention(const double *q, const double *k, const double *v,
                          const int64_t *qpos, const int64_t *kpos,
                          const double *sink, int64_t nq, int64_t nk, int hq,
                          int hkv, int dqk, int dv, int64_t window, double scale,
                          double *o, double *lse) {
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || dqk <= 0 || dv <= 0 || nq < 0 ||
        nk < 0)
        return -1;
    const int group = hq / hkv;
    int bad = 0;

#pragma omp parallel
    {
        double *a = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        char *vis = (char *)malloc((size_t)(nk > 0 ? nk : 1));
        if (!a || !vis) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t row = 0; row < nq * hq; ++row) {
            if (!a || !vis)
                continue;
            const int64_t i = row / hq;
            const int h = (int)(row % hq);
            const int g = h / group;
            const double *qi = q + (i * hq + h) * dqk;

            /* visible set J_i and the logits a_ij (Section 2.2, eq. 1) */
            double m = sink[h];
            for (int64_t j = 0; j < nk; ++j) {
                const int64_t dp = qpos[i] - kpos[j];
                vis[j] = (kpos[j] >= 0) && (dp >= 0) && (window <= 0 || dp < window);
                if (!vis[j])
                    continue;
                const double *kj = k + (j * hkv + g) * dqk;
                double dot = 0.0;
                for (int c = 0; c < dqk; ++c)
                    dot += qi[c] * kj[c];
                a[j] = dot * scale;
                if (a[j] > m) /* m_i = max(max_j a_ij, sink) (eq. 3) */
                    m = a[j];
            }

            /* denominator Z_i = exp(sink - m) + sum_j exp(a_ij - m) (eq. 2) */
            double z = (sink[h] == -INFINITY) ? 0.0 : exp(sink[h] - m);
            for (int64_t j = 0; j < nk; ++j)
                if (vis[j])
                    z += exp(a[j] - m);

            /* o_i = sum_j s_ij v_j (eq. 4); the sink contributes no value */
            double *oi = o + (i * hq + h) * dv;
            for (int c = 0; c < dv; ++c)
                oi[c] = 0.0;
            if (z > 0.0) {
                for (int64_t j = 0; j < nk; ++j) {
                    if (!vis[j])
                        continue;
                    const double s = exp(a[j] - m) / z;
                    const double *vj = v + (j * hkv + g) * dv;
                    for (int c = 0; c < dv; ++c)
                        oi[c] += s * vj[c];
                }
            }
            if (lse)
                lse[i * hq + h] = (z > 0.0) ? m + log(z) : -INFINITY;
        }
        free(a);
        free(vis);
    }
    return bad ? -1 : 0;
}

/*
 * Partial RoPE (Section 2.1: rotary on the first 64 dims of q and k; RoFormer).
 *   x, y [n_tok, n_heads, head_dim]; pos [n_tok].  y may equal x.
 *   style 0: pairs (2c, 2c+1); style 1: pairs (c, c + rope_dim/2).
 *   angle_c = pos * base^(-2c / rope_dim), c = 0 .. rope_dim/2 - 1, in fp64.
 */
int oracle_rope_partial(const double *x, double *y, int64_t n_tok, int n_heads,
                        int head_dim, int rope_dim, const int64_t *pos,
                        double base, int style) {
    if (rope_dim < 0 || rope_dim % 2 != 0 || rope_dim > head_dim || n_tok < 0 ||
        n_heads < 0 || !(base > 0.0) || (style != 0 && style != 1))
        return -1;
    const int half = rope_dim / 2;
    for (int64_t t = 0; t < n_tok; ++t) {
        for (int h = 0; h < n_heads; ++h) {
            const double *xi = x + (t * n_heads + h) * head_dim;
            double *yi = y + (t * n_heads + h) * head_dim;
            double tmp[1024];
            const int n = head_dim < 1024 ? head_dim : 1024;
            for (int c = 0; c < n; ++c)
                tmp[c] = xi[c];
            for (int c = 0; c < half; ++c) {
                const double theta = pow(base, -2.0 * (double)c / (double)rope_dim);
                const double phi = (double)pos[t] * theta;
                const int i0 = style == 0 ? 2 * c : c;
                const int i1 = style == 0 ? 2 * c + 1 : c + half;
                const double x0 = tmp[i0], x1 = tmp[i1];
                tmp[i0] = x0 * cos(phi) - x1 * sin(phi);
                tmp[i1] = x0 * sin(phi) + x1 * cos(phi);
            }
            for (int c = 0; c < n; ++c)
                yi[c] = tmp[c];
        }
    }
    return 0;
}

/*
 * Round each double once, to nearest with ties to even, into bfloat16 (8
 * significant bits, fp32's exponent range; subnormals step 2^-133).  Writes the
 * 16-bit patterns.  NaN maps to the canonical quiet NaN 0x7FC0.
 */
void oracle_round_bf16(const double *x, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        const double d = x[i];
        uint16_t sign = signbit(d) ? 0x8000u : 0u;
        if (isnan(d)) {
            out[i] = 0x7FC0u;
            continue;
        }
        const double a = fabs(d);
        if (isinf(a)) {
            out[i] = sign | 0x7F80u;
            continue;
        }
        double r;
        if (a == 0.0) {
            r = 0.0;
        } else {
            int e;
            frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
            /* a value with exponent e has ulp 2^(e-8); below the normal range the
               ulp is fixed at 2^-133 */
            int ulp_exp = e - 8;
            if (ulp_exp < -133)
                ulp_exp = -133;
            r = ldexp(nearbyint(ldexp(a, -ulp_exp)), ulp_exp);
        }
        /* largest finite bf16 is (2 - 2^-7) * 2^127 */
        if (r > ldexp(2.0 - ldexp(1.0, -7), 127)) {
            out[i] = sign | 0x7F80u;
            continue;
        }
        float f = (float)r; /* exact: r has <= 8 significant bits */
        uint32_t bits;
        memcpy(&bits, &f, 4);
        out[i] = sign | (uint16_t)((bits >> 16) & 0x7FFFu);
    }
}

/*
 * Gradients of oracle_sink_attention for an upstream gradient dout of the loss
 * with respect to o (same layout as o).  Derived from the Section 2.2
 * definitions by the chain rule, with s_ij = e^(a_ij) / Z_i,
 * Z_i = e^(sink) + sum_j e^(a_ij) and p_i = e^(sink) / Z_i (the sink's share):
 *   dv_j   += sum_i s_ij dout_i                          (o_i = sum_j s_ij v_j)
 *   dP_ij   = dout_i . v_j,   D_i = sum_j s_ij dP_ij = dout_i . o_i
 *   dA_ij   = s_ij (dP_ij - D_i)                          (softmax over J_i + sink)
 *   dq_i    = scale sum_j dA_ij k_j,   dk_j += scale sum_i dA_ij q_i
 *   dsink_h = - sum_i p_i D_i   (the sink column has no value, so its dP is 0)
 * dk and dv sum over the query heads of the KV group.  Outputs are overwritten:
 *   dq [nq, hq, dqk]   dk [nk, hkv, dqk]   dv [nk, hkv, dv]   dsink [hq]
 * Plain loops in fp64; the forward weights are recomputed.  Returns 0 / -1.
 */
int oracle_sink_attention_bwd(const double *q, const double *k, const double *v,
                              const int64_t *qpos, const int64_t *kpos,
                              const double *sink, const double *dout, int64_t nq,
                              int64_t nk, int hq, int hkv, int dqk, int dv,
                              int64_t window, double scale, double *dq, double *dk,
                              double *dvv, double *dsink) {
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || dqk <= 0 || dv <= 0 || nq < 0 ||
        nk < 0)
        return -1;
    const int group = hq / hkv;
    memset(dq, 0, sizeof(double) * (size_t)(nq * hq * dqk));
    memset(dk, 0, sizeof(double) * (size_t)(nk * hkv * dqk));
    memset(dvv, 0, sizeof(double) * (size_t)(nk * hkv * dv));
    for (int h = 0; h < hq; ++h)
        dsink[h] = 0.0;
    int bad = 0;

    /* one KV group per iteration: its dk / dv rows and its heads' dq / dsink
     * are written by that iteration only */
#pragma omp parallel for schedule(dynamic, 1)
    for (int g = 0; g < hkv; ++g) {
        double *a = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        double *oi = (double *)malloc(sizeof(double) * (size_t)dv);
        char *vis = (char *)malloc((size_t)(nk > 0 ? nk : 1));
        if (!a || !s || !oi || !vis) {
#pragma omp atomic write
            bad = 1;
        } else {
            for (int h = g * group; h < (g + 1) * group; ++h) {
                for (int64_t i = 0; i < nq; ++i) {
                    const double *qi = q + (i * hq + h) * dqk;
                    const double *di = dout + (i * hq + h) * dv;
                    double m = sink[h];
                    for (int64_t j = 0; j < nk; ++j) {
                        const int64_t dp = qpos[i] - kpos[j];
                        vis[j] = (kpos[j] >= 0) && (dp >= 0) && (window <= 0 || dp < window);
                        if (!vis[j])
                            continue;
                        const double *kj = k + (j * hkv + g) * dqk;
                        double dot = 0.0;
                        for (int c = 0; c < dqk; ++c)
                            dot += qi[c] * kj[c];
                        a[j] = dot * scale;
                        if (a[j] > m)
                            m = a[j];
                    }
                    double z = (sink[h] == -INFINITY) ? 0.0 : exp(sink[h] - m);
                    for (int64_t j = 0; j < nk; ++j)
                        if (vis[j])
                            z += exp(a[j] - m);
                    if (!(z > 0.0))
                        continue; /* nothing visible and no sink: o = 0, no gradient */
                    const double p_sink = (sink[h] == -INFINITY) ? 0.0 : exp(sink[h] - m) / z;
                    for (int c = 0; c < dv; ++c)
                        oi[c] = 0.0;
                    for (int64_t j = 0; j < nk; ++j) {
                        if (!vis[j])
                            continue;
                        s[j] = exp(a[j] - m) / z;
                        const double *vj = v + (j * hkv + g) * dv;
                        for (int c = 0; c < dv; ++c)
                            oi[c] += s[j] * vj[c];
                    }
                    double D = 0.0;
                    for (int c = 0; c < dv; ++c)
                        D += di[c] * oi[c];
                    dsink[h] -= p_sink * D;
                    double *dqi = dq + (i * hq + h) * dqk;
                    for (int64_t j = 0; j < nk; ++j) {
                        if (!vis[j])
                            continue;
                        const double *vj = v + (j * hkv + g) * dv;
                        const double *kj = k + (j * hkv + g) * dqk;
                        double *dvj = dvv + (j * hkv + g) * dv;
                        double *dkj = dk + (j * hkv + g) * dqk;
                        double dP = 0.0;
                        for (int c = 0; c < dv; ++c) {
                            dP += di[c] * vj[c];
                            dvj[c] += s[j] * di[c];
                        }
                        const double dA = s[j] * (dP - D);
                        for (int c = 0; c < dqk; ++c) {
                            dqi[c] += scale * dA * kj[c];
                            dkj[c] += scale * dA * qi[c];
                        }
                    }
                }
            }
        }
        free(a);
        free(s);
        free(oi);
        free(vis);
    }
    return bad ? -1 : 0;
}
