/*
 * FP64 reference for cross-entropy over a large vocabulary.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code with the HIP kernels.
 *
 * It computes the plain textbook definitions, row by row, in double precision:
 *
 *   p_v   = softmax(z)_v = exp(z_v - lse),   lse = m + ln sum_v exp(z_v - m),
 *           m = max_v z_v                      (online-softmax contract of the
 *           TransformerEngine cross-entropy page, Description)
 *   q_v   = (1 - eps) [v = t] + eps / V        (label smoothing, same page,
 *           I/O Contract; the mass eps/V goes to every class, target included)
 *   loss  = - sum_v q_v ln p_v                 (terms with q_v = 0 are skipped)
 *   grad  = g (p_v - q_v)                      (gradient rebuilt from saved
 *           statistics, TransformerEngine PR "Minimize the memory usage of
 *           the fused cross entropy kernel", Changes and Sequence Diagram)
 *
 * A row whose target equals ignore_idx has loss 0 and gradient 0 (same API
 * page, I/O Contract, ignore_idx).  A row whose target is neither ignore_idx
 * nor in [0, V) has NaN loss and NaN gradient (the pages are silent; this is
 * the reading both sides follow).
 *
 * Saved statistics per row (same PR, Sequence Diagram "max/denominator
 * stats"): m, d = sum_v exp(z_v - m), z_t and mean_v z_v.
 *
 * Entropy of the predicted distribution (the optional entropy output of the
 * Liger-Kernel fused cross-entropy PR, Summary), also by definition:
 *
 *   H     = - sum_v p_v ln p_v                 (terms with p_v = 0 skipped)
 *   dH/dz_v = - p_v (ln p_v + H)               (differentiating the sum term
 *           by term through dp_u/dz_v = p_u ([u = v] - p_v))
 *
 * and a row's gradient gains gH * dH/dz when an upstream gradient gH of the
 * entropy is given.  Ignored rows have entropy 0 and no entropy gradient;
 * the entropy does not depend on the target otherwise.
 *
 * Logits are addressed as (d0, d1, V) with element strides ls0, ls1 for the
 * leading dimensions and 1 for V, which covers the (B,SQ,V) and (SQ,B,V)
 * layouts of the API page.  dtype: 0 = FP32, 1 = BF16 bit patterns (uint16),
 * 2 = FP64.  A BF16 value is widened exactly: bits << 16 read as FP32.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC ce_ref.c -o libce_ref.so -lm
 * (no fast-math: IEEE semantics for exp, log, inf and NaN are required).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double load_value(const void *base, int dtype, int64_t off)
{
    if (dtype == 0)
        return (double)((const float *)base)[off];
    if (dtype == 1) {
        uint32_t bits = ((uint32_t)((const uint16_t *)base)[off]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double *)base)[off];
}

static int64_t row_offset(int64_t r, int64_t d1, int64_t s0, int64_t s1)
{
    return (r / d1) * s0 + (r % d1) * s1;
}

/* Max, denominator and log-sum-exp of one row, straight from the definition. */
static void row_lse(const void *z, int dtype, int64_t base, int64_t V,
                    double *m_out, double *d_out, double *lse_out)
{
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double x = load_value(z, dtype, base + v);
        if (x > m || isnan(x))
            m = x;
        if (isnan(m))
            break;
    }
    double d = 0.0;
    if (isnan(m)) {
        d = NAN;
    } else if (isinf(m) && m < 0) {
        /* every logit is -inf: the softmax is undefined */
        d = NAN;
    } else {
        for (int64_t v = 0; v < V; ++v)
            d += exp(load_value(z, dtype, base + v) - m);
    }
    *m_out = m;
    *d_out = d;
    *lse_out = m + log(d);
}

int vce_oracle_forward(const void *logits, int dtype, int64_t d0, int64_t d1, int64_t V,
                       int64_t ls0, int64_t ls1, const int64_t *targets, int64_t ts0,
                       int64_t ts1, double eps, int64_t ignore_idx, const int64_t *rows,
                       int64_t nrows, double *loss, double *stats, double *loss_closed)
{
    if (!logits || !targets || !loss || V <= 0 || d0 < 0 || d1 <= 0)
        return 1;
    int64_t n = rows ? nrows : d0 * d1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = rows ? rows[i] : i;
        int64_t base = row_offset(r, d1, ls0, ls1);
        int64_t t = targets[row_offset(r, d1, ts0, ts1)];
        double *st = stats ? stats + 4 * i : NULL;
        if (t == ignore_idx) {
            loss[i] = 0.0;
            if (loss_closed)
                loss_closed[i] = 0.0;
            if (st)
                st[0] = st[1] = st[2] = st[3] = NAN;
            continue;
        }
        double m, d, lse;
        row_lse(logits, dtype, base, V, &m, &d, &lse);
        double zsum = 0.0;
        for (int64_t v = 0; v < V; ++v)
            zsum += load_value(logits, dtype, base + v);
        double mean = zsum / (double)V;
        int in_range = (t >= 0 && t < V);
        double zt = in_range ? load_value(logits, dtype, base + t) : NAN;

        /* Definition: -sum_v q_v ln p_v with ln p_v = z_v - lse. */
        double acc = 0.0;
        if (!in_range) {
            acc = NAN;
        } else {
            double qoff = eps / (double)V;
            for (int64_t v = 0; v < V; ++v) {
                double q = qoff + (v == t ? 1.0 - eps : 0.0);
                if (q == 0.0)
                    continue;
                acc -= q * (load_value(logits, dtype, base + v) - lse);
            }
        }
        loss[i] = acc;
        if (loss_closed) {
            /* Closed form of the smoothed loss: (1-eps)(lse - z_t) + eps (lse - mean z). */
            double c = (1.0 - eps) * (lse - zt);
            if (eps != 0.0)
                c += eps * (lse - mean);
            loss_closed[i] = c;
        }
        if (st) {
            st[0] = m;
            st[1] = d;
            st[2] = zt;
            st[3] = mean;
        }
    }
    return 0;
}

int vce_oracle_backward(const void *logits, int dtype, int64_t d0, int64_t d1, int64_t V,
                        int64_t ls0, int64_t ls1, const int64_t *targets, int64_t ts0,
                        int64_t ts1, double eps, int64_t ignore_idx, const double *g,
                        const int64_t *rows, int64_t nrows, double *grad)
{
    if (!logits || !targets || !g || !grad || V <= 0 || d0 < 0 || d1 <= 0)
        return 1;
    int64_t n = rows ? nrows : d0 * d1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = rows ? rows[i] : i;
        int64_t base = row_offset(r, d1, ls0, ls1);
        int64_t t = targets[row_offset(r, d1, ts0, ts1)];
        double *out = grad + i * V;
        if (t == ignore_idx) {
            for (int64_t v = 0; v < V; ++v)
                out[v] = 0.0;
            continue;
        }
        if (!(t >= 0 && t < V)) {
            for (int64_t v = 0; v < V; ++v)
                out[v] = NAN;
            continue;
        }
        double m, d, lse;
        row_lse(logits, dtype, base, V, &m, &d, &lse);
        double qoff = eps / (double)V;
        for (int64_t v = 0; v < V; ++v) {
            double p = exp(load_value(logits, dtype, base + v) - lse);
            double q = qoff + (v == t ? 1.0 - eps : 0.0);
            out[v] = g[i] * (p - q);
        }
    }
    return 0;
}

/* Entropy H = -sum_v p_v ln p_v of each row (0 for ignored rows). */
int vce_oracle_entropy(const void *logits, int dtype, int64_t d0, int64_t d1, int64_t V,
                       int64_t ls0, int64_t ls1, const int64_t *targets, int64_t ts0,
                       int64_t ts1, int64_t ignore_idx, const int64_t *rows, int64_t nrows,
                       double *ent)
{
    if (!logits || !targets || !ent || V <= 0 || d0 < 0 || d1 <= 0)
        return 1;
    int64_t n = rows ? nrows : d0 * d1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = rows ? rows[i] : i;
        int64_t base = row_offset(r, d1, ls0, ls1);
        int64_t t = targets[row_offset(r, d1, ts0, ts1)];
        if (t == ignore_idx) {
            ent[i] = 0.0;
            continue;
        }
        double m, d, lse;
        row_lse(logits, dtype, base, V, &m, &d, &lse);
        double h = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            double lp = load_value(logits, dtype, base + v) - lse; /* ln p_v */
            double p = exp(lp);
            if (p == 0.0)
                continue;
            h -= p * lp;
        }
        ent[i] = h;
    }
    return 0;
}

/* grad[i, v] += gH[i] * dH/dz_v with dH/dz_v = -p_v (ln p_v + H) (ignored
 * rows unchanged). */
int vce_oracle_entropy_grad(const void *logits, int dtype, int64_t d0, int64_t d1, int64_t V,
                            int64_t ls0, int64_t ls1, const int64_t *targets, int64_t ts0,
                            int64_t ts1, int64_t ignore_idx, const double *gH,
                            const int64_t *rows, int64_t nrows, double *grad)
{
    if (!logits || !targets || !gH || !grad || V <= 0 || d0 < 0 || d1 <= 0)
        return 1;
    int64_t n = rows ? nrows : d0 * d1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = rows ? rows[i] : i;
        int64_t base = row_offset(r, d1, ls0, ls1);
        int64_t t = targets[row_offset(r, d1, ts0, ts1)];
        if (t == ignore_idx)
            continue;
        double m, d, lse;
        row_lse(logits, dtype, base, V, &m, &d, &lse);
        double h = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            double lp = load_value(logits, dtype, base + v) - lse;
            double p = exp(lp);
            if (p != 0.0)
                h -= p * lp;
        }
        double *out = grad + i * V;
        for (int64_t v = 0; v < V; ++v) {
            double lp = load_value(logits, dtype, base + v) - lse;
            double p = exp(lp);
            if (p != 0.0)
                out[v] += gH[i] * (-p * (lp + h));
        }
    }
    return 0;
}

/* Round doubles to BF16 (nearest, ties to even), including BF16 subnormals.
 * The quantum at magnitude 2^e (e >= -126) is 2^(e-7); below 2^-126 it is
 * the subnormal quantum 2^-133.  nearbyint() rounds half to even in the
 * default rounding mode. */
void vce_oracle_round_bf16(const double *x, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double v = x[i];
        uint16_t sign = signbit(v) ? 0x8000u : 0u;
        double a = fabs(v);
        uint16_t bits;
        if (isnan(v)) {
            bits = 0x7FC0u;
        } else if (a == 0.0) {
            bits = sign;
        } else if (isinf(a)) {
            bits = 0x7F80u | sign;
        } else {
            int e = ilogb(a);
            if (e < -126)
                e = -126;
            double quantum = ldexp(1.0, e - 7);
            double r = nearbyint(a / quantum) * quantum;
            /* largest finite BF16 is (2 - 2^-7) * 2^127 */
            if (r >= ldexp(1.0, 128)) {
                bits = 0x7F80u;
            } else {
                float f = (float)r; /* exact: r has at most 8 significant bits */
                uint32_t fb;
                memcpy(&fb, &f, sizeof fb);
                bits = (uint16_t)(fb >> 16);
            }
            bits |= sign;
        }
        out[i] = bits;
    }
}

int vce_oracle_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
