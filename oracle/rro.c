/*
 * rro.c -- CPU oracle for the deterministic row-reduce path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or constant with the GPU library.
 *
 * Every float result is computed in IEEE double and rounded once at the end.
 * Build: gcc -O2 (no -ffast-math, no FMA contraction), single threaded.
 *
 * Sources (Modular API pages; section names as printed on the pages):
 *   [CA]  "cluster_allreduce" -- description and Parameters (combine_fn is an
 *         associative add/max/min over 32-bit elements; the fold visits ranks
 *         in ascending order).
 *   [RW]  "reduce" (algorithm.gpu.rowwise) -- tier semantics and the
 *         state-carrying overload (a monoid state folded tile by tile along
 *         the last axis); the two-pass softmax (pass 1 a monoid, pass 2 a map).
 *   [FA4] "fa4_splitk_reduce_scatter_write" -- the split-K combine: partials
 *         carry a per-row (max, sum); the combine scales each partition's
 *         output by its weight w[b], accumulates partitions and packs bf16;
 *         every partition, empty or not, takes part.
 *
 * Readings of the pages used here (each is restated where it is used):
 *   - float SUM accumulates in double in index order, rounds once (RNE).
 *   - int32 SUM wraps modulo 2^32.
 *   - float MAX/MIN order values by IEEE 754 totalOrder (so -0 < +0; a NaN
 *     with the sign bit clear is above +inf, one with it set below -inf).
 *   - softmax pass 1 is (max, sum exp(x - max)), pass 2 is exp(x - max)/sum,
 *     rounded once from double to the output type.
 *   - layernorm (named by [RW] as a two-pass algorithm: a statistics pass,
 *     then a pure map) is the usual per-row normalisation: mean, population
 *     variance (divide by n), rstd = 1 / sqrt(var + eps), then
 *     y = (x - mean) * rstd * gamma + beta per column, rounded once.
 *   - the LSE merge takes normalised partials O_p with row statistics
 *     (m_p, l_p); weight w_p = exp(scale*(m_p - M)) * l_p over the non-empty
 *     partitions (l_p > 0 and m_p > -inf), M their largest m_p; the output is
 *     sum_p (w_p / W) O_p with W = sum_p w_p; a row with no non-empty
 *     partition is zero; empty partitions are skipped, so their O_p is never
 *     read into the sum.
 *   - the split-K attention partials that the merge takes are, per query row
 *     and partition of the keys (P contiguous ranges p*n/P .. (p+1)*n/P), the
 *     scores s_j = scale * q.k_j, m_p = max s_j, l_p = sum exp(s_j - m_p) and
 *     O_p = sum exp(s_j - m_p) v_j / l_p; grouped query heads share key/value
 *     head h / (heads / kv_heads); a partition with no key is (-inf, 0, 0).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes used by this file's callers */
#define RRO_F32 0
#define RRO_I32 1
#define RRO_BF16 2
/* op codes */
#define RRO_SUM 0
#define RRO_MAX 1
#define RRO_MIN 2

#define RRO_OK 0
#define RRO_BAD 1

/* ------------------------------------------------------------------ bf16 */

/* Value of a bf16 bit pattern: bf16 is the top half of a binary32. */
double rro_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to the nearest bf16, ties to even (one rounding).
 * bf16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits; normal
 * numbers carry 8 significant bits; the subnormal quantum is 2^-133; the
 * largest finite value is (2 - 2^-7) * 2^127.  NaN maps to a quiet NaN with
 * the same sign.
 */
uint16_t rro_bf16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;

    int e;
    frexp(a, &e);               /* a = f * 2^e, 0.5 <= f < 1: leading bit is 2^(e-1) */
    int q = (e - 1) - 7;        /* weight of the last kept bit for a normal result */
    if (q < -133)
        q = -133;               /* subnormal range: fixed quantum */
    double n = rint(ldexp(a, -q));          /* default mode: nearest, ties to even */
    double r = ldexp(n, q);                 /* rounded magnitude */
    if (r > 0x1.FEp127)
        return (uint16_t)(sign | 0x7F80u);  /* rounds past the largest finite */
    if (r == 0.0)
        return sign;

    int e2;
    double f2 = frexp(r, &e2);
    if (e2 - 1 < -126)                      /* subnormal: r = k * 2^-133, k < 128 */
        return (uint16_t)(sign | (uint16_t)ldexp(r, 133));
    uint16_t exp_field = (uint16_t)(e2 - 1 + 127);
    uint16_t frac = (uint16_t)(ldexp(f2, 8) - 128.0);  /* f2 * 2^8 in [128, 256) */
    return (uint16_t)(sign | (exp_field << 7) | frac);
}

/* ------------------------------------------------------------ element I/O */

static double load_real(const void* base, int dtype, int64_t idx)
{
    if (dtype == RRO_F32)
        return (double)((const float*)base)[idx];
    return rro_bf16_to_double(((const uint16_t*)base)[idx]);
}

static void store_real(void* base, int dtype, int64_t idx, double v)
{
    if (dtype == RRO_F32)
        ((float*)base)[idx] = (float)v;     /* C conversion: round to nearest even */
    else
        ((uint16_t*)base)[idx] = rro_bf16_from_double(v);
}

/* --------------------------------------------------------- totalOrder */

/*
 * IEEE 754 totalOrder restricted to "a strictly before b" for binary32.
 * Every value whose sign bit is set precedes every value whose sign bit is
 * clear (this puts -0 before +0).  With equal signs, compare magnitudes: a
 * NaN's magnitude is above infinity and NaNs compare by payload; the larger
 * magnitude comes last for positive values and first for negative ones.
 */
static int f32_total_before(float a, float b)
{
    int sa = signbit(a) != 0, sb = signbit(b) != 0;
    if (sa != sb)
        return sa;
    int mag_less; /* |a| before |b| in magnitude order */
    int na = isnan(a), nb = isnan(b);
    if (!na && !nb) {
        mag_less = fabsf(a) < fabsf(b);
    } else if (na != nb) {
        mag_less = nb;  /* the NaN has the larger magnitude */
    } else {
        uint32_t ua, ub;
        memcpy(&ua, &a, 4);
        memcpy(&ub, &b, 4);
        mag_less = (ua & 0x007FFFFFu) < (ub & 0x007FFFFFu);
        if ((ua & 0x007FFFFFu) == (ub & 0x007FFFFFu))
            return 0;
    }
    if (!na && !nb && fabsf(a) == fabsf(b))
        return 0;
    return sa ? !mag_less : mag_less;
}

/* ----------------------------------------------------------------- reduce */

/*
 * y[r] = combine over j = 0..cols-1 (index order) of x[r*ld + j].
 * [CA] combine_fn: associative add / max / min on 32-bit elements.
 * [RW] the state-carrying reduce folds each element into the monoid state.
 * MAX/MIN start from the row's first element, so a non-empty row always
 * yields one of its own elements; cols == 0 gives the identity (0 for SUM,
 * -inf / INT32_MIN for MAX, +inf / INT32_MAX for MIN).
 */
int rro_reduce_rows(const void* x, void* y, int64_t rows, int64_t cols, int64_t ld,
                    int dtype, int op)
{
    if (rows < 0 || cols < 0 || ld < cols)
        return RRO_BAD;
    if (op != RRO_SUM && op != RRO_MAX && op != RRO_MIN)
        return RRO_BAD;
    for (int64_t r = 0; r < rows; ++r) {
        if (dtype == RRO_I32) {
            const int32_t* row = (const int32_t*)x + r * ld;
            int32_t out;
            if (op == RRO_SUM) {
                uint32_t acc = 0;                   /* wraps modulo 2^32 */
                for (int64_t j = 0; j < cols; ++j)
                    acc += (uint32_t)row[j];
                out = (int32_t)acc;
            } else if (op == RRO_MAX) {
                int32_t acc = cols ? row[0] : INT32_MIN;
                for (int64_t j = 1; j < cols; ++j)
                    if (row[j] > acc)
                        acc = row[j];
                out = acc;
            } else {
                int32_t acc = cols ? row[0] : INT32_MAX;
                for (int64_t j = 1; j < cols; ++j)
                    if (row[j] < acc)
                        acc = row[j];
                out = acc;
            }
            ((int32_t*)y)[r] = out;
        } else if (dtype == RRO_F32) {
            const float* row = (const float*)x + r * ld;
            float out;
            if (op == RRO_SUM) {
                double acc = 0.0;
                for (int64_t j = 0; j < cols; ++j)
                    acc += (double)row[j];
                out = (float)acc;
            } else if (op == RRO_MAX) {
                float acc = cols ? row[0] : -INFINITY;
                for (int64_t j = 1; j < cols; ++j)
                    if (f32_total_before(acc, row[j]))
                        acc = row[j];
                out = acc;
            } else {
                float acc = cols ? row[0] : INFINITY;
                for (int64_t j = 1; j < cols; ++j)
                    if (f32_total_before(row[j], acc))
                        acc = row[j];
                out = acc;
            }
            ((float*)y)[r] = out;
        } else {
            return RRO_BAD;
        }
    }
    return RRO_OK;
}

/* ------------------------------------------------------ non-last axis */

/*
 * [RW] reduce, Args (ctx.axis is the reduce axis; the other dims are pinned)
 * and tier semantics (the tiled tier owns adjacent output rows): the same
 * fold as rro_reduce_rows, along the middle axis of x laid out
 * [outer][axis][inner] (contiguous), into y [outer][inner]:
 *   y[o][i] = fold over a = 0 .. axis-1, in that order, of x[o][a][i].
 * Same arithmetic as rro_reduce_rows; axis == 0 writes the identity.
 */
int rro_reduce_axis(const void* x, void* y, int64_t outer, int64_t axis, int64_t inner,
                    int dtype, int op)
{
    if (outer < 0 || axis < 0 || inner < 0)
        return RRO_BAD;
    if (op != RRO_SUM && op != RRO_MAX && op != RRO_MIN)
        return RRO_BAD;
    if (dtype != RRO_F32 && dtype != RRO_I32)
        return RRO_BAD;
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t i = 0; i < inner; ++i) {
            const int64_t base = o * axis * inner + i;  /* x[o][0][i]; step inner */
            if (dtype == RRO_I32) {
                const int32_t* xs = (const int32_t*)x;
                int32_t out;
                if (op == RRO_SUM) {
                    uint32_t acc = 0;
                    for (int64_t a = 0; a < axis; ++a)
                        acc += (uint32_t)xs[base + a * inner];
                    out = (int32_t)acc;
                } else {
                    int32_t acc = axis ? xs[base] : (op == RRO_MAX ? INT32_MIN : INT32_MAX);
                    for (int64_t a = 1; a < axis; ++a) {
                        const int32_t v = xs[base + a * inner];
                        if (op == RRO_MAX ? v > acc : v < acc)
                            acc = v;
                    }
                    out = acc;
                }
                ((int32_t*)y)[o * inner + i] = out;
            } else {
                const float* xs = (const float*)x;
                float out;
                if (op == RRO_SUM) {
                    double acc = 0.0;
                    for (int64_t a = 0; a < axis; ++a)
                        acc += (double)xs[base + a * inner];
                    out = (float)acc;
                } else {
                    float acc = axis ? xs[base] : (op == RRO_MAX ? -INFINITY : INFINITY);
                    for (int64_t a = 1; a < axis; ++a) {
                        const float v = xs[base + a * inner];
                        if (op == RRO_MAX ? f32_total_before(acc, v) : f32_total_before(v, acc))
                            acc = v;
                    }
                    out = acc;
                }
                ((float*)y)[o * inner + i] = out;
            }
        }
    }
    return RRO_OK;
}

/* ---------------------------------------------------------------- softmax */

/*
 * [RW] two-pass softmax.  Pass 1: m = max_j x_j, s = sum_j exp(x_j - m).
 * Pass 2 (a pure map): y_j = exp(x_j - m) / s, rounded once to y's type.
 * cols == 0 writes nothing.
 */
int rro_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols,
                     int64_t ld_x, int64_t ld_y, int x_dtype, int y_dtype)
{
    if (rows < 0 || cols < 0 || ld_x < cols || ld_y < cols)
        return RRO_BAD;
    if ((x_dtype != RRO_F32 && x_dtype != RRO_BF16) || (y_dtype != RRO_F32 && y_dtype != RRO_BF16))
        return RRO_BAD;
    for (int64_t r = 0; r < rows; ++r) {
        if (cols == 0)
            continue;
        double m = load_real(x, x_dtype, r * ld_x);
        for (int64_t j = 1; j < cols; ++j) {
            double v = load_real(x, x_dtype, r * ld_x + j);
            if (v > m)
                m = v;
        }
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j)
            s += exp(load_real(x, x_dtype, r * ld_x + j) - m);
        for (int64_t j = 0; j < cols; ++j) {
            double e = exp(load_real(x, x_dtype, r * ld_x + j) - m);
            store_real(y, y_dtype, r * ld_y + j, e / s);
        }
    }
    return RRO_OK;
}

/* --------------------------------------------------------------- layernorm */

/*
 * [RW] description: layernorm is one of the two-pass algorithms -- pass 1
 * reduces the row's statistics, pass 2 is a pure map over the row.  The
 * page names it without a formula; this is the standard one:
 *   mean = (sum_j x_j) / n
 *   var  = (sum_j (x_j - mean)^2) / n          (population variance)
 *   rstd = 1 / sqrt(var + eps)
 *   y_j  = (x_j - mean) * rstd * gamma_j + beta_j
 * gamma == NULL means gamma_j = 1, beta == NULL means beta_j = 0; both are
 * [cols] of w_dtype.  mean_out / rstd_out (float [rows], may be NULL)
 * receive mean and rstd rounded once to float.  cols == 0 writes nothing.
 * Everything in double, each output rounded once.
 */
int rro_layernorm_rows(const void* x, void* y, const void* gamma, const void* beta,
                       float* mean_out, float* rstd_out, int64_t rows, int64_t cols,
                       int64_t ld_x, int64_t ld_y, int x_dtype, int y_dtype, int w_dtype,
                       double eps)
{
    if (rows < 0 || cols < 0 || ld_x < cols || ld_y < cols)
        return RRO_BAD;
    if ((x_dtype != RRO_F32 && x_dtype != RRO_BF16) || (y_dtype != RRO_F32 && y_dtype != RRO_BF16) ||
        (w_dtype != RRO_F32 && w_dtype != RRO_BF16))
        return RRO_BAD;
    for (int64_t r = 0; r < rows; ++r) {
        if (cols == 0)
            continue;
        double sum = 0.0;
        for (int64_t j = 0; j < cols; ++j)
            sum += load_real(x, x_dtype, r * ld_x + j);
        const double mean = sum / (double)cols;
        double sq = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            const double d = load_real(x, x_dtype, r * ld_x + j) - mean;
            sq += d * d;
        }
        const double var = sq / (double)cols;
        const double rstd = 1.0 / sqrt(var + eps);
        for (int64_t j = 0; j < cols; ++j) {
            const double g = gamma ? load_real(gamma, w_dtype, j) : 1.0;
            const double b = beta ? load_real(beta, w_dtype, j) : 0.0;
            const double v = (load_real(x, x_dtype, r * ld_x + j) - mean) * rstd * g + b;
            store_real(y, y_dtype, r * ld_y + j, v);
        }
        if (mean_out)
            mean_out[r] = (float)mean;
        if (rstd_out)
            rstd_out[r] = (float)rstd;
    }
    return RRO_OK;
}

/* --------------------------------------------------------------- LSE merge */

/*
 * [FA4] split-K combine of P partition outputs.
 *   o   [P][rows][depth]  normalised partial outputs O_p
 *   m   [P][rows]         per-row max m_p of partition p's scores
 *   l   [P][rows]         per-row sum l_p = sum exp(score - m_p)
 *   out [rows][depth]     f32 or bf16
 * Partition p is empty when l_p <= 0 or m_p == -inf; empty partitions take
 * part but contribute nothing (their O_p is not read into the sum).
 */
int rro_splitk_lse_merge(const float* o, const float* m, const float* l, void* out,
                         int32_t P, int64_t rows, int32_t depth, float scale, int out_dtype)
{
    if (P < 1 || rows < 0 || depth < 1)
        return RRO_BAD;
    if (out_dtype != RRO_F32 && out_dtype != RRO_BF16)
        return RRO_BAD;
    double* w = (double*)malloc(sizeof(double) * (size_t)P);
    int* live = (int*)malloc(sizeof(int) * (size_t)P);
    if (!w || !live) {
        free(w);
        free(live);
        return RRO_BAD;
    }
    for (int64_t r = 0; r < rows; ++r) {
        /* which partitions are non-empty, and the largest of their maxima */
        int any = 0;
        double M = -INFINITY;
        for (int32_t p = 0; p < P; ++p) {
            double mp = (double)m[(int64_t)p * rows + r];
            double lp = (double)l[(int64_t)p * rows + r];
            live[p] = (lp > 0.0 && mp > -INFINITY);
            if (live[p]) {
                if (!any || mp > M)
                    M = mp;
                any = 1;
            }
        }
        /* weights w_p = exp(scale * (m_p - M)) * l_p and their total W */
        double W = 0.0;
        for (int32_t p = 0; p < P; ++p) {
            w[p] = 0.0;
            if (live[p]) {
                double mp = (double)m[(int64_t)p * rows + r];
                double lp = (double)l[(int64_t)p * rows + r];
                w[p] = exp((double)scale * (mp - M)) * lp;
                W += w[p];
            }
        }
        /* out = sum over non-empty p, in ascending p, of (w_p / W) * O_p */
        for (int32_t d = 0; d < depth; ++d) {
            double acc = 0.0;
            for (int32_t p = 0; p < P; ++p)
                if (live[p])
                    acc += (w[p] / W) * (double)o[((int64_t)p * rows + r) * depth + d];
            store_real(out, out_dtype, r * depth + d, acc);
        }
    }
    free(w);
    free(live);
    return RRO_OK;
}

/*
 * Split-K attention partials, the producer side of the LSE merge
 * ("fa4_splitk_reduce_scatter_write", per-band steps: the partial output of
 * each partition carries its own row max and row sum).
 *
 *   q [batch*heads][q_rows][depth]      bf16 bits
 *   k, v [batch*kv_heads][kv_len][depth] bf16 bits
 * Query head h of batch b reads key/value head h / (heads / kv_heads) of
 * batch b (grouped heads; kv_heads == heads is plain multi-head attention).
 * The keys are cut into P contiguous partitions: partition p holds keys
 * j with p*kv_len/P <= j < (p+1)*kv_len/P (integer division).  For query
 * row i and partition p, with s_j = scale * sum_d q[i][d] * k[j][d]:
 *   m_p    = max over the partition's keys of s_j
 *   l_p    = sum over the partition's keys of exp(s_j - m_p)
 *   O_p[d] = sum over the partition's keys of exp(s_j - m_p) * v[j][d] / l_p
 * (normalised partials, as the merge takes them).  A partition with no key
 * gives m_p = -inf, l_p = 0 and O_p = 0.
 *   o [P][batch*heads*q_rows][depth], m, l [P][batch*heads*q_rows]: float,
 *   each rounded once from double.
 */
int rro_attention_partials(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* o,
                           float* m, float* l, int64_t batch, int64_t heads, int64_t kv_heads,
                           int64_t q_rows, int64_t kv_len, int32_t depth, int32_t P, float scale)
{
    if (batch < 0 || heads < 1 || kv_heads < 1 || heads % kv_heads != 0 || q_rows < 0 ||
        kv_len < 0 || depth < 1 || P < 1)
        return RRO_BAD;
    const int64_t group = heads / kv_heads;
    const int64_t rows = batch * heads * q_rows;
    double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)depth);
    if (!s || !acc) {
        free(s);
        free(acc);
        return RRO_BAD;
    }
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t h = 0; h < heads; ++h) {
            const int64_t kvh = b * kv_heads + h / group;
            const uint16_t* kh = k + kvh * kv_len * depth;
            const uint16_t* vh = v + kvh * kv_len * depth;
            for (int64_t i = 0; i < q_rows; ++i) {
                const int64_t row = (b * heads + h) * q_rows + i;
                const uint16_t* qi = q + row * depth;
                /* scores of every key */
                for (int64_t j = 0; j < kv_len; ++j) {
                    double dot = 0.0;
                    for (int32_t d = 0; d < depth; ++d)
                        dot += rro_bf16_to_double(qi[d]) * rro_bf16_to_double(kh[j * depth + d]);
                    s[j] = (double)scale * dot;
                }
                for (int32_t p = 0; p < P; ++p) {
                    const int64_t j0 = (int64_t)p * kv_len / P;
                    const int64_t j1 = ((int64_t)p + 1) * kv_len / P;
                    float* op = o + ((int64_t)p * rows + row) * depth;
                    if (j1 <= j0) {
                        m[(int64_t)p * rows + row] = -INFINITY;
                        l[(int64_t)p * rows + row] = 0.0f;
                        for (int32_t d = 0; d < depth; ++d)
                            op[d] = 0.0f;
                        continue;
                    }
                    double mp = s[j0];
                    for (int64_t j = j0 + 1; j < j1; ++j)
                        if (s[j] > mp)
                            mp = s[j];
                    double lp = 0.0;
                    for (int32_t d = 0; d < depth; ++d)
                        acc[d] = 0.0;
                    for (int64_t j = j0; j < j1; ++j) {
                        const double e = exp(s[j] - mp);
                        lp += e;
                        for (int32_t d = 0; d < depth; ++d)
                            acc[d] += e * rro_bf16_to_double(vh[j * depth + d]);
                    }
                    m[(int64_t)p * rows + row] = (float)mp;
                    l[(int64_t)p * rows + row] = (float)lp;
                    for (int32_t d = 0; d < depth; ++d)
                        op[d] = (float)(acc[d] / lp);
                }
            }
        }
    }
    free(s);
    free(acc);
    return RRO_OK;
}

/*
 * Split-K attention partials of packed variable-length sequences ([FA4], the
 * ragged placement of the combine's output: its Signature places each output
 * tile by a head index and a row index into a ragged [tokens][heads][depth]
 * tensor, with the tile's row count -- num_output_rows -- cut to the
 * sequence).  Sequences are packed along the token axis:
 *   q [total_q][heads][depth], k, v [total_k][kv_heads][depth]  (bf16 bits);
 *   sequence b has queries cu_q[b] .. cu_q[b+1]-1 and keys
 *   cu_k[b] .. cu_k[b+1]-1 (cu_q, cu_k: batch + 1 non-decreasing offsets,
 *   cu[0] >= 0, cu[batch] <= total).
 * Outputs, one partial row per (token t, head h) at t * heads + h:
 *   o [P][total_q][heads][depth], m, l [P][total_q][heads].
 * For each sequence this is rro_attention_partials of that sequence alone: the
 * keys of sequence b are cut into P contiguous partitions of its own keys
 * (p*n_b/P .. (p+1)*n_b/P - 1), with the same arithmetic in the same order;
 * a sequence without keys gives (-inf, 0, 0) in every partition.  Rows of
 * tokens that belong to no sequence are not written.
 */
int rro_attention_partials_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* cu_q, const int32_t* cu_k, float* o, float* m,
                                  float* l, int64_t batch, int64_t heads, int64_t kv_heads,
                                  int64_t total_q, int64_t total_k, int32_t depth, int32_t P,
                                  float scale)
{
    if (batch < 0 || heads < 1 || kv_heads < 1 || heads % kv_heads != 0 || total_q < 0 ||
        total_k < 0 || depth < 1 || P < 1)
        return RRO_BAD;
    if (cu_q[0] < 0 || cu_k[0] < 0 || cu_q[batch] > total_q || cu_k[batch] > total_k)
        return RRO_BAD;
    for (int64_t b = 0; b < batch; ++b)
        if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b])
            return RRO_BAD;
    const int64_t group = heads / kv_heads;
    const int64_t rows = total_q * heads;
    double* s = (double*)malloc(sizeof(double) * (size_t)(total_k > 0 ? total_k : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)depth);
    if (!s || !acc) {
        free(s);
        free(acc);
        return RRO_BAD;
    }
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t n_k = cu_k[b + 1] - cu_k[b];
        for (int64_t h = 0; h < heads; ++h) {
            const int64_t kvh = h / group;
            for (int64_t t = cu_q[b]; t < cu_q[b + 1]; ++t) {
                const int64_t row = t * heads + h;
                const uint16_t* qi = q + row * depth;
                /* scores of every key of the sequence */
                for (int64_t j = 0; j < n_k; ++j) {
                    const uint16_t* kj = k + ((cu_k[b] + j) * kv_heads + kvh) * depth;
                    double dot = 0.0;
                    for (int32_t d = 0; d < depth; ++d)
                        dot += rro_bf16_to_double(qi[d]) * rro_bf16_to_double(kj[d]);
                    s[j] = (double)scale * dot;
                }
                for (int32_t p = 0; p < P; ++p) {
                    const int64_t j0 = (int64_t)p * n_k / P;
                    const int64_t j1 = ((int64_t)p + 1) * n_k / P;
                    float* op = o + ((int64_t)p * rows + row) * depth;
                    if (j1 <= j0) {
                        m[(int64_t)p * rows + row] = -INFINITY;
                        l[(int64_t)p * rows + row] = 0.0f;
                        for (int32_t d = 0; d < depth; ++d)
                            op[d] = 0.0f;
                        continue;
                    }
                    double mp = s[j0];
                    for (int64_t j = j0 + 1; j < j1; ++j)
                        if (s[j] > mp)
                            mp = s[j];
                    double lp = 0.0;
                    for (int32_t d = 0; d < depth; ++d)
                        acc[d] = 0.0;
                    for (int64_t j = j0; j < j1; ++j) {
                        const double e = exp(s[j] - mp);
                        const uint16_t* vj = v + ((cu_k[b] + j) * kv_heads + kvh) * depth;
                        lp += e;
                        for (int32_t d = 0; d < depth; ++d)
                            acc[d] += e * rro_bf16_to_double(vj[d]);
                    }
                    m[(int64_t)p * rows + row] = (float)mp;
                    l[(int64_t)p * rows + row] = (float)lp;
                    for (int32_t d = 0; d < depth; ++d)
                        op[d] = (float)(acc[d] / lp);
                }
            }
        }
    }
    free(s);
    free(acc);
    return RRO_OK;
}
