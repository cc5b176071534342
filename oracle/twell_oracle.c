/*
 * twell_oracle.c -- plain CPU oracle for the ReLU-sparse gated FFN and its
 * TwELL (tile-wise ELLPACK) encoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or table with the HIP library.
 *
 * What it follows ("Sparser, Faster, Lighter Transformer Language Models",
 * gist.science summary page):
 *   - section 2.1 (TwELL): the columns of the gate activation are cut into
 *     horizontal tiles of width w; inside each tile the nonzeros of a row are
 *     packed with tile-local indices.  The gate activation is ReLU(x.W_g).
 *   - section 2.2 (fused inference): the FFN is up projection x.W_u, gate
 *     activation of x.W_g and down projection h.W_d; the fused kernel, for each
 *     nonzero gate value, reads the matching W_u column and W_d row, takes one
 *     dot product and one scalar product, and accumulates.
 *   - section 2.3 (hybrid format): rows with too many nonzeros go to a dense
 *     backup matrix, the rest stay in the compact ELL part.
 * Readings where the page is silent (all stated in the design notes):
 *   - a gate value is active iff z > 0 strictly (0, -0 and NaN are inactive);
 *   - inside a tile, entries are kept in ascending column order; when a tile
 *     holds more than `cap` actives, the `cap` lowest columns are kept and the
 *     TRUE count is stored;
 *   - a row is an overflow row iff any of its tiles holds more than `cap`;
 *   - stored values are the activation rounded to the storage type: fp32 by
 *     round-to-nearest-even from the fp64 value, bf16 by round-to-nearest-even
 *     of that fp32 value;
 *   - the gate multiplies the up projection: h = ReLU(z) * u.
 *
 * Arithmetic: fp64 throughout, plain loops in the order of the definitions
 * (ascending k for dot products, ascending neuron j for the output sum).
 * Build: gcc -O3 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC (no
 * contraction or reassociation, so the flags do not change any result).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* Round-to-nearest-even of an fp32 value to bfloat16 (kept in an fp32). */
static float orc_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) /* inf and NaN pass through */
        return f;
    uint32_t keep_lsb = (u >> 16) & 1u;   /* tie goes to the even upper half */
    u += 0x7FFFu + keep_lsb;
    u &= 0xFFFF0000u;
    memcpy(&f, &u, 4);
    return f;
}

/* Value as stored in a TwELL / dense-backup array of type vdtype
 * (-1: exact fp64, 0: fp32, 1: bf16). */
static double orc_store(double v, int vdtype)
{
    if (vdtype < 0)
        return v;
    float f = (float)v; /* C's double -> float conversion rounds to nearest even */
    if (vdtype == 1)
        f = orc_bf16_rne(f);
    return (double)f;
}

/* Threads of the OpenMP loops below (timing only; results do not depend on it). */
EXPORT void orc_set_threads(int n) { omp_set_num_threads(n); }
EXPORT int orc_max_threads(void) { return omp_get_max_threads(); }

EXPORT void orc_round_array(const double *in, int64_t n, int vdtype, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_store(in[i], vdtype);
}

/* out[r][j] = sum_k a[rows[r]][k] * b[j][k]  (fp64, ascending k).
 * a: [*][k] row-major, b: [n][k] row-major (e.g. W_g^T), out: [n_rows][n]. */
EXPORT void orc_matmul_nt_rows(const float *a, const int32_t *rows, int n_rows,
                               const float *b, int n, int k, double *out)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n_rows; ++r) {
        const float *ar = a + (int64_t)rows[r] * k;
        for (int j = 0; j < n; ++j) {
            const float *bj = b + (int64_t)j * k;
            double s = 0.0;
            for (int kk = 0; kk < k; ++kk)
                s += (double)ar[kk] * (double)bj[kk];
            out[(int64_t)r * n + j] = s;
        }
    }
}

/* TwELL packer (section 2.1).  z: [T][F] pre-activations.
 * cnt: [T][F/w] true active count per (row, tile);
 * val: [T][F/w][cap] stored values of the kept actives, 0 in unused slots;
 * idx: [T][F/w][cap] tile-local column of each kept active, 0 in unused slots. */
EXPORT void orc_pack_twell(const double *z, int T, int F, int w, int cap, int vdtype,
                           int32_t *cnt, double *val, uint8_t *idx)
{
    const int n_b = F / w;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int b = 0; b < n_b; ++b) {
            int64_t slot0 = ((int64_t)t * n_b + b) * cap;
            for (int s = 0; s < cap; ++s) {
                val[slot0 + s] = 0.0;
                idx[slot0 + s] = 0;
            }
            int k = 0;
            for (int c = 0; c < w; ++c) {
                double v = z[(int64_t)t * F + (int64_t)b * w + c];
                if (v > 0.0) {
                    if (k < cap) {
                        val[slot0 + k] = orc_store(v, vdtype);
                        idx[slot0 + k] = (uint8_t)c;
                    }
                    ++k;
                }
            }
            cnt[(int64_t)t * n_b + b] = k;
        }
    }
}

/* Hybrid partition (section 2.3): row_ovf[t] = 1 iff some tile count > cap;
 * ovf_rows = the overflow rows in ascending order.  Returns their number. */
EXPORT int orc_partition(const int32_t *cnt, int T, int n_b, int cap,
                         int32_t *row_ovf, int32_t *ovf_rows)
{
    int n = 0;
    for (int t = 0; t < T; ++t) {
        int f = 0;
        for (int b = 0; b < n_b; ++b)
            if (cnt[(int64_t)t * n_b + b] > cap)
                f = 1;
        row_ovf[t] = f;
        if (f)
            ovf_rows[n++] = t;
    }
    return n;
}

/* Dense FFN (section 2.2), every neuron:  y[t] = sum_j h[t][j] * u[t][j] * W_d[j],
 * h = max(z, 0) (stored-rounded when hround >= 0), ascending j. */
EXPORT void orc_ffn_dense(const double *z, const double *u, const float *wd,
                          int T, int F, int d, int hround, double *y)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double *yt = y + (int64_t)t * d;
        for (int k = 0; k < d; ++k)
            yt[k] = 0.0;
        for (int j = 0; j < F; ++j) {
            double zz = z[(int64_t)t * F + j];
            double h = zz > 0.0 ? orc_store(zz, hround) : 0.0;
            double s = h * u[(int64_t)t * F + j];
            const float *wdj = wd + (int64_t)j * d;
            for (int k = 0; k < d; ++k)
                yt[k] += s * (double)wdj[k];
        }
    }
}

static double orc_dot(const float *a, const float *b, int d)
{
    double s = 0.0;
    for (int k = 0; k < d; ++k)
        s += (double)a[k] * (double)b[k];
    return s;
}

/* Fused up/down step from a TwELL (section 2.2): for each kept entry, in
 * ascending tile then slot order (ascending neuron j):
 *   j = b*w + idx;  u = x[t] . W_u^T[j];  y[t] += (val * u) * W_d[j].
 * skip_overflow != 0: rows with any tile count > cap get y[t] = 0. */
EXPORT void orc_ffn_twell(const int32_t *cnt, const double *val, const uint8_t *idx,
                          int T, int F, int w, int cap,
                          const float *x, const float *wu_t, const float *wd, int d,
                          int skip_overflow, double *y)
{
    const int n_b = F / w;
#pragma omp parallel for schedule(dynamic, 16)
    for (int t = 0; t < T; ++t) {
        double *yt = y + (int64_t)t * d;
        for (int k = 0; k < d; ++k)
            yt[k] = 0.0;
        int ovf = 0;
        for (int b = 0; b < n_b; ++b)
            if (cnt[(int64_t)t * n_b + b] > cap)
                ovf = 1;
        if (ovf && skip_overflow)
            continue;
        const float *xt = x + (int64_t)t * d;
        for (int b = 0; b < n_b; ++b) {
            int c = cnt[(int64_t)t * n_b + b];
            int m = c < cap ? c : cap;
            for (int s = 0; s < m; ++s) {
                int64_t slot = ((int64_t)t * n_b + b) * cap + s;
                int j = b * w + idx[slot];
                double uj = orc_dot(xt, wu_t + (int64_t)j * d, d);
                double sc = val[slot] * uj;
                const float *wdj = wd + (int64_t)j * d;
                for (int k = 0; k < d; ++k)
                    yt[k] += sc * (double)wdj[k];
            }
        }
    }
}

/* The same fused sum taken over EVERY active neuron of each row, straight
 * from z (no capacity): what the hybrid path must produce for every row.
 * h = z (exact) or its stored rounding (hround >= 0). */
EXPORT void orc_ffn_active(const double *z, int T, int F,
                           const float *x, const float *wu_t, const float *wd, int d,
                           int hround, double *y)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int t = 0; t < T; ++t) {
        double *yt = y + (int64_t)t * d;
        for (int k = 0; k < d; ++k)
            yt[k] = 0.0;
        const float *xt = x + (int64_t)t * d;
        for (int j = 0; j < F; ++j) {
            double zz = z[(int64_t)t * F + j];
            if (!(zz > 0.0))
                continue;
            double h = orc_store(zz, hround);
            double uj = orc_dot(xt, wu_t + (int64_t)j * d, d);
            double sc = h * uj;
            const float *wdj = wd + (int64_t)j * d;
            for (int k = 0; k < d; ++k)
                yt[k] += sc * (double)wdj[k];
        }
    }
}

/* Activation statistics of the gate (the page's L1 activation penalty, section
 * 2.4, and its dead neurons): neuron_cnt[j] = number of rows t with z[t][j] > 0;
 * l1[t][b] = sum over the active columns j of tile b of row t of z[t][j]
 * (the gate activation before rounding; ascending columns, fp64). */
EXPORT void orc_gate_stats(const double *z, int T, int F, int w, int64_t *neuron_cnt, double *l1)
{
    const int n_b = F / w;
    for (int j = 0; j < F; ++j)
        neuron_cnt[j] = 0;
    for (int t = 0; t < T; ++t) {
        for (int b = 0; b < n_b; ++b) {
            double s = 0.0;
            for (int c = 0; c < w; ++c) {
                const int j = b * w + c;
                const double zz = z[(int64_t)t * F + j];
                if (zz > 0.0) {
                    s += zz;
                    neuron_cnt[j] += 1;
                }
            }
            l1[(int64_t)t * n_b + b] = s;
        }
    }
}

/* Backward of the FFN above (the page's training kernels, section 2.4, need
 * the gradients of y = sum over active j of h_j (x.W_u^T[j]) W_d[j]).  With
 * dy [T][d] given, per row t and active neuron j (z > 0, ascending j), h the
 * stored gate value (ReLU(z) rounded as hround says, derivative 1 where active):
 *   u = x_t . W_u^T[j],  g = dy_t . W_d[j],  du = g h,  dz = g u,
 *   dx_t += du W_u^T[j] + dz W_g^T[j],  dW_d[j] += (h u) dy_t,
 *   dW_u^T[j] += du x_t,  dW_g^T[j] += dz x_t.
 * All outputs fp64 and overwritten; rows (t) and neurons (j) in ascending order. */
EXPORT void orc_ffn_backward(const double *z, int T, int F, const float *x, const float *wg_t, const float *wu_t,
                             const float *wd, int d, int hround, const double *dy, double *dx, double *dwg,
                             double *dwu, double *dwd)
{
    for (int64_t i = 0; i < (int64_t)T * d; ++i)
        dx[i] = 0.0;
    for (int64_t i = 0; i < (int64_t)F * d; ++i)
        dwg[i] = dwu[i] = dwd[i] = 0.0;
    for (int t = 0; t < T; ++t) {
        const float *xt = x + (int64_t)t * d;
        const double *dyt = dy + (int64_t)t * d;
        double *dxt = dx + (int64_t)t * d;
        for (int j = 0; j < F; ++j) {
            const double zz = z[(int64_t)t * F + j];
            if (!(zz > 0.0))
                continue;
            const double h = orc_store(zz, hround);
            const float *wuj = wu_t + (int64_t)j * d;
            const float *wgj = wg_t + (int64_t)j * d;
            const float *wdj = wd + (int64_t)j * d;
            const double u = orc_dot(xt, wuj, d);
            double g = 0.0;
            for (int k = 0; k < d; ++k)
                g += dyt[k] * (double)wdj[k];
            const double du = g * h, dz = g * u, hu = h * u;
            for (int k = 0; k < d; ++k) {
                dxt[k] += du * (double)wuj[k] + dz * (double)wgj[k];
                dwd[(int64_t)j * d + k] += hu * dyt[k];
                dwu[(int64_t)j * d + k] += du * (double)xt[k];
                dwg[(int64_t)j * d + k] += dz * (double)xt[k];
            }
        }
    }
}
