/*
 * oracle.c -- plain, slow, fp64 CPU oracle of the any-precision MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code, no
 * header and no table with the HIP library; both read the same synthetic bytes.
 *
 * What it computes (PagedWeight: Efficient MoE LLM Serving with Dynamic
 * Quality-Aware Weight Quantization, arXiv:2607.16184):
 *   - Section 2.1 (routing, Eq. 1 context): a router scores E experts per token
 *     and the top K are selected with routing weights.
 *   - Section 3 / Figure 3 caption: weights are Any-Precision overlaid bit-planes;
 *     a b-bit weight uses a subset of the planes, and a per-bitwidth lookup table
 *     holds the centroid values.  Reading used here: P = 8 parent planes, plane 0
 *     holds the most significant code bit, a b-bit block uses planes 0..b-1, and
 *     the LUT is per output row, LUT[b][row][code].
 *   - Section 3.3 ("Fused Mixed-Precision MoE Kernel"): per linear-block bitwidth
 *     for gate_up and down, expert activation, down projection, output
 *     accumulation.  Activation read as SiLU(gate) * up with gate = rows [0,F)
 *     and up = rows [F,2F) of the gate_up block.
 *   - Section 3.1, Eq. 3: M_i^b, the GPU bytes of block i at b bits (planes + LUT).
 *
 * Everything is computed in fp64 with no intermediate rounding.  fp16 inputs are
 * widened exactly.  Child LUT levels are the one place where fp16 rounding is
 * part of the definition: level b is the pairwise mean of the stored fp16 level
 * b+1, rounded to fp16 (round to nearest, ties to even).
 *
 * Parity pins (tests, CPU only): bit-order one-hot probe, code_b == code_8 >> (8-b),
 * pack/unpack round trip, identity LUT == exact integer matmul, constant LUT closed
 * form, brute force on tiny shapes (independent Python), E=1/k=1/q=8 == dense FFN,
 * LUT ordering invariants, permutation invariants, fp16 conversion against numpy,
 * Eq. 3 byte count, activation against scipy's logistic function, combine on a
 * hand-worked dyadic example, as a gather at top-1, and equal to the layer's own
 * accumulation.  Every exported function is pinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* fp16 <-> fp64 (IEEE 754 binary16), written from the format definition.    */
/* ------------------------------------------------------------------------ */

double apo_h2d(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 1024), e - 25);
    return s ? -v : v;
}

/* Round to nearest, ties to even.  nearbyint() honours the default rounding
 * mode, which is round-to-nearest-even. */
uint16_t apo_d2h(double d)
{
    if (isnan(d))
        return 0x7E00;
    uint16_t s = signbit(d) ? 0x8000 : 0;
    double a = fabs(d);
    if (isinf(a))
        return s | 0x7C00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal quantum 2^-24; a carry to 1024 yields the smallest normal */
        double m = nearbyint(a * 16777216.0);
        return s | (uint16_t)m;
    }
    int ex;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;
    double sig = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (sig >= 2048.0) {
        sig = 1024.0;
        E += 1;
    }
    if (E > 15)
        return s | 0x7C00;
    return s | (uint16_t)((E + 15) << 10) | (uint16_t)((int)sig - 1024);
}

void apo_h2d_array(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = apo_h2d(h[i]);
}

void apo_d2h_array(const double *d, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = apo_d2h(d[i]);
}

/* ------------------------------------------------------------------------ */
/* Format: bit-planes and codes                                              */
/* ------------------------------------------------------------------------ */

/* Bit c%32 of word c/32 of plane p, row n.  Plane layout uint32 [8][N][K/32]. */
static inline int plane_bit(const uint32_t *planes, int64_t N, int64_t K, int p, int64_t n, int64_t c)
{
    const uint32_t w = planes[((int64_t)p * N + n) * (K / 32) + (c >> 5)];
    return (int)((w >> (c & 31)) & 1u);
}

/* q-bit code of (n, c): the top q planes, plane 0 the most significant bit. */
static inline int code_q(const uint32_t *planes, int64_t N, int64_t K, int q, int64_t n, int64_t c)
{
    int code = 0;
    for (int p = 0; p < q; ++p)
        code |= plane_bit(planes, N, K, p, n, c) << (q - 1 - p);
    return code;
}

void apo_unpack_codes(const uint32_t *planes, int64_t N, int64_t K, int q, uint8_t *codes)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < K; ++c)
            codes[n * K + c] = (uint8_t)code_q(planes, N, K, q, n, c);
}

/* Inverse for q = 8: plane p holds bit (7-p) of every parent code. */
void apo_pack_planes(const uint8_t *codes8, int64_t N, int64_t K, uint32_t *planes)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int p = 0; p < 8; ++p)
            for (int64_t w = 0; w < K / 32; ++w) {
                uint32_t word = 0;
                for (int j = 0; j < 32; ++j)
                    word |= (uint32_t)((codes8[n * K + 32 * w + j] >> (7 - p)) & 1) << j;
                planes[((int64_t)p * N + n) * (K / 32) + w] = word;
            }
}

/* ------------------------------------------------------------------------ */
/* LUT levels                                                                */
/* ------------------------------------------------------------------------ */

/* Level b (3..8) of every row from the parent level 8 [N][256]:
 * L_b[n][c] = fp16( (L_{b+1}[n][2c] + L_{b+1}[n][2c+1]) / 2 ), iterated from 8. */
void apo_lut_level(const uint16_t *parent, int64_t N, int b, uint16_t *out)
{
#pragma omp parallel
    {
        uint16_t cur[256], nxt[128];
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            memcpy(cur, parent + n * 256, sizeof(cur));
            for (int lv = 7; lv >= b; --lv) {
                for (int c = 0; c < (1 << lv); ++c)
                    nxt[c] = apo_d2h((apo_h2d(cur[2 * c]) + apo_h2d(cur[2 * c + 1])) / 2.0);
                memcpy(cur, nxt, sizeof(uint16_t) << lv);
            }
            memcpy(out + n * ((int64_t)1 << b), cur, sizeof(uint16_t) << b);
        }
    }
}

/* Eq. 3: GPU bytes of an N x K block at b bits = b planes of N*K/8 bytes plus the
 * fp16 LUT level b of N * 2^b entries. */
int64_t apo_block_bytes(int64_t N, int64_t K, int b)
{
    return N * (int64_t)b * K / 8 + N * ((int64_t)1 << b) * 2;
}

/* ------------------------------------------------------------------------ */
/* Route (Section 2.1): logits, top-k, routing weights, expert-grouped order  */
/* ------------------------------------------------------------------------ */

/*
 * z[t][e] = (sum over h ascending of x[t][h] * Wr[e][h]) + bias[e]   (fp64)
 * top-k by z descending, ties to the lower expert index.
 * renormalize != 0: softmax over the k selected logits; else the full softmax
 * over all E logits evaluated at the selected experts.
 * counts[e], offsets[e] (exclusive scan, offsets[E] = T*k); perm lists the
 * assignments a = t*k + j grouped by expert (e ascending), inside an expert by
 * a ascending; inv_perm[perm[r]] = r.
 * absdot[t][e] (optional) = sum |x*Wr| + |bias|, for rounding-error bounds.
 * Shared experts (n_shared >= 0, the "+4" / "+1" experts of the models in Table 1):
 * experts E .. E+n_shared-1 have no router row and are visited by every token.  The
 * pages give no gate for them; they are appended to every token's assignments after
 * the k routed ones, with weight 1 (their outputs add to the routed mixture).  Rows
 * of ids / w then hold kt = k + n_shared entries, and counts / offsets / perm cover
 * the E + n_shared experts.
 */
void apo_route(const uint16_t *x, const uint16_t *wr, const float *bias, int T, int H, int E, int k,
               int n_shared, int renormalize, double *logits, int32_t *ids, double *w64, float *w32,
               int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm, double *absdot)
{
    const int kt = k + n_shared;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double s = 0.0, sa = 0.0;
            for (int h = 0; h < H; ++h) {
                double p = apo_h2d(x[(int64_t)t * H + h]) * apo_h2d(wr[(int64_t)e * H + h]);
                s += p;
                sa += fabs(p);
            }
            if (bias) {
                s += (double)bias[e];
                sa += fabs((double)bias[e]);
            }
            logits[(int64_t)t * E + e] = s;
            if (absdot)
                absdot[(int64_t)t * E + e] = sa;
        }
        const double *z = logits + (int64_t)t * E;
        /* selection: repeatedly take the largest unselected (lowest e on ties) */
        unsigned char taken[1024];
        memset(taken, 0, sizeof(taken));
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || z[e] > z[best])
                    best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * kt + j] = best;
        }
        double zmax = z[ids[(int64_t)t * kt]];
        double den = 0.0;
        if (renormalize) {
            for (int j = 0; j < k; ++j)
                den += exp(z[ids[(int64_t)t * kt + j]] - zmax);
        } else {
            for (int e = 0; e < E; ++e)
                den += exp(z[e] - zmax);
        }
        for (int j = 0; j < k; ++j) {
            double w = exp(z[ids[(int64_t)t * kt + j]] - zmax) / den;
            w64[(int64_t)t * kt + j] = w;
            w32[(int64_t)t * kt + j] = (float)w;
        }
        for (int s = 0; s < n_shared; ++s) {
            ids[(int64_t)t * kt + k + s] = E + s;
            w64[(int64_t)t * kt + k + s] = 1.0;
            w32[(int64_t)t * kt + k + s] = 1.0f;
        }
    }
    const int R = T * kt, Et = E + n_shared;
    for (int e = 0; e < Et; ++e)
        counts[e] = 0;
    for (int a = 0; a < R; ++a)
        counts[ids[a]]++;
    offsets[0] = 0;
    for (int e = 0; e < Et; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int r = 0;
    for (int e = 0; e < Et; ++e)
        for (int a = 0; a < R; ++a)
            if (ids[a] == e)
                perm[r++] = a;
    for (r = 0; r < R; ++r)
        inv_perm[perm[r]] = r;
}

/* ------------------------------------------------------------------------ */
/* Any-precision block product                                               */
/* ------------------------------------------------------------------------ */

/* W[n][c] = LUT_q[n][code_q(n, c)]  (one row, fp64) */
static void dequant_row(const uint32_t *planes, const uint16_t *lut_q, int q, int64_t N, int64_t K, int64_t n,
                        double *row)
{
    const uint16_t *L = lut_q + n * ((int64_t)1 << q);
    for (int64_t c = 0; c < K; ++c)
        row[c] = apo_h2d(L[code_q(planes, N, K, q, n, c)]);
}

/* out[m][n] = sum_c in[m][c] * W[n][c] for m < M, n < N (fp64). */
void apo_block_gemm(const uint32_t *planes, const uint16_t *lut_q, int q, int64_t N, int64_t K, const double *in,
                    int64_t M, double *out)
{
#pragma omp parallel
    {
        double *row = (double *)malloc(sizeof(double) * K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            dequant_row(planes, lut_q, q, N, K, n, row);
            for (int64_t m = 0; m < M; ++m) {
                double s = 0.0;
                const double *a = in + m * K;
                for (int64_t c = 0; c < K; ++c)
                    s += a[c] * row[c];
                out[m * N + n] = s;
            }
        }
        free(row);
    }
}

/* a[m][f] = SiLU(h[m][f]) * h[m][F + f], SiLU(z) = z / (1 + e^{-z}). */
void apo_act(const double *h, int64_t M, int64_t F, double *a)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t f = 0; f < F; ++f) {
            double g = h[m * 2 * F + f], u = h[m * 2 * F + F + f];
            a[m * F + f] = g / (1.0 + exp(-g)) * u;
        }
}

/* out[t][n] = sum_j w[t][j] * y[inv_perm[t*k + j]][n], summed in j order. */
void apo_combine(const double *y, const double *w, const int32_t *inv_perm, int T, int k, int64_t H, double *out)
{
    for (int t = 0; t < T; ++t)
        for (int64_t n = 0; n < H; ++n) {
            double s = 0.0;
            for (int j = 0; j < k; ++j)
                s += w[t * k + j] * y[(int64_t)inv_perm[t * k + j] * H + n];
            out[(int64_t)t * H + n] = s;
        }
}

/* ------------------------------------------------------------------------ */
/* Whole layer                                                               */
/* ------------------------------------------------------------------------ */

/*
 * One MoE layer forward in fp64.
 *   planes_gu[e] : uint32 [8][2F][H/32]     lutp_gu[e] : fp16 [2F][256] (parent)
 *   planes_dn[e] : uint32 [8][H][F/32]      lutp_dn[e] : fp16 [H][256]
 *   q_gu[e], q_dn[e] : committed bitwidths (3..8)
 * Only assignments of tokens listed in eval_tokens (n_eval of them, NULL = all)
 * are carried through the experts; out is [n_eval][H].  Route outputs are for all
 * T tokens.  If h_out / a_out / y_out are non-NULL (all tokens only) they receive
 * the intermediates in expert-grouped row order: [T*kt][2F], [T*kt][F], [T*kt][H].
 * E routed experts (router rows) plus n_shared shared experts (see apo_route); the
 * plane / LUT / q arrays cover all E + n_shared experts, kt = k + n_shared.
 */
int apo_moe_forward(const uint16_t *x, const uint16_t *wr, const float *bias, int T, int H, int F, int E, int k,
                    int n_shared, int renormalize, const uint32_t *const *planes_gu, const uint16_t *const *lutp_gu,
                    const int32_t *q_gu, const uint32_t *const *planes_dn, const uint16_t *const *lutp_dn,
                    const int32_t *q_dn, const int32_t *eval_tokens, int n_eval, int32_t *ids, double *w64,
                    float *w32, int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm, double *logits,
                    double *out, double *h_out, double *a_out, double *y_out)
{
    const int kt = k + n_shared, Et = E + n_shared;
    const int R = T * kt;
    apo_route(x, wr, bias, T, H, E, k, n_shared, renormalize, logits, ids, w64, w32, counts, offsets, perm, inv_perm,
              NULL);

    unsigned char *want = (unsigned char *)calloc((size_t)T, 1);
    if (!want)
        return 1;
    if (eval_tokens) {
        for (int i = 0; i < n_eval; ++i)
            want[eval_tokens[i]] = 1;
    } else {
        n_eval = T;
        memset(want, 1, (size_t)T);
    }
    /* y for every needed expert row, indexed by its grouped row r */
    double *y = (double *)calloc((size_t)R * H, sizeof(double));
    if (!y) {
        free(want);
        return 1;
    }
    for (int e = 0; e < Et; ++e) {
        /* rows of expert e whose token is evaluated */
        int M = 0;
        int *rows = (int *)malloc(sizeof(int) * (size_t)(counts[e] + 1));
        for (int r = offsets[e]; r < offsets[e + 1]; ++r)
            if (want[perm[r] / kt])
                rows[M++] = r;
        if (M == 0) {
            free(rows);
            continue;
        }
        const int qg = q_gu[e], qd = q_dn[e];
        uint16_t *lut_g = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)2 * F * ((size_t)1 << qg));
        uint16_t *lut_d = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)H * ((size_t)1 << qd));
        apo_lut_level(lutp_gu[e], 2 * (int64_t)F, qg, lut_g);
        apo_lut_level(lutp_dn[e], H, qd, lut_d);

        double *xin = (double *)malloc(sizeof(double) * (size_t)M * H);
        for (int m = 0; m < M; ++m) {
            const int t = perm[rows[m]] / kt;
            for (int c = 0; c < H; ++c)
                xin[(size_t)m * H + c] = apo_h2d(x[(int64_t)t * H + c]);
        }
        double *h = (double *)malloc(sizeof(double) * (size_t)M * 2 * F);
        apo_block_gemm(planes_gu[e], lut_g, qg, 2 * (int64_t)F, H, xin, M, h);
        double *a = (double *)malloc(sizeof(double) * (size_t)M * F);
        apo_act(h, M, F, a);
        double *ye = (double *)malloc(sizeof(double) * (size_t)M * H);
        apo_block_gemm(planes_dn[e], lut_d, qd, H, F, a, M, ye);
        for (int m = 0; m < M; ++m) {
            memcpy(y + (size_t)rows[m] * H, ye + (size_t)m * H, sizeof(double) * H);
            if (h_out)
                memcpy(h_out + (size_t)rows[m] * 2 * F, h + (size_t)m * 2 * F, sizeof(double) * 2 * F);
            if (a_out)
                memcpy(a_out + (size_t)rows[m] * F, a + (size_t)m * F, sizeof(double) * F);
            if (y_out)
                memcpy(y_out + (size_t)rows[m] * H, ye + (size_t)m * H, sizeof(double) * H);
        }
        free(ye);
        free(a);
        free(h);
        free(xin);
        free(lut_d);
        free(lut_g);
        free(rows);
    }
    /* combine for the evaluated tokens, in the order given */
    for (int n_i = 0; n_i < n_eval; ++n_i) {
        const int t = eval_tokens ? eval_tokens[n_i] : n_i;
        for (int n = 0; n < H; ++n) {
            double s = 0.0;
            for (int j = 0; j < kt; ++j)
                s += w64[t * kt + j] * y[(size_t)inv_perm[t * kt + j] * H + n];
            out[(size_t)n_i * H + n] = s;
        }
    }
    free(y);
    free(want);
    return 0;
}

int apo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void apo_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
