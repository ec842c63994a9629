/*
 * CPU oracle for the W4A16 routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or table with the HIP library.
 *
 * Plain, slow, obviously correct.  Floating point is fp64 except where the
 * layer fixes a narrower type:
 *   - FP16 activations into every W4A16 product, so the SwiGLU output h that
 *     feeds the down projection and the layer output y are rounded to FP16
 *     ("Horizon RunMap - architecture", table "Representation and
 *     computation", row "Activation precision"; page "horizonrunmap.com/en",
 *     section "08 / Precision & quality", paragraph "Compute": FP16
 *     activations, FP32 accumulation stages and explicit rounding);
 *   - router logits are FP32 values: the correctly rounded FP32 value of the
 *     exact dot product, so every summation order selects the same experts.
 *     The pages do not say how routing is computed (same section,
 *     "Other components": routing stays outside INT4, FP16 non-routed
 *     weights); this reading is what makes bit-exact expert selection a
 *     well-defined target.
 *
 * Weight format: INT4 codes in 256-value blocks with one FP16 scale per block
 * ("Representation and computation", row "Routed expert source"), value =
 * (code - 8) * scale (the pages fix no zero point; codes 0..15 stand for
 * -8..7).  qpacked v1 layout of a matrix with R rows (outputs) and K columns
 * (reduction), R % 16 == 0, K % 128 == 0:
 *   nibbles: 1024-byte tiles, tile (rg, kt) = rows 16rg..16rg+15 x columns
 *     128kt..128kt+127 at byte (rg*(K/128) + kt)*1024; inside it the 16-byte
 *     chunk 16g + r holds row 16rg + r, columns 128kt + 32g .. +31, byte i
 *     holding column 2i in its low nibble and 2i+1 in its high nibble;
 *   scales: FP16, row 16rg + r, block b (columns 256b .. 256b+255, the last
 *     block may be shorter) at element (rg*ceil(K/256) + b)*16 + r.
 * One expert row = gate nibbles, up nibbles, down nibbles, gate scales, up
 * scales, down scales, each section starting on a 256-byte boundary; gate and
 * up are [I][H], down is [H][I].  The oracle locates each weight by plain
 * address arithmetic, one element at a time.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BLOCK 256

/* ------------------------------------------------------------------ FP16 */

/* IEEE binary16 -> double (exact). */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero or subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);    /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

/* double -> IEEE binary16, round to nearest, ties to even. */
uint16_t oracle_double_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7e00;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = m * 2^-24, m in [0, 1024]; m = 1024 is the
         * smallest normal and has the encoding 0x0400. */
        double m = nearbyint(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)m);
    }
    int ex;
    frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
    double m = nearbyint(ldexp(a, 10 - e));   /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e > 15) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024));
}

/* ----------------------------------------------------------- qpacked read */

/* One INT4 weight of a qpacked v1 matrix with R rows and K columns:
 * (code - 8) * scale, exact in double. */
double oracle_weight(const uint8_t *nib, const uint16_t *scales, int R, int K, int row, int col)
{
    (void)R;
    int rg = row / 16, r = row % 16;
    int kt = col / 128, g = (col % 128) / 32, kk = col % 32;
    size_t tile = (size_t)rg * (K / 128) + kt;
    size_t byte = tile * 1024 + (size_t)(16 * g + r) * 16 + kk / 2;
    int code = (kk % 2 == 0) ? (nib[byte] & 0xf) : (nib[byte] >> 4);
    int nb = (K + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    int b = col / ORACLE_BLOCK;
    double s = oracle_half_to_double(scales[((size_t)rg * nb + b) * 16 + r]);
    return (double)(code - 8) * s;
}

/* Whole matrix, row-major double [R][K]. */
void oracle_dequant_matrix(const uint8_t *nib, const uint16_t *scales, int R, int K, double *out)
{
    for (int r = 0; r < R; ++r)
        for (int c = 0; c < K; ++c)
            out[(size_t)r * K + c] = oracle_weight(nib, scales, R, K, r, c);
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

/* Section offsets of one expert row: gate_q, up_q, down_q, gate_s, up_s, down_s. */
void oracle_row_offsets(int H, int I, size_t off[6], size_t *row_bytes)
{
    size_t nbH = (size_t)(H + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    size_t nbI = (size_t)(I + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    size_t sz[6] = {(size_t)I * H / 2, (size_t)I * H / 2, (size_t)H * I / 2,
                    (size_t)I * nbH * 2, (size_t)I * nbH * 2, (size_t)H * nbI * 2};
    size_t o = 0;
    for (int i = 0; i < 6; ++i) { off[i] = o; o = align256(o + sz[i]); }
    *row_bytes = o;
}

/* ----------------------------------------------------------- router (A1) */

/* Correctly rounded FP32 value of v * 2^-48 for an exact integer v. */
static float rn32_fixed48(__int128 v)
{
    if (v == 0) return 0.0f;
    int neg = v < 0;
    unsigned __int128 a = neg ? (unsigned __int128)(-v) : (unsigned __int128)v;
    int L = 0;
    for (unsigned __int128 t = a; t; t >>= 1) ++L;     /* bit length */
    float res;
    if (L <= 24) {
        res = ldexpf((float)(uint32_t)a, -48);
    } else {
        int sh = L - 24;
        unsigned __int128 mant = a >> sh;
        unsigned __int128 rem = a - (mant << sh);
        unsigned __int128 half = (unsigned __int128)1 << (sh - 1);
        if (rem > half || (rem == half && (mant & 1))) mant += 1;   /* ties to even */
        res = ldexpf((float)(uint32_t)mant, sh - 48);
    }
    return neg ? -res : res;
}

/* Exact FP16 x FP16 dot product, returned as its correctly rounded FP32 value.
 * Every FP16 value is m * 2^q with integer |m| < 2^11 and q >= -24, so each
 * product is an integer multiple of 2^-48; the sum is accumulated exactly as
 * an integer count of 2^-48 units (|sum| < 2^91 fits a 128-bit integer). */
float oracle_exact_dot_rn32(const uint16_t *a, const uint16_t *b, int n, int b_stride)
{
    __int128 acc = 0;
    for (int i = 0; i < n; ++i) {
        uint16_t ha = a[i], hb = b[(size_t)i * b_stride];
        int ea = (ha >> 10) & 0x1f, eb = (hb >> 10) & 0x1f;
        long ma = (ha & 0x3ff) | (ea ? 0x400 : 0);
        long mb = (hb & 0x3ff) | (eb ? 0x400 : 0);
        int qa = (ea ? ea : 1) - 25, qb = (eb ? eb : 1) - 25;   /* value = m * 2^q */
        __int128 p = (__int128)(ma * mb) << (qa + qb + 48);
        if (((ha ^ hb) >> 15) & 1) acc -= p; else acc += p;
    }
    return rn32_fixed48(acc);
}

/* logits[t][e] = RN32(exact sum_h x[t][h] * wr[h][e]) (+ bias[e] as one FP32 add).
 * x: FP16 [T][H]; wr: FP16 [H][E]; bias: FP32 [E] or NULL. */
void oracle_router_logits(const uint16_t *x, const uint16_t *wr, const float *bias,
                          int T, int H, int E, float *logits)
{
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            float l = oracle_exact_dot_rn32(x + (size_t)t * H, wr + e, H, E);
            if (bias) l = l + bias[e];
            logits[(size_t)t * E + e] = l;
        }
}

/* ------------------------------------------------------ top-k, softmax (A2) */

/* ids[t][j]: the k largest logits of token t in descending order, ties to the
 * lower expert index.  w[t][j]: softmax over the k selected logits, fp64. */
void oracle_topk_softmax(const float *logits, int T, int E, int k, int32_t *ids, double *w)
{
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;   /* strict: lower index wins ties */
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        double top = (double)l[ids[(size_t)t * k]];
        double den = 0.0;
        for (int j = 0; j < k; ++j) den += exp((double)l[ids[(size_t)t * k + j]] - top);
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] = exp((double)l[ids[(size_t)t * k + j]] - top) / den;
    }
    free(taken);
}

/* ----------------------------------------------------------- grouping (A3) */

/* Stable counting sort of the T*k (token, slot) pairs by expert.  Pair index
 * p = t*k + j.  offsets[E+1] is the exclusive scan of the counts;
 * sorted_pairs[pos] = p with pairs of one expert in ascending p;
 * pair_pos[p] = pos; active[0..n_active) = experts with a non-zero count,
 * ascending. */
void oracle_group(const int32_t *ids, int T, int E, int k, int32_t *offsets,
                  int32_t *sorted_pairs, int32_t *pair_pos, int32_t *active, int32_t *n_active)
{
    int n = T * k;
    int32_t *fill = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
    for (int e = 0; e <= E; ++e) offsets[e] = 0;
    for (int p = 0; p < n; ++p) offsets[ids[p] + 1] += 1;
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (int p = 0; p < n; ++p) {
        int e = ids[p];
        int pos = offsets[e] + fill[e]++;
        sorted_pairs[pos] = p;
        pair_pos[p] = pos;
    }
    int na = 0;
    for (int e = 0; e < E; ++e)
        if (offsets[e + 1] > offsets[e]) active[na++] = e;
    *n_active = na;
    free(fill);
}

/* ------------------------------------------------- expert FFN (A6, A7) */

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* SwiGLU expert on one FP16 token:
 *   g = Wg x, u = Wu x (fp64),  h = fp16(silu(g) * u),  o = Wd h (fp64).
 * W are dense double matrices already read from the qpacked row
 * (Wg, Wu: [I][H]; Wd: [H][I]).  h_out: FP16 bits [I]; o_out: double [H]. */
void oracle_swiglu_dense(const double *Wg, const double *Wu, const double *Wd, int H, int I,
                         const uint16_t *x, uint16_t *h_out, double *o_out)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *hd = (double *)malloc(sizeof(double) * (size_t)I);
    for (int c = 0; c < H; ++c) xd[c] = oracle_half_to_double(x[c]);
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) {
            g += Wg[(size_t)i * H + c] * xd[c];
            u += Wu[(size_t)i * H + c] * xd[c];
        }
        uint16_t h = oracle_double_to_half(silu(g) * u);
        h_out[i] = h;
        hd[i] = oracle_half_to_double(h);
    }
    for (int r = 0; r < H; ++r) {
        double o = 0.0;
        for (int i = 0; i < I; ++i) o += Wd[(size_t)r * I + i] * hd[i];
        o_out[r] = o;
    }
    free(xd);
    free(hd);
}

/* Read the three matrices of one qpacked expert row into dense doubles. */
void oracle_dequant_expert(const uint8_t *row, int H, int I, double *Wg, double *Wu, double *Wd)
{
    size_t off[6], rb;
    oracle_row_offsets(H, I, off, &rb);
    oracle_dequant_matrix(row + off[0], (const uint16_t *)(row + off[3]), I, H, Wg);
    oracle_dequant_matrix(row + off[1], (const uint16_t *)(row + off[4]), I, H, Wu);
    oracle_dequant_matrix(row + off[2], (const uint16_t *)(row + off[5]), H, I, Wd);
}

/* The offload-qpacked profile ("Horizon RunMap - architecture", section
 * "Historical contracts remain distinct"; "Horizon technical notes —
 * publication edition v1", section "Precision is profile-specific"): the
 * low-bit source is dequantized into FP16 execution slots, so every weight is
 * the FP16 value nearest (code - 8) * scale.  Same matrices as
 * oracle_dequant_expert, each weight rounded to FP16. */
void oracle_dequant_expert_fp16(const uint8_t *row, int H, int I, double *Wg, double *Wu, double *Wd)
{
    oracle_dequant_expert(row, H, I, Wg, Wu, Wd);
    size_t n = (size_t)I * H;
    for (size_t i = 0; i < n; ++i) {
        Wg[i] = oracle_half_to_double(oracle_double_to_half(Wg[i]));
        Wu[i] = oracle_half_to_double(oracle_double_to_half(Wu[i]));
        Wd[i] = oracle_half_to_double(oracle_double_to_half(Wd[i]));
    }
}

/* ------------------------------------------------ FP16 shared expert (A8) */

/* Shared expert with FP16 weights, same rounding points as a routed expert:
 *   os = Wsd fp16(silu(Wsg x) * (Wsu x)),  sigma = 1 / (1 + exp(-(wgate . x))).
 * Wsg, Wsu: FP16 [Is][H]; Wsd: FP16 [H][Is]; wgate: FP16 [H]. */
void oracle_shared_ffn(const uint16_t *x, const uint16_t *Wsg, const uint16_t *Wsu,
                       const uint16_t *Wsd, const uint16_t *wgate, int T, int H, int Is,
                       double *os, double *sigma)
{
    double *hd = (double *)malloc(sizeof(double) * (size_t)Is);
    for (int t = 0; t < T; ++t) {
        const uint16_t *xt = x + (size_t)t * H;
        for (int i = 0; i < Is; ++i) {
            double g = 0.0, u = 0.0;
            for (int c = 0; c < H; ++c) {
                double xc = oracle_half_to_double(xt[c]);
                g += oracle_half_to_double(Wsg[(size_t)i * H + c]) * xc;
                u += oracle_half_to_double(Wsu[(size_t)i * H + c]) * xc;
            }
            hd[i] = oracle_half_to_double(oracle_double_to_half(silu(g) * u));
        }
        for (int r = 0; r < H; ++r) {
            double o = 0.0;
            for (int i = 0; i < Is; ++i) o += oracle_half_to_double(Wsd[(size_t)r * Is + i]) * hd[i];
            os[(size_t)t * H + r] = o;
        }
        double z = 0.0;
        for (int c = 0; c < H; ++c) z += oracle_half_to_double(wgate[c]) * oracle_half_to_double(xt[c]);
        sigma[t] = 1.0 / (1.0 + exp(-z));
    }
    free(hd);
}

/* ----------------------------------------------------------- combine (A9) */

/* y[t] = fp16( sum_j w[t][j] * o[pair (t,j)] (+ sigma[t] * os[t]) ), fp64 sum in j order.
 * o: double [T*k][H] indexed by pair p = t*k + j. */
void oracle_combine(const double *o, const double *w, const double *os, const double *sigma,
                    int T, int H, int k, uint16_t *y)
{
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += w[(size_t)t * k + j] * o[((size_t)t * k + j) * H + c];
            if (os) acc += sigma[t] * os[(size_t)t * H + c];
            y[(size_t)t * H + c] = oracle_double_to_half(acc);
        }
}

/* ------------------------------------------------------------ whole layer */

/* The routed-expert layer on T tokens:
 *   route (A1, A2) -> group (A3) -> per expert, per routed token: SwiGLU from
 *   the expert's qpacked row (A6, A7) -> weighted combine (A9).
 * rows: E expert rows of row_bytes each, expert e at rows + e*row_bytes.
 * Outputs (any may be NULL except y): logits FP32 [T][E], ids [T][k],
 * w double [T][k], h FP16 [T*k][I] and o double [T*k][H] indexed by pair
 * p = t*k + j.  shared_os / shared_sigma: optional shared-expert terms
 * (double [T][H] and [T]).  Returns 0, or -1 on allocation failure. */
static int layer_impl(const uint16_t *x, const uint16_t *wr, const float *bias, const uint8_t *rows,
                      size_t row_bytes, int T, int H, int I, int E, int k,
                      const double *shared_os, const double *shared_sigma,
                      uint16_t *y, float *logits_out, int32_t *ids_out, double *w_out,
                      uint16_t *h_out, double *o_out, int fp16_weights)
{
    int n = T * k;
    float *logits = (float *)malloc(sizeof(float) * (size_t)T * E);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    double *w = (double *)malloc(sizeof(double) * (size_t)n);
    double *o = (double *)malloc(sizeof(double) * (size_t)n * H);
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
    double *Wg = (double *)malloc(sizeof(double) * (size_t)I * H);
    double *Wu = (double *)malloc(sizeof(double) * (size_t)I * H);
    double *Wd = (double *)malloc(sizeof(double) * (size_t)H * I);
    int rc = -1;
    if (!logits || !ids || !w || !o || !h || !Wg || !Wu || !Wd) goto done;

    oracle_router_logits(x, wr, bias, T, H, E, logits);
    oracle_topk_softmax(logits, T, E, k, ids, w);
    for (int e = 0; e < E; ++e) {
        int used = 0;
        for (int p = 0; p < n; ++p) used |= (ids[p] == e);
        if (!used) continue;
        if (fp16_weights) oracle_dequant_expert_fp16(rows + (size_t)e * row_bytes, H, I, Wg, Wu, Wd);
        else oracle_dequant_expert(rows + (size_t)e * row_bytes, H, I, Wg, Wu, Wd);
        for (int p = 0; p < n; ++p) {
            if (ids[p] != e) continue;
            oracle_swiglu_dense(Wg, Wu, Wd, H, I, x + (size_t)(p / k) * H, h, o + (size_t)p * H);
            if (h_out) memcpy(h_out + (size_t)p * I, h, sizeof(uint16_t) * (size_t)I);
        }
    }
    oracle_combine(o, w, shared_os, shared_sigma, T, H, k, y);
    if (logits_out) memcpy(logits_out, logits, sizeof(float) * (size_t)T * E);
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)n);
    if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)n);
    if (o_out) memcpy(o_out, o, sizeof(double) * (size_t)n * H);
    rc = 0;
done:
    free(logits); free(ids); free(w); free(o); free(h); free(Wg); free(Wu); free(Wd);
    return rc;
}

int oracle_layer(const uint16_t *x, const uint16_t *wr, const float *bias, const uint8_t *rows,
                 size_t row_bytes, int T, int H, int I, int E, int k,
                 const double *shared_os, const double *shared_sigma,
                 uint16_t *y, float *logits_out, int32_t *ids_out, double *w_out,
                 uint16_t *h_out, double *o_out)
{
    return layer_impl(x, wr, bias, rows, row_bytes, T, H, I, E, k, shared_os, shared_sigma, y, logits_out, ids_out,
                      w_out, h_out, o_out, 0);
}

/* The same layer in the offload-qpacked profile: expert weights rounded to
 * FP16 (oracle_dequant_expert_fp16), everything else unchanged. */
int oracle_layer_fp16_slots(const uint16_t *x, const uint16_t *wr, const float *bias, const uint8_t *rows,
                            size_t row_bytes, int T, int H, int I, int E, int k,
                            const double *shared_os, const double *shared_sigma,
                            uint16_t *y, float *logits_out, int32_t *ids_out, double *w_out,
                            uint16_t *h_out, double *o_out)
{
    return layer_impl(x, wr, bias, rows, row_bytes, T, H, I, E, k, shared_os, shared_sigma, y, logits_out, ids_out,
                      w_out, h_out, o_out, 1);
}

/* ------------------------------------------------------- array helpers */

void oracle_halves_to_doubles(const uint16_t *h, double *d, size_t n)
{
    for (size_t i = 0; i < n; ++i) d[i] = oracle_half_to_double(h[i]);
}

void oracle_doubles_to_halves(const double *d, uint16_t *h, size_t n)
{
    for (size_t i = 0; i < n; ++i) h[i] = oracle_double_to_half(d[i]);
}
