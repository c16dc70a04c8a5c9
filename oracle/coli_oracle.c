/*
 * coli_oracle.c -- plain, slow, single-threaded CPU oracle of one int4
 * routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg load this file.  It shares no code, header
 * or table with the HIP library and must be built without -ffast-math and
 * with -ffp-contract=off, so every floating-point operation below is exactly
 * the one written.
 *
 * What one layer computes, per token (Colibri, getting-started page,
 * "トークンごとの処理経路": Route, then Union across the batch, then the
 * experts; README "Il percorso di ogni token": placement changes speed, never
 * router decisions or weight precision).  The pages give no formula; the
 * readings taken here are:
 *
 *  Route    logit[t][e] = canonical fp32 dot(x_t, W_r[:, e]) + b[e]:
 *           partial[l] = fmaf chain over k = l, l+64, l+128, ... ascending
 *           (l = 0..63), then a fixed tree for s = 32,16,...,1 of
 *           partial[i] = partial[i] + partial[i+s], then + b[e].  The
 *           GPU uses the same order, so logits agree bit for bit.
 *  Top-k    the k largest logits under (logit desc, expert id asc); -0 and
 *           +0 compare equal; slot order is rank order.  Selecting on logits
 *           equals selecting on sigmoid scores because sigmoid is strictly
 *           increasing.
 *  Weights  w_j = sigmoid(l_j) / sum_i sigmoid(l_i) over the k selected
 *           (fp64); no extra routed scaling factor.
 *  Union    ascending unique expert ids; counts[E]; offsets = exclusive
 *           prefix sum of counts; gather = entries t*k+j ordered by
 *           (expert asc, token asc).  The shared expert is not in the union.
 *  Experts  int4 two's-complement nibbles (element 2j low nibble, 2j+1 high
 *           nibble), one fp16 scale per `group` consecutive reduction
 *           elements (32 in the fixed configurations; 64 in the container the
 *           README's "Scarica il modello" section ships), w = q * s exactly
 *           in fp64.  The scale sections hold [rows x K/group] fp16.
 *           Weights are 4-bit as above or, with bits = 8, one two's-complement
 *           byte per element in [-128, 127] (the README's "Scarica il
 *           modello" section and the getting-started page require int8 for
 *           the MTP head; the pages give no layout, so the int8 blob keeps
 *           the int4 blob's sections, row order and group scales).  SwiGLU: h = silu(Wg x) * (Wu x),
 *           silu(z) = z * sigmoid(z), y_e = Wd h, all fp64.
 *  Combine  y_t = sum_j w_j * y_{e_j}(x_t) + y_shared(x_t), fp64, where the
 *           shared expert (one always-on expert of the same shape) has
 *           weight 1.
 *
 * Parity pins live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ABI_VERSION 3
#define ALIGN 256

int coli_oracle_version(void) { return ORACLE_ABI_VERSION; }

/* ---------------------------------------------------------------- scalars */

static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* IEEE binary16 -> double, exactly. */
static double half_bits_to_double(uint16_t h)
{
    int sign = h >> 15;
    int ex = (h >> 10) & 31;
    int man = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                 /* subnormal */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man + 1024), ex - 25);     /* 1.man * 2^(ex-15) */
    return sign ? -v : v;
}

double coli_oracle_half_to_double(uint16_t h) { return half_bits_to_double(h); }

/* Signed int4 at reduction index k of a packed row. */
static int nibble_at(const uint8_t *row, int k)
{
    uint8_t b = row[k >> 1];
    int v = (k & 1) ? (b >> 4) : (b & 15);
    return v >= 8 ? v - 16 : v;
}

int coli_oracle_nibble(const uint8_t *row, int k) { return nibble_at(row, k); }

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ---------------------------------------------------------------- route */

/* Canonical fp32 router logit of one (token, expert).  x_bf16 selects the
 * activation storage: 0 -> float32, 1 -> bf16 bit patterns. */
static float router_logit(const void *x, int x_bf16, const float *w,
                          int hidden, int n_experts, int e, float bias)
{
    float partial[64];
    for (int l = 0; l < 64; ++l) {
        float acc = 0.0f;
        for (int k = l; k < hidden; k += 64) {
            float xv = x_bf16 ? bf16_bits_to_float(((const uint16_t *)x)[k])
                              : ((const float *)x)[k];
            acc = fmaf(xv, w[(size_t)k * n_experts + e], acc);
        }
        partial[l] = acc;
    }
    for (int s = 32; s >= 1; s >>= 1)
        for (int i = 0; i < s; ++i)
            partial[i] = partial[i] + partial[i + s];
    return partial[0] + bias;
}

/* logits[t*E + e] for all t < n_tok; returns -1 on bad sizes. */
int coli_oracle_router(const void *x, int x_bf16, const float *w_router,
                       const float *bias, int n_tok, int hidden, int n_experts,
                       float *logits)
{
    if (hidden <= 0 || hidden % 64 != 0 || n_experts <= 0 || n_tok < 0)
        return -1;
    size_t xs = x_bf16 ? sizeof(uint16_t) : sizeof(float);
    for (int t = 0; t < n_tok; ++t) {
        const char *xt = (const char *)x + (size_t)t * hidden * xs;
        for (int e = 0; e < n_experts; ++e)
            logits[(size_t)t * n_experts + e] = router_logit(
                xt, x_bf16, w_router, hidden, n_experts, e,
                bias ? bias[e] : 0.0f);
    }
    return 0;
}

/* a ranks before b under (logit desc, id asc). */
static int ranks_before(float la, int a, float lb, int b)
{
    if (la > lb) return 1;
    if (la < lb) return 0;
    return a < b;
}

int coli_oracle_topk(const float *logits, int n_tok, int n_experts, int top_k,
                     int32_t *idx, double *weight)
{
    if (top_k < 1 || top_k > n_experts)
        return -1;
    char *taken = (char *)malloc((size_t)n_experts);
    if (!taken)
        return -2;
    for (int t = 0; t < n_tok; ++t) {
        const float *l = logits + (size_t)t * n_experts;
        for (int e = 0; e < n_experts; ++e)
            if (!isfinite(l[e])) {
                free(taken);
                return -3;
            }
        memset(taken, 0, (size_t)n_experts);
        double sum = 0.0;
        for (int j = 0; j < top_k; ++j) {
            int best = -1;
            for (int e = 0; e < n_experts; ++e)
                if (!taken[e] && (best < 0 || ranks_before(l[e], e, l[best], best)))
                    best = e;
            taken[best] = 1;
            idx[(size_t)t * top_k + j] = best;
            double s = sigmoid((double)l[best]);
            weight[(size_t)t * top_k + j] = s;
            sum += s;
        }
        for (int j = 0; j < top_k; ++j)
            weight[(size_t)t * top_k + j] /= sum;
    }
    free(taken);
    return 0;
}

/* ---------------------------------------------------------------- union */

int coli_oracle_union(const int32_t *idx, int n_tok, int top_k, int n_experts,
                      int32_t *n_union, int32_t *union_ids, int32_t *counts,
                      int32_t *offsets, int32_t *gather)
{
    for (int e = 0; e < n_experts; ++e)
        counts[e] = 0;
    for (int i = 0; i < n_tok * top_k; ++i) {
        int e = idx[i];
        if (e < 0 || e >= n_experts)
            return -1;
        counts[e] += 1;
    }
    int nu = 0;
    offsets[0] = 0;
    for (int e = 0; e < n_experts; ++e) {
        if (counts[e] > 0)
            union_ids[nu++] = e;
        offsets[e + 1] = offsets[e] + counts[e];
    }
    *n_union = nu;
    int pos = 0;
    for (int e = 0; e < n_experts; ++e)
        for (int t = 0; t < n_tok; ++t)
            for (int j = 0; j < top_k; ++j)
                if (idx[(size_t)t * top_k + j] == e)
                    gather[pos++] = t * top_k + j;
    return 0;
}

/* ---------------------------------------------------------------- experts */

static size_t align_up(size_t n) { return (n + ALIGN - 1) / ALIGN * ALIGN; }

/* Section offsets of a canonical blob: gate_q, up_q, down_q, gate_s, up_s,
 * down_s, total. */
static void blob_offsets(int hidden, int inter, int group, int bits, size_t off[7])
{
    size_t sz[6] = {
        (size_t)inter * hidden * bits / 8, (size_t)inter * hidden * bits / 8,
        (size_t)hidden * inter * bits / 8,
        (size_t)inter * (hidden / group) * 2, (size_t)inter * (hidden / group) * 2,
        (size_t)hidden * (inter / group) * 2,
    };
    size_t o = 0;
    for (int i = 0; i < 6; ++i) {
        off[i] = o;
        o = align_up(o + sz[i]);
    }
    off[6] = o;
}

/* A format the layout supports: 4- or 8-bit weights, a group size that is
 * positive and divides both widths (and even widths for 4-bit packing). */
static int format_ok(int hidden, int inter, int group, int bits)
{
    return (bits == 4 || bits == 8) && group > 0 && hidden > 0 && inter > 0 &&
           hidden % group == 0 && inter % group == 0 && hidden % 2 == 0 && inter % 2 == 0;
}

size_t coli_oracle_blob_bytes(int hidden, int inter, int group, int bits)
{
    size_t off[7];
    if (!format_ok(hidden, inter, group, bits))
        return 0;
    blob_offsets(hidden, inter, group, bits, off);
    return off[6];
}

/* Weight k of a packed row: a nibble (bits 4) or a byte (bits 8), two's
 * complement. */
static int weight_at(const uint8_t *row, int k, int bits)
{
    return bits == 4 ? nibble_at(row, k) : (int)(int8_t)row[k];
}

/* Row r of a [rows x K] int4 or int8 matrix with fp16 group scales,
 * dequantised to fp64: out[k] = q[r][k] * s[r][k / group]. */
static void dequant_row(const uint8_t *q, const uint16_t *s, int K, int group, int bits, int r,
                        double *out)
{
    const uint8_t *row = q + (size_t)r * ((size_t)K * bits / 8);
    const uint16_t *srow = s + (size_t)r * (K / group);
    for (int g = 0; g < K / group; ++g) {
        double scale = half_bits_to_double(srow[g]);
        for (int k = g * group; k < (g + 1) * group; ++k)
            out[k] = (double)weight_at(row, k, bits) * scale;
    }
}

/* y[H] = SwiGLU expert applied to x[H], all fp64.  scratch >= I + 2*H
 * doubles. */
static void expert_ffn(const uint8_t *blob, int hidden, int inter, int group, int bits,
                       const double *x, double *y, double *scratch)
{
    size_t off[7];
    blob_offsets(hidden, inter, group, bits, off);
    const uint8_t *gq = blob + off[0], *uq = blob + off[1], *dq = blob + off[2];
    const uint16_t *gs = (const uint16_t *)(blob + off[3]);
    const uint16_t *us = (const uint16_t *)(blob + off[4]);
    const uint16_t *ds = (const uint16_t *)(blob + off[5]);
    double *h = scratch;
    double *wa = scratch + inter;
    double *wb = wa + hidden;
    for (int r = 0; r < inter; ++r) {
        dequant_row(gq, gs, hidden, group, bits, r, wa);
        dequant_row(uq, us, hidden, group, bits, r, wb);
        double g = 0.0, v = 0.0;
        for (int k = 0; k < hidden; ++k) {
            g += wa[k] * x[k];
            v += wb[k] * x[k];
        }
        h[r] = g * sigmoid(g) * v;
    }
    for (int n = 0; n < hidden; ++n) {
        dequant_row(dq, ds, inter, group, bits, n, wa);
        double acc = 0.0;
        for (int r = 0; r < inter; ++r)
            acc += wa[r] * h[r];
        y[n] = acc;
    }
}

int coli_oracle_expert_ffn(const uint8_t *blob, int hidden, int inter, int group, int bits,
                           const double *x, double *y)
{
    if (!format_ok(hidden, inter, group, bits))
        return -1;
    double *scratch = (double *)malloc(sizeof(double) * ((size_t)inter + 2 * (size_t)hidden));
    if (!scratch)
        return -2;
    expert_ffn(blob, hidden, inter, group, bits, x, y, scratch);
    free(scratch);
    return 0;
}

/* Dequantise one [rows x K] matrix of a blob to fp64 (row-major). which:
 * 0 gate, 1 up, 2 down. */
int coli_oracle_dequant(const uint8_t *blob, int hidden, int inter, int group, int bits,
                        int which, double *out)
{
    size_t off[7];
    if (which < 0 || which > 2 || !format_ok(hidden, inter, group, bits))
        return -1;
    blob_offsets(hidden, inter, group, bits, off);
    int rows = which == 2 ? hidden : inter;
    int K = which == 2 ? inter : hidden;
    const uint8_t *q = blob + off[which];
    const uint16_t *s = (const uint16_t *)(blob + off[3 + which]);
    for (int r = 0; r < rows; ++r)
        dequant_row(q, s, K, group, bits, r, out + (size_t)r * K);
    return 0;
}

/* ---------------------------------------------------------------- layer */

/* y[n_sel x H] (fp64) for the tokens listed in sel[], given the routing
 * (idx, weight) of the whole batch.  blobs[e] must be non-NULL for every
 * expert some selected token routes to; shared may be NULL (no shared
 * expert). */
int coli_oracle_layer_tokens(const void *x, int x_bf16, int hidden, int inter, int group,
                             int bits, int top_k, const int32_t *idx, const double *weight,
                             const uint8_t *const *blobs, const uint8_t *shared,
                             const int32_t *sel, int n_sel, double *y)
{
    if (!format_ok(hidden, inter, group, bits))
        return -1;
    double *xt = (double *)malloc(sizeof(double) * (size_t)hidden);
    double *ye = (double *)malloc(sizeof(double) * (size_t)hidden);
    double *scratch = (double *)malloc(sizeof(double) * ((size_t)inter + 2 * (size_t)hidden));
    if (!xt || !ye || !scratch) {
        free(xt); free(ye); free(scratch);
        return -2;
    }
    size_t xs = x_bf16 ? sizeof(uint16_t) : sizeof(float);
    for (int i = 0; i < n_sel; ++i) {
        int t = sel[i];
        const char *xr = (const char *)x + (size_t)t * hidden * xs;
        for (int k = 0; k < hidden; ++k)
            xt[k] = x_bf16 ? (double)bf16_bits_to_float(((const uint16_t *)xr)[k])
                           : (double)((const float *)xr)[k];
        double *yt = y + (size_t)i * hidden;
        for (int n = 0; n < hidden; ++n)
            yt[n] = 0.0;
        for (int j = 0; j < top_k; ++j) {
            int e = idx[(size_t)t * top_k + j];
            if (!blobs[e]) {
                free(xt); free(ye); free(scratch);
                return -1;
            }
            double w = weight[(size_t)t * top_k + j];
            expert_ffn(blobs[e], hidden, inter, group, bits, xt, ye, scratch);
            for (int n = 0; n < hidden; ++n)
                yt[n] += w * ye[n];
        }
        if (shared) {
            expert_ffn(shared, hidden, inter, group, bits, xt, ye, scratch);
            for (int n = 0; n < hidden; ++n)
                yt[n] += ye[n];
        }
    }
    free(xt); free(ye); free(scratch);
    return 0;
}
