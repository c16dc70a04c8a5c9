/* Drives every entry point of the CPU oracle on small inputs from a fixed
 * linear congruential sequence, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer: any out-of-bounds access, leak or undefined
 * operation aborts the run.  Exit status 0 means every call returned its
 * documented code. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int coli_oracle_router(const void *x, int x_bf16, const float *w, const float *bias, int n_tok, int hidden,
                       int n_experts, float *logits);
int coli_oracle_topk(const float *logits, int n_tok, int n_experts, int top_k, int32_t *idx, double *weight);
int coli_oracle_union(const int32_t *idx, int n_tok, int top_k, int n_experts, int32_t *n_union,
                      int32_t *union_ids, int32_t *counts, int32_t *offsets, int32_t *gather);
size_t coli_oracle_blob_bytes(int hidden, int inter, int group, int bits);
int coli_oracle_dequant(const uint8_t *blob, int hidden, int inter, int group, int bits, int which, double *out);
int coli_oracle_expert_ffn(const uint8_t *blob, int hidden, int inter, int group, int bits, const double *x,
                           double *y);
int coli_oracle_layer_tokens(const void *x, int x_bf16, int hidden, int inter, int group, int bits, int top_k,
                             const int32_t *idx, const double *weight, const uint8_t *const *blobs,
                             const uint8_t *shared, const int32_t *sel, int n_sel, double *y);

static uint32_t state = 12345u;
static uint32_t next(void) { state = state * 1664525u + 1013904223u; return state >> 8; }
static float unit(void) { return (float)(next() % 2001) / 1000.0f - 1.0f; }

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void)
{
    enum { H = 128, I = 64, E = 6, K = 3, T = 5 };
    float xf[T * H], w[H * E], bias[E], logits[T * E];
    uint16_t xb[T * H];
    for (int i = 0; i < T * H; ++i) {
        xf[i] = unit();
        uint32_t u;
        memcpy(&u, &xf[i], 4);
        xb[i] = (uint16_t)(u >> 16);
    }
    for (int i = 0; i < H * E; ++i) w[i] = unit() * 0.1f;
    for (int e = 0; e < E; ++e) bias[e] = unit();
    CHECK(coli_oracle_router(xf, 0, w, bias, T, H, E, logits) == 0);
    CHECK(coli_oracle_router(xb, 1, w, NULL, T, H, E, logits) == 0);
    CHECK(coli_oracle_router(xf, 0, w, bias, T, 100, E, logits) == -1);

    int32_t idx[T * E];
    double wt[T * E];
    CHECK(coli_oracle_topk(logits, T, E, K, idx, wt) == 0);
    CHECK(coli_oracle_topk(logits, T, E, E, idx, wt) == 0);          /* k = E */
    CHECK(coli_oracle_topk(logits, T, E, E + 1, idx, wt) == -1);
    CHECK(coli_oracle_topk(logits, T, E, K, idx, wt) == 0);

    int32_t nu, ids[E], counts[E], offsets[E + 1], gather[T * K];
    CHECK(coli_oracle_union(idx, T, K, E, &nu, ids, counts, offsets, gather) == 0);
    CHECK(offsets[E] == T * K);
    int32_t bad[T * K];
    memcpy(bad, idx, sizeof bad);
    bad[1] = E;
    CHECK(coli_oracle_union(bad, T, K, E, &nu, ids, counts, offsets, gather) == -1);

    for (int bits = 4; bits <= 8; bits += 4) {
        for (int g = 32; g <= 64; g += 32) {
            size_t n = coli_oracle_blob_bytes(H, I, g, bits);
            CHECK(n > 0);
            uint8_t *blobs_mem[E + 1];
            for (int e = 0; e <= E; ++e) {
                blobs_mem[e] = (uint8_t *)malloc(n);
                CHECK(blobs_mem[e] != NULL);
                for (size_t i = 0; i < n; ++i) blobs_mem[e][i] = (uint8_t)next();
                /* scale sections: small positive fp16 values (0x1c00..0x23ff) */
                size_t qbytes = (size_t)3 * H * I * bits / 8;
                for (size_t i = (qbytes + 255) / 256 * 256; i + 1 < n; i += 2) {
                    uint16_t h = (uint16_t)(0x1c00 + next() % 0x800);
                    memcpy(blobs_mem[e] + i, &h, 2);
                }
            }
            double *dq = (double *)malloc(sizeof(double) * H * I);
            CHECK(dq != NULL);
            for (int which = 0; which < 3; ++which)
                CHECK(coli_oracle_dequant(blobs_mem[0], H, I, g, bits, which, dq) == 0);
            CHECK(coli_oracle_dequant(blobs_mem[0], H, I, g, bits, 3, dq) == -1);
            free(dq);
            double xd[H], yd[H];
            for (int k = 0; k < H; ++k) xd[k] = xf[k];
            CHECK(coli_oracle_expert_ffn(blobs_mem[1], H, I, g, bits, xd, yd) == 0);
            CHECK(coli_oracle_expert_ffn(blobs_mem[1], H, I, 48, bits, xd, yd) == -1);
            const uint8_t *table[E];
            for (int e = 0; e < E; ++e) table[e] = blobs_mem[e];
            int32_t sel[T];
            for (int t = 0; t < T; ++t) sel[t] = T - 1 - t;
            double *y = (double *)malloc(sizeof(double) * T * H);
            CHECK(y != NULL);
            CHECK(coli_oracle_layer_tokens(xb, 1, H, I, g, bits, K, idx, wt, table, blobs_mem[E], sel, T, y) == 0);
            CHECK(coli_oracle_layer_tokens(xf, 0, H, I, g, bits, K, idx, wt, table, NULL, sel, 2, y) == 0);
            table[idx[0]] = NULL;                                  /* a missing blob is an error */
            CHECK(coli_oracle_layer_tokens(xf, 0, H, I, g, bits, K, idx, wt, table, NULL, sel + T - 1, 1, y) == -1);
            free(y);
            for (int e = 0; e <= E; ++e) free(blobs_mem[e]);
        }
    }
    CHECK(coli_oracle_blob_bytes(H, I, 48, 4) == 0);
    CHECK(coli_oracle_blob_bytes(H, I, 32, 6) == 0);
    printf("oracle driver ok\n");
    return 0;
}
