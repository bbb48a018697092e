/*
 * Oracle exercise for the sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer): every
 * entry point of oracle/rl_oracle.c on small inputs, including its error paths, with several
 * thread counts.  Exits 0 when every call returns what its header promises; a sanitizer report
 * aborts with a non-zero status.  Inputs come from a fixed 64-bit LCG (contents do not matter
 * here, only that every code path and buffer edge is touched).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t qtype;
    int32_t reserved;
    uint64_t gate_off, up_off, down_off;
} orc_desc;

double orc_fp16_to_double(uint16_t h);
double orc_bf16_to_double(uint16_t b);
int orc_block_bytes(int qtype);
int orc_dequant(int qtype, const uint8_t* blocks, int64_t n_values, double* out);
int orc_group_pairs(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* pair_src, int32_t* inv);
int orc_moe_prefill(const uint16_t* x, const int32_t* ids, const float* w, const uint8_t* arena,
                    const orc_desc* desc, int E, int H, int I, int T, int k, const int32_t* tokens,
                    int n_tokens, double* out, double* h_out, int nthreads);
int orc_moe_block(const uint16_t* x, const int32_t* ids, const float* w, const uint8_t* arena, const orc_desc* desc,
                  int E, int H, int I, int T, int k, int shared, const float* shared_gate, const float* residual,
                  const int32_t* tokens, int n_tokens, double* out, int nthreads);
int orc_route(const float* logits, int T, int E, int k, int32_t* ids, double* w);

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(st >> 33);
}

static int fails = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++fails;                                               \
        }                                                          \
    } while (0)

/* n blocks of a type with valid random contents (T1 digit bytes below 243, scale d = a small
 * fp16 value) */
static void fill_blocks(int qtype, uint8_t* p, int n) {
    const int bb = orc_block_bytes(qtype);
    for (int b = 0; b < n; ++b) {
        uint8_t* blk = p + (size_t)b * bb;
        for (int i = 0; i < bb; ++i) blk[i] = (uint8_t)rnd();
        blk[0] = 0x00;
        blk[1] = 0x24 + (uint8_t)(rnd() % 4); /* fp16 around 2^-6 */
        if (qtype == 2)
            for (int i = 5; i < 57; ++i) blk[i] = (uint8_t)(rnd() % 243);
    }
}

static uint16_t bf16_of(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    return (uint16_t)(u >> 16);
}

int main(void) {
    /* conversions */
    CHECK(orc_fp16_to_double(0x3C00) == 1.0);
    CHECK(orc_fp16_to_double(0xC000) == -2.0);
    CHECK(orc_fp16_to_double(0x0001) == ldexp(1.0, -24));
    CHECK(isinf(orc_fp16_to_double(0x7C00)));
    CHECK(orc_bf16_to_double(0x3F80) == 1.0);
    CHECK(orc_block_bytes(1) == 74 && orc_block_bytes(2) == 57 && orc_block_bytes(3) < 0);

    /* block decode, both types, and the error paths */
    for (int q = 1; q <= 2; ++q) {
        const int nb = 5, bb = orc_block_bytes(q);
        uint8_t* blk = (uint8_t*)malloc((size_t)nb * bb);
        double* out = (double*)malloc(sizeof(double) * nb * 256);
        fill_blocks(q, blk, nb);
        CHECK(orc_dequant(q, blk, nb * 256, out) == 0);
        CHECK(orc_dequant(q, blk, 100, out) == -1);
        if (q == 2) {
            blk[bb + 20] = 250; /* second block: a digit byte outside 0..242 */
            CHECK(orc_dequant(q, blk, nb * 256, out) == -2);
        }
        free(blk);
        free(out);
    }
    CHECK(orc_dequant(7, NULL, 256, NULL) == -1);

    /* grouping, including a bad id */
    {
        const int T = 9, k = 3, E = 5, P = T * k;
        int32_t ids[27], off[6], src[27], inv[27];
        for (int p = 0; p < P; ++p) ids[p] = (int32_t)(rnd() % E);
        CHECK(orc_group_pairs(ids, T, k, E, off, src, inv) == 0);
        CHECK(off[0] == 0 && off[E] == P);
        for (int p = 0; p < P; ++p) CHECK(src[inv[p]] == p);
        ids[4] = E;
        CHECK(orc_group_pairs(ids, T, k, E, off, src, inv) == -1);
    }

    /* the layer and the block for both types and several thread counts */
    for (int q = 1; q <= 2; ++q) {
        const int E = 4, H = 256, I = 64, T = 6, k = 2;
        const int bb = orc_block_bytes(q), mb = H * I / 256 * bb; /* bytes per matrix */
        uint8_t* arena = (uint8_t*)malloc((size_t)3 * E * mb);
        orc_desc desc[4];
        for (int e = 0; e < E; ++e) {
            fill_blocks(q, arena + (size_t)3 * e * mb, 3 * H * I / 256);
            desc[e].qtype = q;
            desc[e].reserved = 0;
            desc[e].gate_off = (uint64_t)3 * e * mb;
            desc[e].up_off = desc[e].gate_off + mb;
            desc[e].down_off = desc[e].up_off + mb;
        }
        uint16_t* x = (uint16_t*)malloc(sizeof(uint16_t) * T * H);
        for (int i = 0; i < T * H; ++i) x[i] = bf16_of((float)((int)(rnd() % 2001) - 1000) / 500.0f);
        int32_t ids[12];
        float w[12], gate[6];
        for (int i = 0; i < T * k; ++i) {
            ids[i] = (int32_t)(rnd() % E);
            w[i] = (float)(rnd() % 100) / 100.0f;
        }
        for (int t = 0; t < T; ++t) gate[t] = 0.5f;
        float* res = (float*)malloc(sizeof(float) * T * H);
        for (int i = 0; i < T * H; ++i) res[i] = (float)i * 1e-3f;
        double* out = (double*)malloc(sizeof(double) * T * H);
        double* out2 = (double*)malloc(sizeof(double) * T * H);
        double* h = (double*)malloc(sizeof(double) * T * k * I);
        CHECK(orc_moe_prefill(x, ids, w, arena, desc, E, H, I, T, k, NULL, 0, out, h, 1) == 0);
        CHECK(orc_moe_prefill(x, ids, w, arena, desc, E, H, I, T, k, NULL, 0, out2, NULL, 3) == 0);
        CHECK(memcmp(out, out2, sizeof(double) * T * H) == 0);
        for (int i = 0; i < T * H; ++i) CHECK(isfinite(out[i]));
        const int32_t sel[2] = {5, 1};
        CHECK(orc_moe_prefill(x, ids, w, arena, desc, E, H, I, T, k, sel, 2, out2, NULL, 2) == 0);
        CHECK(memcmp(out2, out + 5 * H, sizeof(double) * H) == 0);
        CHECK(orc_moe_block(x, ids, w, arena, desc, E, H, I, T, k, E - 1, gate, res, NULL, 0, out, 2) == 0);
        CHECK(orc_moe_block(x, NULL, NULL, arena, desc, E, H, I, T, 0, 0, gate, NULL, NULL, 0, out, 1) == 0);
        CHECK(orc_moe_block(x, ids, w, arena, desc, E, H, I, T, k, E, gate, res, NULL, 0, out, 1) == -1);
        ids[3] = -1;
        CHECK(orc_moe_prefill(x, ids, w, arena, desc, E, H, I, T, k, NULL, 0, out, NULL, 1) == -1);
        free(arena);
        free(x);
        free(res);
        free(out);
        free(out2);
        free(h);
    }

    /* router: random logits, rows of equal logits, bad shapes */
    {
        const int T = 4, E = 9, k = 3;
        float lg[36];
        int32_t ids[12];
        double w[12];
        for (int i = 0; i < T * E; ++i) lg[i] = (float)((int)(rnd() % 200) - 100) / 50.0f;
        for (int e = 0; e < E; ++e) lg[2 * E + e] = 1.0f; /* a row of ties */
        CHECK(orc_route(lg, T, E, k, ids, w) == 0);
        CHECK(ids[6] == 0 && ids[7] == 1 && ids[8] == 2);
        for (int t = 0; t < T; ++t) CHECK(fabs(w[t * k] + w[t * k + 1] + w[t * k + 2] - 1.0) < 1e-12);
        CHECK(orc_route(lg, T, E, E + 1, ids, w) == -1);
        CHECK(orc_route(lg, T, 0, 1, ids, w) == -1);
    }

    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer exercise: all checks passed\n");
    return 0;
}
