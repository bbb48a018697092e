/*
 * Plain CPU oracle for the routed-expert MoE FFN stage of prompt ingestion.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline
 * leg may load this library.  It shares no code with the HIP library and includes none of
 * its headers.
 *
 * What it computes (Red Lite dev75 "Prompt ingestion" and "Decode" sections; dev72
 * "2-row verify" section and "GPU profiling", second profile):
 *   - token-expert pairs are grouped per expert (the unit of expert work in the pages);
 *   - for each pair (token t, selection slot j, expert e):
 *       g = Wg_e x_t,  u = Wu_e x_t,  h = silu(g) * u,  y = Wd_e h
 *   - out_t = sum over j = 0..k-1, in selection order, of w[t][j] * y_{t,j}
 *     (the MoE tail sums the expert outputs in the row's selection order).
 * Expert weights are 256-value blocks of the Q2B / T1 formats and are decoded here with
 * scalar loops straight from the format definition.
 * Also the router, the step before the path: softmax over the experts, the k most probable in
 * descending order (ties to the lower id), renormalised weights (orc_route).
 *
 * Precision: every floating-point step is IEEE double; the decoded weights d*s*c are exact
 * in double, x is bf16 (exact in double), silu uses the C library exp.
 *
 * Threads: experts are split over threads, every pair result is computed by exactly one
 * thread in a fixed order, and the combine runs per token in selection order, so results do
 * not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q2B 1
#define ORC_T1 2

typedef struct {
    int32_t qtype;
    int32_t reserved;
    uint64_t gate_off, up_off, down_off;
} orc_desc;

/* ---------------------------------------------------------------- scalar conversions */

/* IEEE binary16 -> double from the bit fields: sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is subnormal (fraction * 2^-24), exponent 31 is inf/NaN. */
double orc_fp16_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 31;
    int fr = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + fr), ex - 25);
    return sign ? -v : v;
}

/* bfloat16 -> double: the bf16 bits are the high half of an IEEE binary32. */
double orc_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ---------------------------------------------------------------- block decode */

int orc_block_bytes(int qtype) {
    if (qtype == ORC_Q2B) return 74;
    if (qtype == ORC_T1) return 57;
    return -1;
}

/* Value o (0..255) of one Q2B block: d * s * (q - 1.5). */
static double q2b_value(const uint8_t* blk, int o) {
    double d = orc_fp16_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    int sb = o / 16;
    int s = (blk[2 + sb / 2] >> (4 * (sb % 2))) & 15;
    int q = (blk[10 + o / 4] >> (2 * (o % 4))) & 3;
    return d * (double)s * ((double)q - 1.5);
}

/* Value o (0..255) of one T1 block: d * s * (digit - 1), digit o%5 of byte 5 + o/5. */
static double t1_value(const uint8_t* blk, int o) {
    double d = orc_fp16_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    uint32_t sc = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16);
    int s = (int)((sc >> (3 * (o / 32))) & 7);
    int byte = blk[5 + o / 5];
    int digit = byte;
    for (int i = 0; i < o % 5; ++i) digit /= 3;
    digit %= 3;
    return d * (double)s * (double)(digit - 1);
}

static int valid_block(int qtype, const uint8_t* blk) {
    if (qtype == ORC_Q2B) return 1;
    if (qtype == ORC_T1) {
        for (int i = 0; i < 52; ++i)
            if (blk[5 + i] > 242) return 0; /* a byte holds at most five base-3 digits */
        return 1;
    }
    return 0;
}

/* Decode n_values (a multiple of 256) consecutive values.  Returns 0, or -1 for an unknown
 * type / bad size, or -2 for a T1 byte outside 0..242. */
int orc_dequant(int qtype, const uint8_t* blocks, int64_t n_values, double* out) {
    int bb = orc_block_bytes(qtype);
    if (bb < 0 || n_values < 0 || n_values % 256) return -1;
    for (int64_t b = 0; b < n_values / 256; ++b) {
        const uint8_t* blk = blocks + b * bb;
        if (!valid_block(qtype, blk)) return -2;
        for (int o = 0; o < 256; ++o)
            out[b * 256 + o] = qtype == ORC_Q2B ? q2b_value(blk, o) : t1_value(blk, o);
    }
    return 0;
}

/* Full [rows x cols] matrix whose row-major flattening is cut into 256-value blocks. */
static int decode_matrix(int qtype, const uint8_t* base, int rows, int cols, double* out) {
    return orc_dequant(qtype, base, (int64_t)rows * cols, out);
}

/* ---------------------------------------------------------------- pair grouping */

/* Pairs (t, j) grouped per expert, ordered by (expert, token, slot).
 *   offsets[E+1]   exclusive prefix sum of the per-expert pair counts
 *   pair_src[P]    t*k + j of the pair at each sorted position
 *   inv[T*k]       sorted position of pair (t, j)
 * Returns 0, or -1 if an id is outside [0, E) (outputs then unspecified). */
int orc_group_pairs(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* pair_src, int32_t* inv) {
    int64_t P = (int64_t)T * k;
    int32_t* fill = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
    if (!fill) return -3;
    for (int e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (ids[p] < 0 || ids[p] >= E) {
            free(fill);
            return -1;
        }
        offsets[ids[p] + 1] += 1;
    }
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = ids[(int64_t)t * k + j];
            int pos = offsets[e] + fill[e]++;
            pair_src[pos] = t * k + j;
            inv[(int64_t)t * k + j] = pos;
        }
    free(fill);
    return 0;
}

/* ---------------------------------------------------------------- expert FFN */

/* silu(z) = z / (1 + e^-z) */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One pair: g_i = sum_c Wg[i][c] x[c], u_i likewise (c ascending), h_i = silu(g_i) u_i,
 * y_c = sum_i Wd[c][i] h_i (i ascending). */
static void pair_ffn(const double* Wg, const double* Wu, const double* Wd, const double* xf, int H, int I,
                     double* h, double* y) {
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        const double* rg = Wg + (int64_t)i * H;
        const double* ru = Wu + (int64_t)i * H;
        for (int c = 0; c < H; ++c) {
            g += rg[c] * xf[c];
            u += ru[c] * xf[c];
        }
        h[i] = silu(g) * u;
    }
    for (int c = 0; c < H; ++c) {
        double acc = 0.0;
        const double* rd = Wd + (int64_t)c * I;
        for (int i = 0; i < I; ++i) acc += rd[i] * h[i];
        y[c] = acc;
    }
}

typedef struct {
    const uint16_t* x;
    const int32_t* ids;
    const uint8_t* arena;
    const orc_desc* desc;
    int E, H, I, T, k;
    const int32_t* tokens; /* the tokens to compute (indices into x / ids) */
    int n_tokens;
    double* y;             /* [n_tokens][k][H] */
    double* h;             /* optional [n_tokens][k][I] */
    int next_expert;
    int err;
    pthread_mutex_t mu;
} job_t;

static void* worker(void* arg) {
    job_t* jb = (job_t*)arg;
    int H = jb->H, I = jb->I, k = jb->k;
    double* Wg = (double*)malloc(sizeof(double) * (size_t)I * H);
    double* Wu = (double*)malloc(sizeof(double) * (size_t)I * H);
    double* Wd = (double*)malloc(sizeof(double) * (size_t)I * H);
    double* xf = (double*)malloc(sizeof(double) * (size_t)H);
    double* hb = (double*)malloc(sizeof(double) * (size_t)I);
    if (!Wg || !Wu || !Wd || !xf || !hb) {
        pthread_mutex_lock(&jb->mu);
        jb->err = -3;
        pthread_mutex_unlock(&jb->mu);
        goto done;
    }
    for (;;) {
        pthread_mutex_lock(&jb->mu);
        int e = jb->next_expert++;
        pthread_mutex_unlock(&jb->mu);
        if (e >= jb->E) break;
        int used = 0;
        for (int ti = 0; ti < jb->n_tokens && !used; ++ti)
            for (int j = 0; j < k; ++j)
                if (jb->ids[(int64_t)jb->tokens[ti] * k + j] == e) used = 1;
        if (!used) continue;
        const orc_desc* dsc = jb->desc + e;
        int q = dsc->qtype;
        int rc = decode_matrix(q, jb->arena + dsc->gate_off, I, H, Wg);
        if (!rc) rc = decode_matrix(q, jb->arena + dsc->up_off, I, H, Wu);
        if (!rc) rc = decode_matrix(q, jb->arena + dsc->down_off, H, I, Wd);
        if (rc) {
            pthread_mutex_lock(&jb->mu);
            jb->err = rc;
            pthread_mutex_unlock(&jb->mu);
            continue;
        }
        for (int ti = 0; ti < jb->n_tokens; ++ti) {
            int t = jb->tokens[ti];
            for (int j = 0; j < k; ++j) {
                if (jb->ids[(int64_t)t * k + j] != e) continue;
                for (int c = 0; c < H; ++c) xf[c] = orc_bf16_to_double(jb->x[(int64_t)t * H + c]);
                double* yp = jb->y + ((int64_t)ti * k + j) * H;
                pair_ffn(Wg, Wu, Wd, xf, H, I, hb, yp);
                if (jb->h) memcpy(jb->h + ((int64_t)ti * k + j) * I, hb, sizeof(double) * (size_t)I);
            }
        }
    }
done:
    free(Wg);
    free(Wu);
    free(Wd);
    free(xf);
    free(hb);
    return NULL;
}

/* Routed-expert layer on a list of tokens.
 *   x [T][H] bf16 bits, ids/w [T][k] (column j = j-th selection), arena + desc[E]
 *   tokens[n_tokens]: which tokens to compute (NULL = all T in order)
 *   out [n_tokens][H]: sum over j in selection order of w[t][j] * y_{t,j}
 *   h_out (optional) [n_tokens][k][I]: the per-pair h
 * Returns 0; -1 bad id/shape; -2 invalid block byte; -3 out of memory. */
int orc_moe_prefill(const uint16_t* x, const int32_t* ids, const float* w, const uint8_t* arena,
                    const orc_desc* desc, int E, int H, int I, int T, int k, const int32_t* tokens,
                    int n_tokens, double* out, double* h_out, int nthreads) {
    if (T < 0 || k < 1 || E < 1 || H < 1 || I < 1) return -1;
    int32_t* all = NULL;
    if (!tokens) {
        all = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
        if (!all) return -3;
        for (int t = 0; t < T; ++t) all[t] = t;
        tokens = all;
        n_tokens = T;
    }
    for (int ti = 0; ti < n_tokens; ++ti) {
        if (tokens[ti] < 0 || tokens[ti] >= T) {
            free(all);
            return -1;
        }
        for (int j = 0; j < k; ++j) {
            int e = ids[(int64_t)tokens[ti] * k + j];
            if (e < 0 || e >= E) {
                free(all);
                return -1;
            }
        }
    }
    double* y = (double*)calloc((size_t)n_tokens * k * H + 1, sizeof(double));
    if (!y) {
        free(all);
        return -3;
    }
    job_t jb;
    memset(&jb, 0, sizeof(jb));
    jb.x = x;
    jb.ids = ids;
    jb.arena = arena;
    jb.desc = desc;
    jb.E = E;
    jb.H = H;
    jb.I = I;
    jb.T = T;
    jb.k = k;
    jb.tokens = tokens;
    jb.n_tokens = n_tokens;
    jb.y = y;
    jb.h = h_out;
    pthread_mutex_init(&jb.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, worker, &jb) == 0) ++started;
    if (started == 0) worker(&jb);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&jb.mu);
    if (jb.err) {
        free(y);
        free(all);
        return jb.err;
    }
    /* combine: for each token, acc starts at +0 and adds w[t][j] * y_{t,j} for j = 0..k-1 */
    for (int ti = 0; ti < n_tokens; ++ti) {
        int t = tokens[ti];
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) acc += (double)w[(int64_t)t * k + j] * y[((int64_t)ti * k + j) * H + c];
            out[(int64_t)ti * H + c] = acc;
        }
    }
    free(y);
    free(all);
    return 0;
}

/* ---------------------------------------------------------------- the MoE block: shared expert, residual */

/* The MoE block around the routed experts (Red Lite dev75, "Prompt ingestion": the prefill
 * profile lists the shared expert beside the routed experts; the block's output joins the
 * residual stream):
 *   out_t = ((sum over j = 0..k-1, in selection order, of w[t][j] * y_{t,j}) + g_t * s_t) + r_t
 * where s_t = Wd_s (silu(Wg_s x_t) * (Wu_s x_t)) is the shared expert, a dense SwiGLU FFN of the
 * same shapes stored like the routed ones (descriptor `shared` of desc[E]), g_t = shared_gate[t]
 * (the caller's per-token gate of the shared expert), r_t = residual[t] (NULL: no residual).  The
 * shared term is one more term of the same ordered sum, taken after the routed ones; k may be 0
 * (the shared expert alone).  Arguments otherwise as orc_moe_prefill.  Returns as
 * orc_moe_prefill, and -1 for a `shared` outside [0, E). */
int orc_moe_block(const uint16_t* x, const int32_t* ids, const float* w, const uint8_t* arena, const orc_desc* desc,
                  int E, int H, int I, int T, int k, int shared, const float* shared_gate, const float* residual,
                  const int32_t* tokens, int n_tokens, double* out, int nthreads) {
    if (T < 0 || k < 0 || shared < 0 || shared >= E || !shared_gate) return -1;
    const int k1 = k + 1;
    int32_t* ids1 = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * k1);
    float* w1 = (float*)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * k1);
    if (!ids1 || !w1) {
        free(ids1);
        free(w1);
        return -3;
    }
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            ids1[(int64_t)t * k1 + j] = ids[(int64_t)t * k + j];
            w1[(int64_t)t * k1 + j] = w[(int64_t)t * k + j];
        }
        ids1[(int64_t)t * k1 + k] = shared;
        w1[(int64_t)t * k1 + k] = shared_gate[t];
    }
    int rc = orc_moe_prefill(x, ids1, w1, arena, desc, E, H, I, T, k1, tokens, n_tokens, out, NULL, nthreads);
    free(ids1);
    free(w1);
    if (rc || !residual) return rc;
    const int n = tokens ? n_tokens : T;
    for (int ti = 0; ti < n; ++ti) {
        const int t = tokens ? tokens[ti] : ti;
        for (int c = 0; c < H; ++c) out[(int64_t)ti * H + c] += (double)residual[(int64_t)t * H + c];
    }
    return 0;
}

/* ---------------------------------------------------------------- router (the step before the path) */

/* Router of one layer (reading of the MoE routing the pages take as given: softmax over the
 * experts, the k most probable experts in descending order, their probabilities renormalised
 * to sum to one; Red Lite dev72 "2-row verify" section keeps each row's selection order).
 *   logits[T][E]   fp32 router logits
 *   ids[T][k]      column j = the j-th selection: descending probability, ties to the lower id
 *   w[T][k]        p_{ids[t][j]} / (sum over j' = 0..k-1, in selection order, of p_{ids[t][j']})
 * with p = softmax(logits[t]) over all E experts, in double: m = max logit,
 * p_e = exp(l_e - m) / sum_e' exp(l_e' - m) (e' ascending).  p is strictly increasing in the
 * logit, so "descending probability" is "descending logit": the selection compares the fp32
 * logits themselves (exact), and equal logits are equal probabilities (ties).
 * Selection is k passes of a plain scan for the best remaining expert.
 * Returns 0; -1 on a bad shape (E < 1, k < 1 or k > E); -3 on allocation failure. */
int orc_route(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
    if (E < 1 || k < 1 || k > E) return -1;
    double* p = (double*)malloc((size_t)E * sizeof(double));
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    if (!p || !taken) {
        free(p);
        free(taken);
        return -3;
    }
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        double m = (double)l[0];
        for (int e = 1; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - m);
            z += p[e];
        }
        for (int e = 0; e < E; ++e) p[e] /= z;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e; /* strict: an equal logit keeps the lower id */
            }
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += p[ids[(int64_t)t * k + j]];
        for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = p[ids[(int64_t)t * k + j]] / s;
    }
    free(p);
    free(taken);
    return 0;
}
