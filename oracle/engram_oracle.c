/*
 * Engram oracle: a plain, slow, literal CPU implementation of the four engram
 * stages (hash, row gather + dequant, wkv projection, gate).
 *
 * TEST INFRASTRUCTURE ONLY.  It is called by the tests, by the smoke check and
 * by the benchmark's CPU-baseline leg, never by the product path.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * Sources (the pages; citations name page, item and section):
 *   [atlas]   docs.atlascybernetics.ai, "spark_model/layers/engram_v41.rs":
 *             module doc (stages 1-4), `EngramHasher::hash`,
 *             `EngramHashTables::from_flat`, `ENGRAM_ROW_BYTES`,
 *             `EngramV41::upload_qk`, `EngramV41::rows_from_q2k`.
 *   [metrale] docs.metrale.ai, "metrale_model_arch/deepseek_v41_ref/engram.rs":
 *             `NgramHashState::forward`, `f32_to_e4m3_rne`, `e4m3_to_f32`,
 *             `regen_table`, `embed_rows`, `linear_bf16`, `gate_and_add`.
 *
 * Precision follows the pages: integer hash in wrapping 64-bit arithmetic,
 * f32 accumulation with a bf16 result for the projection, f32 for the gate.
 * Built with -ffp-contract=off so every f32 product and sum is rounded on its
 * own, as the pages' Rust evaluates them.
 *
 * Readings taken where the pages are silent:
 *   - Q2_K block layout: the pages give only its size (84 bytes, one block per
 *     256-wide row).  The layout used is GGML's k-quant block: 16 scale bytes
 *     (low nibble = sub-block scale, high nibble = sub-block min), 64 bytes of
 *     2-bit quants, fp16 d, fp16 dmin.  Element e of the row reads quant byte
 *     qs[32*(e/128) + e%32] at bit 2*((e%128)/32), with sub-block e/16; the
 *     value is d*scale*q - dmin*min, rounded once to bf16.
 *   - e4m3 scales are f32 powers of two, one per scale_block values of a row,
 *     laid out [row][head_dim/scale_block] as the metrale `EngramTables` keeps
 *     them.
 *   - The gate output stays f32 on the highway (atlas stage 4); rounding it
 *     to bf16 as the metrale reference does is kept behind a flag.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* f32 -> bf16 bits, round to nearest, ties to even (the `to_bf16_rne` the
 * metrale reference rounds every bf16 value with).  bf16 keeps the top 16 bits
 * of the f32 pattern; the dropped 16 bits decide the rounding. */
uint16_t orc_bf16_from_f32(float x)
{
    uint32_t u = f32_bits(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);          /* quiet NaN */
    uint32_t hi = u >> 16, lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1;                                       /* may carry into the exponent */
    return (uint16_t)hi;
}

float orc_f32_from_bf16(uint16_t b) { return bits_f32((uint32_t)b << 16); }

void orc_bf16_from_f32_n(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_bf16_from_f32(x[i]);
}

/* IEEE binary16 -> f32, from the format's definition: 1 sign bit, 5 exponent
 * bits (bias 15), 10 fraction bits; exponent 0 is subnormal (frac * 2^-24). */
float orc_f32_from_f16(uint16_t h)
{
    int sign = (h >> 15) & 1, e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (float)(sign ? -v : v);
}

/* e4m3fn decode ([metrale] `e4m3_to_f32`): exponent field 15 with mantissa 7
 * is NaN; exponent 0 is subnormal m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7). */
float orc_e4m3_to_f32(uint8_t b)
{
    float sign = (b & 0x80) ? -1.0f : 1.0f;
    int e = (b >> 3) & 0x0F;
    float m = (float)(b & 0x07);
    if (e == 15 && m == 7.0f)
        return NAN;
    if (e == 0)
        return sign * m / 8.0f * ldexpf(1.0f, -6);
    return sign * (1.0f + m / 8.0f) * ldexpf(1.0f, e - 7);
}

/* f32 -> e4m3fn code, written from the format itself ([metrale]
 * `f32_to_e4m3_rne` is the saturating, round-to-nearest-even encoder the
 * pages use).  Codes 0x00..0x7E are the non-negative finite e4m3fn values in
 * increasing order (0x7F is NaN), so the magnitude's code is the one whose
 * value lies nearest |x|; exactly half-way between two neighbours the even
 * code wins.  Magnitudes at or past the largest finite value, 448 (0x7E),
 * including infinity, take 0x7E; NaN takes 0x7F; the sign bit is copied. */
uint8_t orc_f32_to_e4m3_rne(float x)
{
    if (isnan(x))
        return 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    const double a = fabs((double)x);
    int below = 0;                         /* the largest code whose value <= a */
    for (int c = 1; c <= 0x7E; c++)
        if ((double)orc_e4m3_to_f32((uint8_t)c) <= a)
            below = c;
    if (below == 0x7E)
        return sign | 0x7E;
    /* both neighbours and their midpoint are exact in double */
    const double half_way = 0.5 * ((double)orc_e4m3_to_f32((uint8_t)below) +
                                   (double)orc_e4m3_to_f32((uint8_t)(below + 1)));
    int code;
    if (a < half_way)
        code = below;
    else if (a > half_way)
        code = below + 1;
    else
        code = (below & 1) ? below + 1 : below;
    return sign | (uint8_t)code;
}

/* ------------------------------------------------------------ 1. the hash */

/* Euclidean remainder a mod p for p > 0, in [0, p) (Rust `rem_euclid`). */
static int64_t rem_euclid(int64_t a, int64_t p)
{
    int64_t r = a % p;
    return r < 0 ? r + p : r;
}

/* Hash `seqlen` token ids placed at start_pos ([atlas] `EngramHasher::hash`,
 * [metrale] `NgramHashState::forward`).
 *
 * cache      [max_seq] compressed ids of every position seen so far (the
 *            caller keeps it between calls; zero-initialised, reset = zero)
 * multipliers[n_layers][max_ngram], primes/offsets [n_layers][cols] with
 *            cols = (max_ngram-1)*n_heads and slot (n-2)*n_heads + head
 * out        [seqlen][n_layers][cols] row ids
 *
 * Returns 0, -1 when start_pos+seqlen > max_seq (nothing written), or -2 when
 * a token id lies outside token_map (the cache holds the positions before it,
 * as the page's loop leaves it). */
int orc_hash(int64_t vocab, const int64_t *token_map, int64_t pad_id,
             int64_t n_layers, int64_t max_ngram, int64_t n_heads,
             const int64_t *multipliers, const int64_t *primes, const int64_t *offsets,
             int64_t *cache, int64_t max_seq,
             const int64_t *input_ids, int64_t seqlen, int64_t start_pos, int64_t *out)
{
    const int64_t ng = max_ngram, nl = n_layers, cols = (max_ngram - 1) * n_heads;
    if (start_pos + seqlen > max_seq)
        return -1;
    /* map every new token into the compressed space and record it */
    for (int64_t s = 0; s < seqlen; s++) {
        int64_t id = input_ids[s];
        if (id < 0 || id >= vocab)
            return -2;
        cache[start_pos + s] = token_map[id];
    }
    int64_t *tokens = (int64_t *)malloc(sizeof(int64_t) * (size_t)ng);
    for (int64_t s = 0; s < seqlen; s++) {
        int64_t pos = start_pos + s;
        /* the n-gram window, newest first; once a shift reaches before
         * position 0 or hits an unmapped (-1) id, it and every larger shift
         * read the pad id */
        int blocked = 0;
        for (int64_t shift = 0; shift < ng; shift++) {
            int64_t src = cache[pos >= shift ? pos - shift : 0];
            blocked = blocked || pos < shift || src == -1;
            tokens[shift] = blocked ? pad_id : src;
        }
        for (int64_t li = 0; li < nl; li++) {
            const int64_t *m = multipliers + li * ng;
            /* wrapping i64 multiply = multiply modulo 2^64 */
            uint64_t rolling = (uint64_t)tokens[0] * (uint64_t)m[0];
            for (int64_t i = 1; i < ng; i++) {
                rolling ^= (uint64_t)tokens[i] * (uint64_t)m[i];
                for (int64_t h = 0; h < n_heads; h++) {
                    int64_t col = (i - 1) * n_heads + h;
                    out[(s * nl + li) * cols + col] =
                        rem_euclid((int64_t)rolling, primes[li * cols + col]) +
                        offsets[li * cols + col];
                }
            }
        }
    }
    free(tokens);
    return 0;
}

/* --------------------------------------------------- 2. rows and dequant */

/* One Q2_K block (84 bytes) -> 256 bf16 values (layout: see file header). */
void orc_q2k_row(const uint8_t *blk, uint16_t *out)
{
    const uint8_t *scales = blk, *qs = blk + 16;
    float d = orc_f32_from_f16((uint16_t)(blk[80] | (blk[81] << 8)));
    float dmin = orc_f32_from_f16((uint16_t)(blk[82] | (blk[83] << 8)));
    for (int e = 0; e < 256; e++) {
        int sub = e / 16;
        int q = (qs[32 * (e / 128) + e % 32] >> (2 * ((e % 128) / 32))) & 3;
        float sc = (float)(scales[sub] & 15), mn = (float)(scales[sub] >> 4);
        float y = d * sc * (float)q - dmin * mn;
        out[e] = orc_bf16_from_f32(y);
    }
}

/* One e4m3 row -> bf16: code times its block's power-of-two scale, then bf16
 * ([metrale] `regen_table`).  scales has head_dim/scale_block entries. */
void orc_e4m3_row(const uint8_t *codes, const float *scales, int64_t head_dim,
                  int64_t scale_block, uint16_t *out)
{
    for (int64_t d = 0; d < head_dim; d++)
        out[d] = orc_bf16_from_f32(orc_e4m3_to_f32(codes[d]) * scales[d / scale_block]);
}

/* Gather rows by hash id ([metrale] `embed_rows` over the dequantised table;
 * the dequant is row-wise, so dequantising the gathered rows is the same).
 * ids [n_ids] -> out [n_ids][256].  Returns -1 if an id is outside the table. */
int orc_gather_q2k(const uint8_t *table, int64_t n_rows, const int64_t *ids, int64_t n_ids,
                   uint16_t *out)
{
    for (int64_t i = 0; i < n_ids; i++) {
        if (ids[i] < 0 || ids[i] >= n_rows)
            return -1;
        orc_q2k_row(table + ids[i] * 84, out + i * 256);
    }
    return 0;
}

int orc_gather_e4m3(const uint8_t *codes, const float *scales, int64_t n_rows,
                    int64_t head_dim, int64_t scale_block, const int64_t *ids, int64_t n_ids,
                    uint16_t *out)
{
    int64_t nb = head_dim / scale_block;
    for (int64_t i = 0; i < n_ids; i++) {
        if (ids[i] < 0 || ids[i] >= n_rows)
            return -1;
        orc_e4m3_row(codes + ids[i] * head_dim, scales + ids[i] * nb, head_dim,
                     scale_block, out + i * head_dim);
    }
    return 0;
}

/* ----------------------------------------------------- 3. the projection */

typedef struct {
    const uint16_t *x, *w;
    uint16_t *y;
    int64_t rows, in_f, out_f, o0, o1;
} linear_job;

static void *linear_worker(void *arg)
{
    const linear_job *j = (const linear_job *)arg;
    for (int64_t o = j->o0; o < j->o1; o++) {
        const uint16_t *wr = j->w + o * j->in_f;
        for (int64_t r = 0; r < j->rows; r++) {
            const uint16_t *xr = j->x + r * j->in_f;
            float acc = 0.0f;                 /* f32 sum in index order */
            for (int64_t k = 0; k < j->in_f; k++)
                acc += orc_f32_from_bf16(xr[k]) * orc_f32_from_bf16(wr[k]);
            j->y[r * j->out_f + o] = orc_bf16_from_f32(acc);
        }
    }
    return NULL;
}

/* y[r][o] = bf16( sum_k x[r][k] * w[o][k] ), f32 accumulation
 * ([metrale] `linear_bf16`; x [rows][in_f], w [out_f][in_f], y [rows][out_f],
 * all bf16 bits).  Output columns are split across nthreads threads; each
 * output is computed exactly as the single-threaded loop would. */
void orc_linear_bf16(const uint16_t *x, int64_t rows, int64_t in_f, const uint16_t *w,
                     int64_t out_f, uint16_t *y, int64_t nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > out_f)
        nthreads = out_f > 0 ? out_f : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    linear_job *jobs = (linear_job *)malloc(sizeof(linear_job) * (size_t)nthreads);
    for (int64_t t = 0; t < nthreads; t++) {
        jobs[t] = (linear_job){x, w, y, rows, in_f, out_f,
                               out_f * t / nthreads, out_f * (t + 1) / nthreads};
        pthread_create(&th[t], NULL, linear_worker, &jobs[t]);
    }
    for (int64_t t = 0; t < nthreads; t++)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/* ----------------------------------------------------------- 4. the gate */

/* The three f32 sums a gate row needs, accumulated in index order: the
 * highway's energy h.h, the key's energy key.key and the weighted product
 * sum (h * qk) * key, where qk, the gate weight, is the f32 product of the
 * two bf16 weights q and k ([atlas] `upload_qk`). */
static void gate_sums(const float *h, const uint16_t *key, const uint16_t *q_w,
                      const uint16_t *k_w, int64_t dim, float *hh, float *kk, float *dot)
{
    float s_hh = 0.0f, s_kk = 0.0f, s_dot = 0.0f;
    for (int64_t d = 0; d < dim; d++) {
        const float kd = orc_f32_from_bf16(key[d]);
        const float weight = orc_f32_from_bf16(q_w[d]) * orc_f32_from_bf16(k_w[d]);
        s_hh += h[d] * h[d];
        s_kk += kd * kd;
        s_dot += h[d] * weight * kd;
    }
    *hh = s_hh;
    *kk = s_kk;
    *dot = s_dot;
}

/* The gate of one row ([metrale] `gate_and_add`): the weighted product sum
 * scaled by the reciprocal rms of h and of the key (each with eps under the
 * root) and by 1/sqrt(dim); the square root of that score's magnitude, not
 * taken below 1e-6, carries the score's sign into a logistic sigmoid. */
static float gate_scalar(float hh, float kk, float dot, int64_t dim, float eps)
{
    const float fdim = (float)dim;
    const float norm = (1.0f / sqrtf(hh / fdim + eps)) * (1.0f / sqrtf(kk / fdim + eps));
    const float score = dot * norm * powf(fdim, -0.5f);
    const float root = sqrtf(fmaxf(fabsf(score), 1e-6f));
    return 1.0f / (1.0f + expf(-copysignf(root, score)));
}

typedef struct {
    float *h;
    const uint16_t *kv, *q_w, *k_w;
    int64_t hc, dim, t0, t1;
    float eps;
    int round_bf16;
} gate_job;

/* Tokens t0..t1-1: for each stream, its gate from the three sums, then
 * h += gate * value in f32 (rounded to bf16 afterwards only under the flag). */
static void *gate_worker(void *arg)
{
    const gate_job *j = (const gate_job *)arg;
    const int64_t hc = j->hc, dim = j->dim, kv_w = dim * (hc + 1);
    for (int64_t t = j->t0; t < j->t1; t++) {
        const uint16_t *kv_t = j->kv + t * kv_w;
        const uint16_t *value = kv_t + hc * dim;
        for (int64_t c = 0; c < hc; c++) {
            float *h = j->h + (t * hc + c) * dim;
            float hh, kk, dot;
            gate_sums(h, kv_t + c * dim, j->q_w + c * dim, j->k_w + c * dim, dim, &hh, &kk, &dot);
            const float gate = gate_scalar(hh, kk, dot, dim, j->eps);
            for (int64_t d = 0; d < dim; d++) {
                const float y = h[d] + gate * orc_f32_from_bf16(value[d]);
                h[d] = j->round_bf16 ? orc_f32_from_bf16(orc_bf16_from_f32(y)) : y;
            }
        }
    }
    return NULL;
}

/* In place on h [tokens][hc][dim] (f32): for every token and stream, the
 * normalised dot of the stream against its key, the signed-sqrt sigmoid gate,
 * and h += gate * value ([metrale] `gate_and_add`; f32 highway per [atlas]
 * stage 4).  kv [tokens][dim*(hc+1)] bf16 bits: key c = kv[t][c*dim..],
 * value = kv[t][hc*dim..].  q_w, k_w [hc][dim] bf16 bits.  Tokens are split
 * across nthreads threads. */
void orc_gate_and_add(float *h, const uint16_t *kv, const uint16_t *q_w, const uint16_t *k_w,
                      int64_t tokens, int64_t hc, int64_t dim, float eps, int64_t round_bf16,
                      int64_t nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > tokens)
        nthreads = tokens > 0 ? tokens : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    gate_job *jobs = (gate_job *)malloc(sizeof(gate_job) * (size_t)nthreads);
    for (int64_t t = 0; t < nthreads; t++) {
        jobs[t] = (gate_job){h, kv, q_w, k_w, hc, dim, tokens * t / nthreads,
                             tokens * (t + 1) / nthreads, eps, (int)round_bf16};
        pthread_create(&th[t], NULL, gate_worker, &jobs[t]);
    }
    for (int64_t t = 0; t < nthreads; t++)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}
