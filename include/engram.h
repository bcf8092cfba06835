/*
 * engram.h -- C ABI of the MI355X (gfx950) engram hot path.
 *
 * The DeepSeek-V4.1 engram layer, per token: hash the token's window of the
 * last max_ngram compressed ids into `cols` table row ids, gather and
 * dequantise those rows to bf16, project their concatenation through `wkv`
 * into a key for each hyper-connection stream and a value the streams share,
 * and gate the value onto the FP32 highway (atlascybernetics "spark_model/layers/engram_v41.rs", module
 * doc, stages 1-4; metrale "metrale_model_arch/deepseek_v41_ref/engram.rs",
 * module doc).
 *
 * Conventions for every entry point:
 *   - Pointers named d_* are device memory owned by the caller (this library
 *     never allocates or frees device memory); every other pointer is host
 *     memory, read during the call only.
 *   - bf16 values travel as uint16_t bit patterns.  Arrays are row-major and
 *     densely packed, with the shapes given in brackets.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work: they return before the GPU runs it and never synchronise,
 *     except engram_check.
 *   - Return value: ENGRAM_OK (0) or a negative ENGRAM_E_* code.  Every
 *     argument check runs on the host before any launch; a refused call
 *     enqueues nothing and leaves every buffer untouched.  engram_last_error()
 *     returns the message of the calling thread's last failure.
 *   - A stateless call with T = 0 checks its sizes and returns ENGRAM_OK
 *     without touching memory; its array pointers may then be NULL.
 *   - Errors only the device can see (a token id outside the vocabulary, a
 *     row id outside the table) are recorded in a caller-supplied int32
 *     error word (d_err, nullable) as a bit mask of ENGRAM_DEVERR_*; the
 *     offending item is processed as documented per call, never read out of
 *     bounds.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENGRAM_ABI_VERSION 7

#define ENGRAM_OK 0
#define ENGRAM_E_ARG (-1)          /* null pointer, bad size or geometry          */
#define ENGRAM_E_RANGE (-2)        /* start_pos+T > max_seq, T > max_tokens, ...   */
#define ENGRAM_E_UNSUPPORTED (-3)  /* hc outside 1..4, head_dim, format, limits    */
#define ENGRAM_E_STATE (-4)        /* call order of the stateful context           */
#define ENGRAM_E_HIP (-5)          /* the HIP runtime refused a launch or copy     */
#define ENGRAM_E_DEVICE (-6)       /* engram_check: the device error word is set   */

/* bits of the device error word */
#define ENGRAM_DEVERR_TOKEN 1      /* token id < 0 or >= vocab                     */
#define ENGRAM_DEVERR_ROW 2        /* row id < 0 or >= the table's row count       */
#define ENGRAM_DEVERR_POSITION 4   /* graph mode: a step past max_seq              */

/* limits of the hash geometry (the hash constants travel as kernel arguments) */
#define ENGRAM_MAX_LAYERS 4
#define ENGRAM_MAX_NGRAM 8
#define ENGRAM_MAX_SLOTS 128       /* n_layers * (max_ngram - 1) * n_heads         */

/* Q2_K row: one 84-byte super-block per 256-wide row (atlascybernetics
 * "engram_v41.rs", ENGRAM_ROW_BYTES and module doc stage 2). */
#define ENGRAM_Q2K_ROW_BYTES 84

/* The message of the calling thread's last refused or failed call ("" if
 * none); valid until that thread's next failing call. */
const char *engram_last_error(void);
/* ENGRAM_ABI_VERSION of the built library: a binding checks it against the
 * header it was written for. */
int32_t engram_abi_version(void);

/* ------------------------------------------------------------------ hash */

/* The hash tables (atlascybernetics "engram_v41.rs", EngramHashTables and
 * from_flat).  cols = (max_ngram - 1) * n_heads; slot (n-2)*n_heads + head
 * holds the constants of n-gram size n (2..max_ngram) and head `head`.
 *   n_layers in 1..ENGRAM_MAX_LAYERS, max_ngram in 2..ENGRAM_MAX_NGRAM,
 *   n_heads >= 1, n_layers * cols <= ENGRAM_MAX_SLOTS;
 *   d_token_map [vocab] int64, device: compressed id of every token, -1 =
 *               unmapped (treated as pad and blocking every larger shift);
 *   pad_id      the pad token's compressed id (token_map[pad token]);
 *   multipliers [n_layers][max_ngram] host, each >= 0 (the pages' tables are
 *               unsigned values that must fit i64);
 *   primes      [n_layers][cols] host, each > 0;
 *   offsets     [n_layers][cols] host, each >= 0, offset + prime <= 2^62. */
typedef struct engram_hash_tables {
    int32_t n_layers;
    int32_t max_ngram;
    int32_t n_heads;
    int32_t reserved;
    int64_t vocab;
    int64_t pad_id;
    const int64_t *d_token_map;
    const int64_t *multipliers;
    const int64_t *primes;
    const int64_t *offsets;
} engram_hash_tables;

/* Hash T tokens placed at positions start_pos .. start_pos+T-1
 * (atlascybernetics "engram_v41.rs", EngramHasher::hash; metrale
 * "engram.rs", NgramHashState::forward).
 *   d_ids      [T] int32 token ids;
 *   d_history  [max_seq] int64, the sequence's compressed-id cache: read at
 *              positions < start_pos (look-back of the previous calls;
 *              never-written positions must hold 0, as the zero-initialised
 *              cache does), written at start_pos .. start_pos+T-1;
 *   d_row_ids  [T][n_layers][cols] int64 output:
 *              id = rem_euclid(window hash, prime) + offset, the window hash
 *              of n-gram size n being the XOR over shifts i < n of
 *              token[i] * multiplier[i] in wrapping 64-bit arithmetic, with
 *              the sticky pad rule of the pages;
 *   d_err      nullable; a token id outside [0, vocab) sets
 *              ENGRAM_DEVERR_TOKEN and is hashed as an unmapped (-1) token.
 * Refuses (ENGRAM_E_RANGE) start_pos + T > max_seq. T = 0 is a no-op. */
int32_t engram_hash(const engram_hash_tables *tables, const int32_t *d_ids, int64_t T,
                    int64_t start_pos, int64_t *d_history, int64_t max_seq,
                    int64_t *d_row_ids, int32_t *d_err, void *stream);

/* The same hash for B sequences at one common position, each with its own
 * cache (metrale "engram.rs", NgramHashState: input_ids [batch, seqlen],
 * cache [batch * max_seq], output [batch, seqlen, n_layers, n_hash_cols]):
 *   d_ids [B][T] int32, d_history [B][max_seq] int64 (row b is sequence b's
 *   cache, as in engram_hash), d_row_ids [B*T][n_layers][cols] int64.
 * B = 1 is engram_hash.  B = 0 or T = 0 is a no-op. */
int32_t engram_hash_batch(const engram_hash_tables *tables, const int32_t *d_ids, int64_t B,
                          int64_t T, int64_t start_pos, int64_t *d_history, int64_t max_seq,
                          int64_t *d_row_ids, int32_t *d_err, void *stream);

/* -------------------------------------------------------- gather + dequant */

#define ENGRAM_FMT_Q2K 0
#define ENGRAM_FMT_E4M3 1

/* One layer's table, in device memory or in pinned host memory mapped for
 * the device (engram_map_host: the kernels then read the rows across the
 * host link).
 *   ENGRAM_FMT_Q2K: d_data [n_rows][84] Q2_K blocks (16 bytes of 4-bit
 *       scale/min pairs, 64 bytes of 2-bit quants, fp16 d, fp16 dmin; GGML's
 *       k-quant block, which the pages name by size only), head_dim = 256,
 *       d_scales = NULL;
 *   ENGRAM_FMT_E4M3: d_data [n_rows][head_dim] fp8 e4m3fn codes, d_scales
 *       [n_rows][head_dim/scale_block] f32 powers of two (metrale
 *       "engram.rs", EngramTables: scales per scale_block values);
 *       head_dim a multiple of 16 up to 1024, scale_block a multiple of 16
 *       dividing head_dim. */
typedef struct engram_table {
    int32_t fmt;
    int32_t head_dim;
    int32_t scale_block;
    int32_t reserved;
    int64_t n_rows;
    const uint8_t *d_data;
    const float *d_scales;
} engram_table;

/* Tables larger than device memory can stay in host memory (atlascybernetics
 * "engram_v41.rs": the pages read each step's 84-byte rows on the host, from
 * checkpoint shards, with EngramRowReader).  Given a pointer into pinned host
 * memory (hipHostMalloc, or a framework's pinned allocation), stores in
 * *device the address under which the kernels read it; engram_table.d_data
 * and d_scales may be such addresses.  A decode step reads only its cols rows
 * a layer, so it pays the link's read latency (a few microseconds a launch);
 * a long prefill's gather becomes bound by the link's rate for small reads.
 *   ENGRAM_E_ARG for NULL pointers or memory the device cannot map (not
 *   pinned); nothing is allocated or copied. */
int32_t engram_map_host(const void *host, const void **device);

/* rows[t*cols + c] = dequant(table row d_row_ids[t*id_stride + c]) as bf16
 * (atlascybernetics "engram_v41.rs", rows_from_q2k and layer_row_ids;
 * metrale "engram.rs", regen_table and embed_rows).  Q2_K: y = d*scale*q -
 * dmin*min rounded once to bf16; e4m3: y = bf16(e4m3 value * block scale).
 *   d_row_ids  ids of token t at d_row_ids + t*id_stride (id_stride >= cols;
 *              for layer l of an engram_hash output pass
 *              d_row_ids + l*cols and id_stride = n_layers*cols);
 *   d_rows     [T*cols][head_dim] bf16 output, i.e. [T][cols*head_dim];
 *   d_err      nullable; an id outside [0, n_rows) sets ENGRAM_DEVERR_ROW and
 *              its row is written as zeros. */
int32_t engram_gather_dequant(const engram_table *table, const int64_t *d_row_ids, int64_t T,
                              int32_t cols, int64_t id_stride, uint16_t *d_rows,
                              int32_t *d_err, void *stream);

/* ------------------------------------------------------------- projection */

/* y[t][n] = bf16( sum_k x[t][k] * w[n][k] ) with f32 accumulation
 * (metrale "engram.rs", linear_bf16; atlascybernetics "engram_v41.rs",
 * module doc stage 3: [tokens, cols*head_dim] x wkv^T -> [tokens,
 * dim*(hc+1)]).  A bandwidth-bound GEMV serves T = 1 and 2 <= T <= 4 (the
 * tokens in one pass over the weights; each token's outputs then equal those
 * of a one-token call bit for bit), an MFMA GEMM laid out as a weight stream
 * 5 <= T <= 128 (K a multiple of 1024), the tiled MFMA GEMM larger T.
 *   d_x [T][K], d_w [N][K], d_y [T][N], all bf16; K a multiple of 64. */
int32_t engram_project(const uint16_t *d_x, const uint16_t *d_w, uint16_t *d_y, int64_t T,
                       int64_t K, int64_t N, void *stream);

/* The same projection for one token with the weight matrix given as Q2_K
 * blocks, as the GGUF ships wkv (atlascybernetics "engram_v41.rs",
 * EngramLayerWeights::wkv_q2k and EngramV41's single-token projection over
 * the raw blocks: 84 bytes per 256 weights instead of 512).  Weight k of
 * output row n is value k%256 of block k/256 of that row, decoded as a table
 * row is (bf16(d*scale*q - dmin*min)); the sum is f32, rounded once to bf16.
 * Results equal engram_project's at one token over the bf16 expansion
 * (engram_dequant_q2k) bit for bit: both add the products in the same order
 * (the pages' byte-identical results).
 *   d_x [T][K] bf16 (16-byte aligned), d_wkv_q2k [N][K/256][84] (4-byte
 *   aligned), d_y [T][N] bf16; T in 0..1 (more tokens: ENGRAM_E_UNSUPPORTED,
 *   use engram_project); K a multiple of 256 up to 8192. */
int32_t engram_project_q2k(const uint16_t *d_x, const uint8_t *d_wkv_q2k, uint16_t *d_y,
                           int64_t T, int64_t K, int64_t N, void *stream);

/* Blocks 0..n_blocks-1 of a Q2_K array -> bf16 [n_blocks][256], each decoded
 * as a table row (atlascybernetics "engram_v41.rs", the dequant_q2_k_to_bf16
 * kernel EngramV41 holds): the bf16 expansion of a weight matrix shipped as
 * Q2_K blocks, for the many-token GEMM.  d_blocks 4-byte, d_out 16-byte
 * aligned. */
int32_t engram_dequant_q2k(const uint8_t *d_blocks, int64_t n_blocks, uint16_t *d_out,
                           void *stream);

/* ------------------------------------------------------------------- gate */

/* qk[i] = f32(q[i]) * f32(k[i]) for n values (atlascybernetics
 * "engram_v41.rs", EngramV41::upload_qk): the gate's [hc][dim] weight. */
int32_t engram_qk_product(const uint16_t *d_q, const uint16_t *d_k, float *d_qk, int64_t n,
                          void *stream);

/* In place on the FP32 highway h [T][hc][dim] (metrale "engram.rs",
 * gate_and_add; atlascybernetics "engram_v41.rs", module doc stage 4): for
 * each token t and stream c, with key = kv[t][c*dim ..], value =
 * kv[t][hc*dim ..]:
 *   s    = (sum h*qk*key) / sqrt(sum h^2/dim + eps) / sqrt(sum key^2/dim + eps)
 *          / sqrt(dim)
 *   gate = sigmoid(sign(s) * sqrt(max(|s|, 1e-6)))
 *   h   += gate * value          (kept in f32)
 *   d_kv [T][dim*(hc+1)] bf16, d_qk [hc][dim] f32; hc in 1..4 (EngramV41::new),
 *   dim a multiple of 256. */
int32_t engram_gate_apply(float *d_h, const uint16_t *d_kv, const float *d_qk, int64_t T,
                          int32_t hc, int64_t dim, float eps, void *stream);

/* ------------------------------------------- one layer, no caller scratch */

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  One engram
 * layer over T tokens of one sequence, computing what engram_forward
 * computes for layer hash_index of a step at start_pos, with no context and
 * no workspace: the step's row ids, rows and kv live in a static device array
 * of ENGRAM_STATIC_SCRATCH_BYTES inside this library (one per device, held
 * until the process ends), and the call allocates nothing.  The caller
 * passes the inputs (hash tables, the layer's table, wkv [dim*(hc+1)]
 * [cols*head_dim] bf16, qk [hc][dim] f32, ids [T] int32), the sequence's
 * history [max_seq] int64 (read before start_pos, written at start_pos ..
 * start_pos+T-1, as engram_hash does) and the highway h [T][hc][dim] f32,
 * gated in place.  d_err nullable, as for engram_hash / engram_gather_dequant.
 *   The scratch must hold T*n_layers*cols*8 + T*cols*head_dim*2 +
 *   T*dim*(hc+1)*2 bytes (each part rounded up to 256): ENGRAM_E_RANGE
 *   otherwise (at 2 layers of 24 columns, head_dim 256, dim 4096, hc 4: up to
 *   625 tokens).
 *   Every call on a device shares that device's scratch and leaves its
 *   contents there: calls that overlap on one device (another stream,
 *   another thread) race.  One token (head_dim 256, at most 32 columns) runs
 *   hash, gather and projection as one kernel, then the gate, as
 *   engram_forward's decode step does; more tokens run the staged kernels.
 *   Checks as engram_forward's; T = 0 is a no-op. */
#define ENGRAM_STATIC_SCRATCH_BYTES (32 << 20)
int32_t engram_layer_static(const engram_hash_tables *tables, int32_t hash_index,
                            const engram_table *table, const uint16_t *d_wkv, const float *d_qk,
                            int32_t hc, int64_t dim, float eps, const int32_t *d_ids, int64_t T,
                            int64_t start_pos, int64_t *d_history, int64_t max_seq, float *d_h,
                            int32_t *d_err, void *stream);

/* --------------------------------------------------- stateful engram layer */

/* The engram of one sequence, or of `batch` sequences that advance together
 * (metrale "engram.rs", NgramHashState's batch rows): hash tables, up to
 * n_layers registered layers and a caller-owned workspace holding the hasher
 * history of every sequence, the step's row ids, the dequantised rows, the
 * projection output and the device error word (atlascybernetics
 * "engram_v41.rs", EngramV41 and EngramHasher; "deepseek_v41_layer.rs",
 * V41Runtime::step_hashes).  A step's tokens of all sequences go through one
 * pass over each layer's weights.  Calls on one context must not overlap. */
typedef struct engram_ctx engram_ctx;

/* Geometry: hc in 1..4; dim a multiple of 256 up to 2^20; head_dim of every
 * layer's table; eps of the gate; batch sequences (0 or 1: one; up to 4096);
 * max_tokens per sequence per call; max_seq positions of history per
 * sequence (batch * max_seq at most 2^40; batch * max_tokens * cols *
 * head_dim below 2^31, the projection's operand limit).
 * hash.multipliers/primes/offsets are copied at create. */
typedef struct engram_config {
    int32_t hc;
    int32_t head_dim;
    int64_t dim;
    float eps;
    int32_t batch;          /* sequences (0 = 1); they advance together */
    int64_t max_tokens;     /* tokens per sequence per call */
    int64_t max_seq;
    engram_hash_tables hash;
} engram_config;

/* Device bytes the workspace needs for cfg (0 if cfg is invalid). */
size_t engram_workspace_bytes(const engram_config *cfg);

/* Validates cfg, carves d_workspace (>= engram_workspace_bytes(cfg) bytes,
 * 256-byte aligned, caller-owned, must outlive the context) and returns a
 * host-side context in *out.  Call engram_reset before the first forward. */
int32_t engram_ctx_create(const engram_config *cfg, void *d_workspace, size_t workspace_bytes,
                          engram_ctx **out);

/* Registers layer hash_index (0 .. n_layers-1): its table, wkv [dim*(hc+1)]
 * [cols*head_dim] bf16 and qk [hc][dim] f32 (atlascybernetics
 * "engram_v41.rs", add_layer and EngramLayerWeights).  Refuses a table with
 * fewer rows than max(offset + prime) of that layer, so every hashed id is a
 * valid row.  Re-registering replaces the layer's pointers (and drops its
 * Q2_K wkv). */
int32_t engram_ctx_add_layer(engram_ctx *ctx, int32_t hash_index, const engram_table *table,
                             const uint16_t *d_wkv, const float *d_qk);

/* Registers the layer's wkv also as Q2_K blocks [dim*(hc+1)][K/256][84]
 * (atlascybernetics "engram_v41.rs", EngramLayerWeights::wkv_q2k; NULL drops
 * them): every one-token forward of the layer then projects from these
 * blocks (engram_project_q2k's arithmetic) and the bf16 wkv serves T > 1.
 * The layer must be registered; K = cols*head_dim a multiple of 256 up to
 * 8192; blocks 4-byte aligned and caller-owned. */
int32_t engram_ctx_set_wkv_q2k(engram_ctx *ctx, int32_t hash_index, const uint8_t *d_wkv_q2k);

/* History := 0, position := 0, device error word := 0, no step open. */
int32_t engram_reset(engram_ctx *ctx, void *stream);

/* Resume a sequence: the history rows in the workspace (engram_ctx_buffers'
 * layout: [batch][max_seq] int64 at the workspace's start) hold the
 * compressed ids of the first pos tokens, restored by the caller (say from a
 * checkpoint of an earlier context's workspace); the next step hashes at pos.
 * The hasher's state is exactly those entries and the position, so the steps
 * that follow equal an uninterrupted run's.  No step is open afterwards; the
 * device error word is cleared (on `stream`); in graph mode the device
 * position is set too.  pos in 0..max_seq (ENGRAM_E_RANGE otherwise). */
int32_t engram_ctx_set_position(engram_ctx *ctx, int64_t pos, void *stream);

/* One engram layer over the next T tokens of every sequence, gating d_h
 * [batch][T][hc][dim] in place.  hash_index 0 opens a step: it hashes the
 * tokens d_ids [batch][T] (sequence b's in row b, against its own history)
 * for every layer at the current position and advances the position by T
 * (the look-back carries across prefill chunks and decode steps).  hash_index > 0 reuses the open step's row ids (d_ids is ignored
 * and may be NULL) and must pass the same T (atlascybernetics
 * "deepseek_v41_layer.rs", V41Runtime::step_hashes: computed by the first
 * engram layer, reused by the second).
 * Refuses T > max_tokens or position + T > max_seq (ENGRAM_E_RANGE),
 * an unregistered layer, a call with no open step / another T, or a context
 * that has not been through engram_reset (ENGRAM_E_STATE).  Calls on one
 * context must not overlap (one stream, or ordered streams): they share its
 * workspace. */
int32_t engram_forward(engram_ctx *ctx, int32_t hash_index, const int32_t *d_ids, int64_t T,
                       float *d_h, void *stream);

/* Synchronises `stream`, reads the device error word and returns
 * ENGRAM_E_DEVICE if it is set (the word keeps its bits until engram_reset). */
int32_t engram_check(engram_ctx *ctx, void *stream);

/* Current position (tokens hashed since the last reset); -1 for NULL. */
int64_t engram_position(const engram_ctx *ctx);

/* Device views into the workspace (any output may be NULL): the open step's
 * row ids [batch*T][n_layers][cols] int64, the last forward's rows
 * [batch*T][cols*head_dim] bf16 and kv [batch*T][dim*(hc+1)] bf16 (token b*T+t
 * is token t of sequence b).  Valid until the next forward. */
int32_t engram_ctx_buffers(const engram_ctx *ctx, int64_t **d_row_ids, uint16_t **d_rows,
                           uint16_t **d_kv, int32_t **d_err);

/* One decode token of a one-sequence context (T = 1, head_dim 256, at most
 * 32 columns) runs hash,
 * gather + dequant and the projection of a layer as one kernel, then the gate
 * (enabled by default).  Results and workspace contents (row ids of every
 * layer, rows, kv, history, highway) are bit-identical to the staged path's.
 * enable = 0 selects the staged kernels for every call. */
int32_t engram_ctx_set_fused_decode(engram_ctx *ctx, int32_t enable);

/* Stage timing with HIP events recorded on the forward's stream, around each
 * kernel of every engram_forward while enabled (stages: 0 hash, 1 gather,
 * 2 projection -- the one-launch decode kernel counts here --, 3 gate).  engram_ctx_timing synchronises the events and
 * returns, per stage, the summed milliseconds and the number of launches
 * since timing was enabled; it then clears them. */
int32_t engram_ctx_set_timing(engram_ctx *ctx, int32_t enable);
int32_t engram_ctx_timing(engram_ctx *ctx, double *ms_per_stage /*[4]*/,
                          int64_t *launches_per_stage /*[4]*/);

/* Graph mode, for replaying captured decode steps (atlascybernetics
 * "spark_model/layers/deepseek_v41_layer.rs", GraphMode and the per-layer
 * graphs: a decode step's launches are captured once with fixed pointers and
 * replayed, and an oracle mode compares replay with eager execution bit for
 * bit).  While enabled, each
 * engram_forward must be a single-token step of the one-launch decode kernels
 * (T = 1 and the conditions of engram_ctx_set_fused_decode, or 2-4 sequences
 * with at most 64 hash slots; anything else: ENGRAM_E_STATE), and its kernels
 * read the step's position from a device word in the workspace instead of
 * taking it from the host: the gate of the last hash index moves the word on
 * by one, so the same launches, captured into a hipGraph on `stream`, replay
 * successive steps.  The caller writes each step's token ids into the d_ids
 * buffer it captured (and its highway into d_h) before a replay.  The host
 * no longer checks the position: a step at max_seq or beyond sets
 * ENGRAM_DEVERR_POSITION and writes no history; while that bit is set (until
 * engram_reset or engram_ctx_set_position clears the error word) every gate
 * of graph mode leaves its highway untouched, and the step's row ids, rows
 * and kv are unspecified.  Stage timing must be off (its events cannot be
 * captured).
 *   enable = 1: enqueues the store of the host's position into the device
 *   word on `stream` (nothing if already enabled).  enable = 0: synchronises
 *   `stream` and reads the device word back as the host's position
 *   (engram_position).  ENGRAM_E_STATE before the first engram_reset, with
 *   timing on, or with the one-launch decode kernels off. */
int32_t engram_ctx_set_graph_mode(engram_ctx *ctx, int32_t enable, void *stream);

/* Frees the context's host bookkeeping and its timing events (NULL: no-op).
 * The workspace stays the caller's; work already enqueued on it is not
 * waited for, so destroy a context only after its stream has finished. */
void engram_ctx_destroy(engram_ctx *ctx);

/* ------------------------------------------------------------ measurement */

/* Not a step of the method: the yardstick the streaming projections are
 * measured against.  Reads d_src [bytes] once, in the decode projection's
 * access pattern (each of 8192 wavefronts streams 12 KiB rows as 1 KiB
 * non-temporal loads, the next row in flight while one is consumed),
 * XOR-folds every 32-bit word and stores wavefront w's fold in d_sink[w]
 * (d_sink [ENGRAM_STREAM_SINK_WORDS]): the XOR of the sink words is the XOR
 * of every word of d_src.  Its rate over a buffer resident in HBM is the
 * practical ceiling of a read stream on the device.
 *   bytes: a positive multiple of ENGRAM_STREAM_ROW_BYTES; d_src 16-byte
 *   aligned, d_sink 4-byte aligned (ENGRAM_E_ARG otherwise). */
#define ENGRAM_STREAM_ROW_BYTES 12288
#define ENGRAM_STREAM_SINK_WORDS 8192
int32_t engram_stream_read(const void *d_src, int64_t bytes, uint32_t *d_sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
