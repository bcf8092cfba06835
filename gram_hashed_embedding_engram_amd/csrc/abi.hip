// The C ABI (include/engram.h): host-side validation, the stateful context
// and dispatch to the kernels.  Every check runs before any launch, so a
// refused call enqueues nothing (metrale "engram_v41" module index,
// invariants: refusals happen before any copy or launch).
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace engram {

static thread_local std::string g_last_error;

int32_t fail(int32_t code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int32_t launch_status(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(ENGRAM_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return ENGRAM_OK;
}

constexpr int kMaxDevices = 64;

int device_cus()
{
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

#define CHECK(cond, code, ...)                                                               \
    do {                                                                                     \
        if (!(cond))                                                                         \
            return fail(code, __VA_ARGS__);                                                  \
    } while (0)

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Positions start_pos .. start_pos+T-1 lie inside a history of max_seq
// entries (all three non-negative; written so that no sum can overflow).
bool fits_history(int64_t start_pos, int64_t T, int64_t max_seq)
{
    return start_pos <= max_seq && T <= max_seq - start_pos;
}

constexpr int64_t kMaxElems = (int64_t)1 << 31;
constexpr int32_t kMaxBatch = 4096;         // sequences per context
constexpr int64_t kMaxSeq = (int64_t)1 << 40; // history entries per context

// Hash tables -> kernel constants (atlascybernetics "engram_v41.rs",
// EngramHashTables::from_flat: geometry and array checks).
int32_t make_consts(const engram_hash_tables *t, HashConsts *c)
{
    CHECK(t, ENGRAM_E_ARG, "engram hash tables: NULL");
    CHECK(t->n_layers > 0 && t->max_ngram >= 2 && t->n_heads > 0, ENGRAM_E_ARG,
          "engram geometry: %d layers, ngram %d, heads %d", t->n_layers, t->max_ngram,
          t->n_heads);
    CHECK(t->n_layers <= ENGRAM_MAX_LAYERS && t->max_ngram <= ENGRAM_MAX_NGRAM, ENGRAM_E_UNSUPPORTED,
          "engram geometry: %d layers (max %d), ngram %d (max %d)", t->n_layers,
          ENGRAM_MAX_LAYERS, t->max_ngram, ENGRAM_MAX_NGRAM);
    const int64_t cols = (int64_t)(t->max_ngram - 1) * t->n_heads;
    CHECK(cols * t->n_layers <= ENGRAM_MAX_SLOTS, ENGRAM_E_UNSUPPORTED,
          "engram geometry: %lld hash slots exceed %d", (long long)(cols * t->n_layers),
          ENGRAM_MAX_SLOTS);
    CHECK(t->vocab > 0 && t->d_token_map, ENGRAM_E_ARG, "engram token_map: vocab %lld, ptr %p",
          (long long)t->vocab, (const void *)t->d_token_map);
    CHECK(t->multipliers && t->primes && t->offsets, ENGRAM_E_ARG,
          "engram hash constants: NULL array");
    std::memset(c, 0, sizeof *c);
    c->nl = t->n_layers;
    c->ng = t->max_ngram;
    c->nh = t->n_heads;
    c->cols = (int32_t)cols;
    c->vocab = t->vocab;
    c->pad_id = t->pad_id;
    for (int64_t i = 0; i < (int64_t)t->n_layers * t->max_ngram; i++) {
        CHECK(t->multipliers[i] >= 0, ENGRAM_E_ARG,
              "engram.multipliers[%lld] = %lld is negative (the tables hold values that fit i64)",
              (long long)i, (long long)t->multipliers[i]);
        c->mult[i] = t->multipliers[i];
    }
    for (int64_t i = 0; i < t->n_layers * cols; i++) {
        CHECK(t->primes[i] > 0, ENGRAM_E_ARG, "engram.primes[%lld] = %lld must be positive",
              (long long)i, (long long)t->primes[i]);
        CHECK(t->offsets[i] >= 0 && t->offsets[i] <= ((int64_t)1 << 62) - t->primes[i],
              ENGRAM_E_ARG, "engram.offsets[%lld] = %lld out of range", (long long)i,
              (long long)t->offsets[i]);
        c->prime[i] = t->primes[i];
        c->offset[i] = t->offsets[i];
    }
    return ENGRAM_OK;
}

int32_t check_table(const engram_table *tab)
{
    CHECK(tab, ENGRAM_E_ARG, "engram table: NULL");
    CHECK(tab->n_rows > 0 && tab->d_data, ENGRAM_E_ARG, "engram table: %lld rows, data %p",
          (long long)tab->n_rows, (const void *)tab->d_data);
    if (tab->fmt == ENGRAM_FMT_Q2K) {
        CHECK(tab->head_dim == 256, ENGRAM_E_UNSUPPORTED,
              "engram Q2_K table: a row is one 256-value block, so head_dim is 256 (got %d)",
              tab->head_dim);
        CHECK(aligned(tab->d_data, 4), ENGRAM_E_ARG, "engram Q2_K table must be 4-byte aligned");
    } else if (tab->fmt == ENGRAM_FMT_E4M3) {
        CHECK(tab->head_dim >= 16 && tab->head_dim <= 1024 && tab->head_dim % 16 == 0,
              ENGRAM_E_UNSUPPORTED, "engram e4m3 head_dim %d: a multiple of 16 up to 1024",
              tab->head_dim);
        CHECK(tab->scale_block >= 16 && tab->scale_block % 16 == 0 &&
                  tab->head_dim % tab->scale_block == 0,
              ENGRAM_E_UNSUPPORTED, "engram e4m3 scale_block %d must be a multiple of 16 dividing %d",
              tab->scale_block, tab->head_dim);
        CHECK(tab->d_scales, ENGRAM_E_ARG, "engram e4m3 table: NULL scales");
        CHECK(aligned(tab->d_data, 16) && aligned(tab->d_scales, 4), ENGRAM_E_ARG,
              "engram e4m3 table: codes must be 16-byte and scales 4-byte aligned");
    } else {
        return fail(ENGRAM_E_UNSUPPORTED, "engram table format %d", tab->fmt);
    }
    return ENGRAM_OK;
}

int32_t check_project(const uint16_t *x, const uint16_t *w, const uint16_t *y, int64_t T,
                      int64_t K, int64_t N)
{
    CHECK(T >= 0, ENGRAM_E_ARG, "engram project: T = %lld", (long long)T);
    CHECK(K >= 64 && K % 64 == 0, ENGRAM_E_UNSUPPORTED,
          "engram project: K = %lld must be a positive multiple of 64", (long long)K);
    CHECK(N >= 16 && N % 16 == 0, ENGRAM_E_UNSUPPORTED,
          "engram project: N = %lld must be a positive multiple of 16", (long long)N);
    // the GEMM addresses each operand with 32-bit byte offsets, tile tails
    // (up to 255 rows past the end) included
    CHECK(T < kMaxElems / K - 256 && N < kMaxElems / K - 256 && T * N < ((int64_t)1 << 40),
          ENGRAM_E_UNSUPPORTED, "engram project: operands of %lld x %lld x %lld exceed 2^31 elements",
          (long long)T, (long long)K, (long long)N);
    if (T == 0)
        return ENGRAM_OK;                 // nothing to read or write
    CHECK(x && w && y, ENGRAM_E_ARG, "engram project: NULL pointer");
    CHECK(aligned(x, 16) && aligned(w, 16) && aligned(y, 16), ENGRAM_E_ARG,
          "engram project: x, w, y must be 16-byte aligned");
    return ENGRAM_OK;
}

int32_t dispatch_project(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t T, int64_t K,
                         int64_t N, const Launch &l)
{
    if (T == 0)
        return ENGRAM_OK;
    if (T == 1 && K <= kGemvMaxK)
        return launch_gemv(x, w, y, T, K, N, l);
    if (gemv_multi_fits(T, K))
        return launch_gemv_multi(x, w, y, T, K, N, l);
    if (gemm_small_fits(T, K, N))
        return launch_gemm_small(x, w, y, T, K, N, l);
    if (T <= kGemvMaxT && K <= kGemvMaxK)
        return launch_gemv(x, w, y, T, K, N, l);
    return launch_gemm(x, w, y, T, K, N, l);
}

int32_t check_project_q2k(const uint16_t *x, const uint8_t *w, const uint16_t *y, int64_t T,
                          int64_t K, int64_t N)
{
    CHECK(T >= 0, ENGRAM_E_ARG, "engram project_q2k: T = %lld", (long long)T);
    CHECK(T <= 1, ENGRAM_E_UNSUPPORTED,
          "engram project_q2k: one token per call (T = %lld); more take engram_project",
          (long long)T);
    CHECK(K >= 256 && K % 256 == 0 && K <= kQ2kWkvMaxK, ENGRAM_E_UNSUPPORTED,
          "engram project_q2k: K = %lld must be a multiple of 256 up to %lld", (long long)K,
          (long long)kQ2kWkvMaxK);
    CHECK(N >= 1 && N < ((int64_t)1 << 31), ENGRAM_E_UNSUPPORTED,
          "engram project_q2k: N = %lld", (long long)N);
    if (T == 0)
        return ENGRAM_OK;
    CHECK(x && w && y, ENGRAM_E_ARG, "engram project_q2k: NULL pointer");
    CHECK(aligned(x, 16) && aligned(w, 4) && aligned(y, 2), ENGRAM_E_ARG,
          "engram project_q2k: x must be 16-byte, wkv_q2k 4-byte, y 2-byte aligned");
    return ENGRAM_OK;
}

int32_t check_gate(const float *h, const uint16_t *kv, const float *qk, int64_t T, int32_t hc,
                   int64_t dim, float eps)
{
    CHECK(T >= 0, ENGRAM_E_ARG, "engram gate: T = %lld", (long long)T);
    CHECK(hc >= 1 && hc <= 4, ENGRAM_E_UNSUPPORTED,
          "engram gate: %d hyper-connection streams, 1 to 4 supported", hc);
    CHECK(dim >= 256 && dim % 256 == 0 && dim <= (1 << 20), ENGRAM_E_UNSUPPORTED,
          "engram gate: dim = %lld must be a multiple of 256", (long long)dim);
    CHECK(std::isfinite(eps) && eps >= 0.0f, ENGRAM_E_ARG, "engram gate: eps = %g", (double)eps);
    CHECK(T < ((int64_t)1 << 24) / hc, ENGRAM_E_RANGE, "engram gate: %lld x %d rows exceed 2^24",
          (long long)T, hc);
    if (T == 0)
        return ENGRAM_OK;
    CHECK(h && kv && qk, ENGRAM_E_ARG, "engram gate: NULL pointer");
    CHECK(aligned(h, 16) && aligned(kv, 8) && aligned(qk, 16), ENGRAM_E_ARG,
          "engram gate: h and qk must be 16-byte, kv 8-byte aligned");
    return ENGRAM_OK;
}

}  // namespace
}  // namespace engram

using namespace engram;

// ------------------------------------- scratch of the call that allocates nothing

// engram_layer_static keeps its call's row ids, rows and kv here instead of
// in caller memory: one array per device, resident from the library's load
// until the process ends.  Every call on a device shares that device's copy
// and leaves the last call's contents in it, so calls that overlap on one
// device race.  Host code never passes this name to a kernel (on the host it
// is a stand-in, not a device address): it passes the address that
// hipGetSymbolAddress returned for the current device.
static __device__ __align__(256) uint8_t scratch[ENGRAM_STATIC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];     // per device, looked up once

// The current device's address of `scratch`, looked up on the first call on
// that device with that device current, then reused.
int32_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(ENGRAM_E_HIP, "engram layer_static: hipGetDevice: %s", hipGetErrorString(e));
    }
    CHECK(dev >= 0 && dev < kMaxDevices, ENGRAM_E_HIP, "engram layer_static: device %d", dev);
    std::lock_guard<std::mutex> guard(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(ENGRAM_E_HIP, "engram layer_static: hipGetSymbolAddress(scratch): %s",
                        hipGetErrorString(e));
        }
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return ENGRAM_OK;
}

}  // namespace

// ------------------------------------------------------------ the context

struct TimingRec {
    int stage;
    hipEvent_t a, b;
};

struct engram_ctx {
    engram_config cfg;
    HashConsts consts;
    int32_t nl = 0, cols = 0;
    int64_t kv_width = 0;
    // workspace views
    int64_t *history = nullptr, *row_ids = nullptr;
    uint16_t *rows = nullptr, *kv = nullptr;
    int32_t *err = nullptr;
    struct Layer {
        bool set = false;
        engram_table tab{};
        const uint16_t *wkv = nullptr;
        const uint8_t *wkv_q2k = nullptr;   // one-token projections read these if set
        const float *qk = nullptr;
    } layers[ENGRAM_MAX_LAYERS];
    int64_t pos = 0;
    bool step_open = false;
    int64_t step_T = 0;
    int64_t step_start = 0;
    bool fused_decode = true;
    bool was_reset = false;
    bool timing = false;
    // graph mode: one-token decode steps read their position from *d_pos
    // (in the workspace's error slot), which the step's last gate advances
    bool graph_mode = false;
    int64_t *d_pos = nullptr;
    std::vector<TimingRec> recs;
    std::vector<hipEvent_t> pool;
};

namespace {

struct Carve {
    size_t history, row_ids, rows, kv, err, total;
};

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

// sequences of a context (0 in the config means one)
int64_t batch_of(const engram_config *cfg) { return cfg->batch > 0 ? cfg->batch : 1; }

bool carve(const engram_config *cfg, Carve *c)
{
    // every field bounded first, so that no size below overflows
    if (!cfg || cfg->max_tokens <= 0 || cfg->max_seq <= 0 || cfg->dim <= 0 || cfg->hc <= 0 ||
        cfg->head_dim <= 0 || cfg->hash.n_layers <= 0 || cfg->hash.max_ngram < 2 ||
        cfg->hash.n_heads <= 0 || cfg->batch < 0 || cfg->batch > kMaxBatch)
        return false;
    if (cfg->max_tokens > kMaxElems || cfg->max_seq > kMaxSeq || cfg->dim > (1 << 20) ||
        cfg->hc > 4 || cfg->head_dim > 1024 || cfg->hash.n_layers > ENGRAM_MAX_LAYERS ||
        cfg->hash.max_ngram > ENGRAM_MAX_NGRAM || cfg->hash.n_heads > ENGRAM_MAX_SLOTS ||
        batch_of(cfg) * cfg->max_tokens > kMaxElems || batch_of(cfg) * cfg->max_seq > kMaxSeq)
        return false;
    const int64_t cols = (int64_t)(cfg->hash.max_ngram - 1) * cfg->hash.n_heads;
    const int64_t B = batch_of(cfg), M = B * cfg->max_tokens;
    size_t off = 0;
    c->history = off;
    off += round256(sizeof(int64_t) * (size_t)(B * cfg->max_seq));
    c->row_ids = off;
    off += round256(sizeof(int64_t) * (size_t)(M * cfg->hash.n_layers * cols));
    c->rows = off;
    off += round256(2 * (size_t)(M * cols * cfg->head_dim));
    c->kv = off;
    off += round256(2 * (size_t)(M * cfg->dim * (cfg->hc + 1)));
    c->err = off;
    off += 256;
    c->total = off;
    return true;
}

// The step that layer 0 just hashed (at ctx->step_start, T tokens a
// sequence) is open for the other layers; the position moves past it.
void open_step(engram_ctx *ctx, int64_t T)
{
    if (!ctx->graph_mode)       // (graph mode: the position moves on the device)
        ctx->pos = ctx->step_start + T;
    ctx->step_open = true;
    ctx->step_T = T;
}

hipEvent_t take_event(engram_ctx *ctx)
{
    if (!ctx->pool.empty()) {
        hipEvent_t e = ctx->pool.back();
        ctx->pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}

// Runs one stage's launch on stream s; with timing on, the runtime records a
// pair of events with the stage's kernel dispatch itself.
template <class F>
int32_t staged(engram_ctx *ctx, int stage, hipStream_t s, F &&launch)
{
    Launch l;
    l.stream = s;
    if (!ctx->timing)
        return launch(l);
    l.start = take_event(ctx);
    l.stop = take_event(ctx);
    if (!l.start || !l.stop)
        return fail(ENGRAM_E_HIP, "engram timing: hipEventCreate failed");
    const int32_t rc = launch(l);
    ctx->recs.push_back({stage, l.start, l.stop});
    return rc;
}

Launch on(void *stream)
{
    Launch l;
    l.stream = as_stream(stream);
    return l;
}

}  // namespace

// ------------------------------------------------------------ entry points

extern "C" {

const char *engram_last_error(void) { return g_last_error.c_str(); }

int32_t engram_abi_version(void) { return ENGRAM_ABI_VERSION; }

int32_t engram_map_host(const void *host, const void **device)
{
    CHECK(host && device, ENGRAM_E_ARG, "engram map_host: NULL pointer");
    void *d = nullptr;
    const hipError_t e = hipHostGetDevicePointer(&d, const_cast<void *>(host), 0);
    if (e != hipSuccess)
        (void)hipGetLastError();   // a refused pointer leaves no error for the next call
    CHECK(e == hipSuccess && d, ENGRAM_E_ARG,
          "engram map_host: %p is not pinned host memory the device can map (%s)", host,
          hipGetErrorString(e));
    *device = d;
    return ENGRAM_OK;
}

int32_t engram_hash_batch(const engram_hash_tables *tables, const int32_t *d_ids, int64_t B,
                          int64_t T, int64_t start_pos, int64_t *d_history, int64_t max_seq,
                          int64_t *d_row_ids, int32_t *d_err, void *stream)
{
    HashConsts c;
    int32_t rc = make_consts(tables, &c);
    if (rc != ENGRAM_OK)
        return rc;
    CHECK(B >= 0 && T >= 0 && start_pos >= 0 && max_seq >= 0, ENGRAM_E_ARG,
          "engram hash: B %lld, T %lld, start_pos %lld, max_seq %lld", (long long)B,
          (long long)T, (long long)start_pos, (long long)max_seq);
    CHECK(fits_history(start_pos, T, max_seq), ENGRAM_E_RANGE,
          "engram hasher: %lld positions, %lld tokens from position %lld", (long long)max_seq,
          (long long)T, (long long)start_pos);
    CHECK(B == 0 || T == 0 || B <= ((int64_t)1 << 40) / T, ENGRAM_E_RANGE,
          "engram hash: %lld x %lld tokens", (long long)B, (long long)T);
    if (B == 0 || T == 0)
        return ENGRAM_OK;
    CHECK(d_ids && d_history && d_row_ids, ENGRAM_E_ARG, "engram hash: NULL pointer");
    return launch_hash(c, tables->d_token_map, d_ids, B, T, start_pos, d_history, max_seq,
                       d_row_ids, d_err, on(stream));
}

int32_t engram_hash(const engram_hash_tables *tables, const int32_t *d_ids, int64_t T,
                    int64_t start_pos, int64_t *d_history, int64_t max_seq, int64_t *d_row_ids,
                    int32_t *d_err, void *stream)
{
    return engram_hash_batch(tables, d_ids, 1, T, start_pos, d_history, max_seq, d_row_ids, d_err,
                             stream);
}

int32_t engram_gather_dequant(const engram_table *table, const int64_t *d_row_ids, int64_t T,
                              int32_t cols, int64_t id_stride, uint16_t *d_rows, int32_t *d_err,
                              void *stream)
{
    int32_t rc = check_table(table);
    if (rc != ENGRAM_OK)
        return rc;
    CHECK(T >= 0 && cols >= 1 && id_stride >= cols, ENGRAM_E_ARG,
          "engram gather: T %lld, cols %d, id_stride %lld", (long long)T, cols,
          (long long)id_stride);
    CHECK(id_stride <= ENGRAM_MAX_SLOTS && T <= ((int64_t)1 << 40) / id_stride, ENGRAM_E_RANGE,
          "engram gather: %lld tokens of %lld ids", (long long)T, (long long)id_stride);
    if (T == 0)
        return ENGRAM_OK;
    CHECK(d_row_ids && d_rows, ENGRAM_E_ARG, "engram gather: NULL pointer");
    CHECK(aligned(d_rows, 16) && aligned(d_row_ids, 8), ENGRAM_E_ARG,
          "engram gather: rows must be 16-byte, ids 8-byte aligned");
    return launch_gather(*table, d_row_ids, T, cols, id_stride, d_rows, d_err, on(stream));
}

int32_t engram_project(const uint16_t *d_x, const uint16_t *d_w, uint16_t *d_y, int64_t T,
                       int64_t K, int64_t N, void *stream)
{
    int32_t rc = check_project(d_x, d_w, d_y, T, K, N);
    if (rc != ENGRAM_OK)
        return rc;
    return dispatch_project(d_x, d_w, d_y, T, K, N, on(stream));
}

int32_t engram_project_q2k(const uint16_t *d_x, const uint8_t *d_wkv_q2k, uint16_t *d_y,
                           int64_t T, int64_t K, int64_t N, void *stream)
{
    int32_t rc = check_project_q2k(d_x, d_wkv_q2k, d_y, T, K, N);
    if (rc != ENGRAM_OK || T == 0)
        return rc;
    return launch_gemv_q2k(d_x, d_wkv_q2k, d_y, K, N, on(stream));
}

int32_t engram_dequant_q2k(const uint8_t *d_blocks, int64_t n_blocks, uint16_t *d_out,
                           void *stream)
{
    CHECK(n_blocks >= 0 && n_blocks < ((int64_t)1 << 40), ENGRAM_E_ARG,
          "engram dequant_q2k: %lld blocks", (long long)n_blocks);
    if (n_blocks == 0)
        return ENGRAM_OK;
    CHECK(d_blocks && d_out, ENGRAM_E_ARG, "engram dequant_q2k: NULL pointer");
    CHECK(aligned(d_blocks, 4) && aligned(d_out, 16), ENGRAM_E_ARG,
          "engram dequant_q2k: blocks must be 4-byte, out 16-byte aligned");
    return launch_dequant_q2k(d_blocks, n_blocks, d_out, on(stream));
}

int32_t engram_qk_product(const uint16_t *d_q, const uint16_t *d_k, float *d_qk, int64_t n,
                          void *stream)
{
    CHECK(n >= 0, ENGRAM_E_ARG, "engram qk: n = %lld", (long long)n);
    if (n == 0)
        return ENGRAM_OK;
    CHECK(d_q && d_k && d_qk, ENGRAM_E_ARG, "engram qk: NULL pointer");
    return launch_qk_product(d_q, d_k, d_qk, n, on(stream));
}

int32_t engram_stream_read(const void *d_src, int64_t bytes, uint32_t *d_sink, void *stream)
{
    CHECK(bytes > 0 && bytes % ENGRAM_STREAM_ROW_BYTES == 0, ENGRAM_E_ARG,
          "engram stream_read: %lld bytes is not a positive multiple of %d", (long long)bytes,
          ENGRAM_STREAM_ROW_BYTES);
    CHECK(d_src && d_sink, ENGRAM_E_ARG, "engram stream_read: NULL pointer");
    CHECK((reinterpret_cast<uintptr_t>(d_src) & 15) == 0 &&
              (reinterpret_cast<uintptr_t>(d_sink) & 3) == 0,
          ENGRAM_E_ARG, "engram stream_read: misaligned buffer");
    return launch_stream_read(d_src, bytes, d_sink, on(stream));
}

int32_t engram_gate_apply(float *d_h, const uint16_t *d_kv, const float *d_qk, int64_t T,
                          int32_t hc, int64_t dim, float eps, void *stream)
{
    int32_t rc = check_gate(d_h, d_kv, d_qk, T, hc, dim, eps);
    if (rc != ENGRAM_OK)
        return rc;
    return launch_gate(d_h, d_kv, d_qk, T, hc, dim, eps, on(stream));
}

int32_t engram_layer_static(const engram_hash_tables *tables, int32_t hash_index,
                            const engram_table *table, const uint16_t *d_wkv, const float *d_qk,
                            int32_t hc, int64_t dim, float eps, const int32_t *d_ids, int64_t T,
                            int64_t start_pos, int64_t *d_history, int64_t max_seq, float *d_h,
                            int32_t *d_err, void *stream)
{
    HashConsts c;
    int32_t rc = make_consts(tables, &c);
    if (rc != ENGRAM_OK)
        return rc;
    CHECK(hash_index >= 0 && hash_index < c.nl, ENGRAM_E_ARG,
          "engram layer_static: hash index %d outside 0..%d", hash_index, c.nl - 1);
    rc = check_table(table);
    if (rc != ENGRAM_OK)
        return rc;
    CHECK(T >= 0 && start_pos >= 0 && max_seq >= 0, ENGRAM_E_ARG,
          "engram layer_static: T %lld, start_pos %lld, max_seq %lld", (long long)T,
          (long long)start_pos, (long long)max_seq);
    CHECK(fits_history(start_pos, T, max_seq), ENGRAM_E_RANGE,
          "engram hasher: %lld positions, %lld tokens from position %lld", (long long)max_seq,
          (long long)T, (long long)start_pos);
    int64_t need_rows = 0;
    for (int col = 0; col < c.cols; col++) {
        const int slot = hash_index * c.cols + col;
        const int64_t top = c.offset[slot] + c.prime[slot];
        need_rows = top > need_rows ? top : need_rows;
    }
    CHECK(table->n_rows >= need_rows, ENGRAM_E_RANGE,
          "engram layer_static: table has %lld rows, the hash reaches row %lld",
          (long long)table->n_rows, (long long)need_rows - 1);
    const int64_t K = (int64_t)c.cols * table->head_dim, N = dim * (hc + 1);
    // sizes (and, for T > 0, pointers) of the projection and the gate; rows
    // and kv live in the 256-byte aligned scratch, so the caller's wkv stands
    // in for them in the pointer checks
    rc = check_gate(d_h, d_wkv, d_qk, T, hc, dim, eps);
    if (rc != ENGRAM_OK)
        return rc;
    rc = check_project(d_wkv, d_wkv, d_wkv, T, K, N);
    if (rc != ENGRAM_OK)
        return rc;
    const size_t off_rows = round256(sizeof(int64_t) * (size_t)(T * c.nl * c.cols));
    const size_t off_kv = off_rows + round256(2 * (size_t)(T * K));
    const size_t need = off_kv + round256(2 * (size_t)(T * N));
    CHECK(need <= (size_t)ENGRAM_STATIC_SCRATCH_BYTES, ENGRAM_E_RANGE,
          "engram layer_static: %lld tokens need %zu bytes of row ids, rows and kv; the static "
          "scratch holds %lld",
          (long long)T, need, (long long)ENGRAM_STATIC_SCRATCH_BYTES);
    if (T == 0)
        return ENGRAM_OK;
    CHECK(d_ids && d_history, ENGRAM_E_ARG, "engram layer_static: NULL ids or history");
    void *base = nullptr;
    rc = scratch_address(&base);
    if (rc != ENGRAM_OK)
        return rc;
    int64_t *row_ids = (int64_t *)base;
    uint16_t *rows = (uint16_t *)((char *)base + off_rows);
    uint16_t *kv = (uint16_t *)((char *)base + off_kv);
    const Launch l = on(stream);
    if (T == 1 && table->head_dim == 256 && c.cols <= kDecodeMaxCols) {
        // one decode token: hash, gather + dequant and projection in one launch
        const DecodePos dpos{start_pos, nullptr, max_seq};
        rc = launch_decode(c, tables->d_token_map, d_ids, dpos, d_history, hash_index, true,
                           *table, d_wkv, nullptr, kv, N, row_ids, rows, d_err, l);
    } else {
        rc = launch_hash(c, tables->d_token_map, d_ids, 1, T, start_pos, d_history, max_seq,
                         row_ids, d_err, l);
        if (rc == ENGRAM_OK)
            rc = launch_gather(*table, row_ids + (int64_t)hash_index * c.cols, T, c.cols,
                               (int64_t)c.nl * c.cols, rows, d_err, l);
        if (rc == ENGRAM_OK)
            rc = dispatch_project(rows, d_wkv, kv, T, K, N, l);
    }
    if (rc == ENGRAM_OK)
        rc = launch_gate(d_h, kv, d_qk, T, hc, dim, eps, l);
    return rc;
}

size_t engram_workspace_bytes(const engram_config *cfg)
{
    Carve c;
    return carve(cfg, &c) ? c.total : 0;
}

int32_t engram_ctx_create(const engram_config *cfg, void *d_workspace, size_t workspace_bytes,
                          engram_ctx **out)
{
    CHECK(cfg && out, ENGRAM_E_ARG, "engram ctx: NULL config or output");
    *out = nullptr;
    HashConsts c;
    int32_t rc = make_consts(&cfg->hash, &c);
    if (rc != ENGRAM_OK)
        return rc;
    CHECK(cfg->hc >= 1 && cfg->hc <= 4, ENGRAM_E_UNSUPPORTED,
          "engram gate: %d hyper-connection streams, 1 to 4 supported", cfg->hc);
    CHECK(cfg->dim >= 256 && cfg->dim % 256 == 0, ENGRAM_E_UNSUPPORTED,
          "engram dim %lld must be a multiple of 256", (long long)cfg->dim);
    CHECK(cfg->head_dim >= 16 && cfg->head_dim % 16 == 0 && cfg->head_dim <= 1024,
          ENGRAM_E_UNSUPPORTED, "engram head_dim %d", cfg->head_dim);
    CHECK(std::isfinite(cfg->eps) && cfg->eps >= 0.0f, ENGRAM_E_ARG, "engram eps %g",
          (double)cfg->eps);
    CHECK(cfg->batch >= 0 && cfg->batch <= kMaxBatch, ENGRAM_E_ARG,
          "engram ctx: batch %d outside 0..%d", cfg->batch, kMaxBatch);
    CHECK(cfg->max_tokens >= 1 && cfg->max_seq >= 1, ENGRAM_E_ARG,
          "engram ctx: max_tokens %lld, max_seq %lld", (long long)cfg->max_tokens,
          (long long)cfg->max_seq);
    CHECK(cfg->max_tokens <= kMaxElems && cfg->max_seq <= kMaxSeq &&
              batch_of(cfg) * cfg->max_seq <= kMaxSeq && cfg->dim <= (1 << 20),
          ENGRAM_E_UNSUPPORTED, "engram ctx: max_tokens %lld, max_seq %lld x %lld, dim %lld",
          (long long)cfg->max_tokens, (long long)batch_of(cfg), (long long)cfg->max_seq,
          (long long)cfg->dim);
    const int64_t K = (int64_t)c.cols * cfg->head_dim, N = cfg->dim * (cfg->hc + 1);
    CHECK(K % 64 == 0, ENGRAM_E_UNSUPPORTED, "engram ctx: cols*head_dim = %lld not a multiple of 64",
          (long long)K);
    CHECK(batch_of(cfg) * cfg->max_tokens < kMaxElems / K - 256 && N < kMaxElems / K - 256,
          ENGRAM_E_UNSUPPORTED,
          "engram ctx: projection operands exceed 2^31 elements");
    Carve cv;
    CHECK(carve(cfg, &cv), ENGRAM_E_UNSUPPORTED, "engram ctx: geometry out of range");
    CHECK(d_workspace && aligned(d_workspace, 256), ENGRAM_E_ARG,
          "engram ctx: workspace must be non-NULL and 256-byte aligned");
    CHECK(workspace_bytes >= cv.total, ENGRAM_E_RANGE, "engram ctx: workspace %zu bytes, %zu needed",
          workspace_bytes, cv.total);
    engram_ctx *ctx = new engram_ctx();
    ctx->cfg = *cfg;
    ctx->cfg.hash.multipliers = ctx->cfg.hash.primes = ctx->cfg.hash.offsets = nullptr;
    ctx->consts = c;
    ctx->nl = c.nl;
    ctx->cols = c.cols;
    ctx->kv_width = N;
    char *ws = (char *)d_workspace;
    ctx->history = (int64_t *)(ws + cv.history);
    ctx->row_ids = (int64_t *)(ws + cv.row_ids);
    ctx->rows = (uint16_t *)(ws + cv.rows);
    ctx->kv = (uint16_t *)(ws + cv.kv);
    ctx->err = (int32_t *)(ws + cv.err);
    ctx->d_pos = (int64_t *)(ws + cv.err + 8);
    *out = ctx;
    return ENGRAM_OK;
}

int32_t engram_ctx_add_layer(engram_ctx *ctx, int32_t hash_index, const engram_table *table,
                             const uint16_t *d_wkv, const float *d_qk)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram add_layer: NULL context");
    CHECK(hash_index >= 0 && hash_index < ctx->nl, ENGRAM_E_ARG,
          "engram add_layer: hash index %d outside 0..%d", hash_index, ctx->nl - 1);
    int32_t rc = check_table(table);
    if (rc != ENGRAM_OK)
        return rc;
    CHECK(table->head_dim == ctx->cfg.head_dim, ENGRAM_E_ARG,
          "engram add_layer: table head_dim %d, context %d", table->head_dim, ctx->cfg.head_dim);
    int64_t need = 0;
    for (int c = 0; c < ctx->cols; c++) {
        const int slot = hash_index * ctx->cols + c;
        const int64_t top = ctx->consts.offset[slot] + ctx->consts.prime[slot];
        need = top > need ? top : need;
    }
    CHECK(table->n_rows >= need, ENGRAM_E_RANGE,
          "engram add_layer: table has %lld rows, the hash reaches row %lld",
          (long long)table->n_rows, (long long)need - 1);
    CHECK(d_wkv && d_qk && aligned(d_wkv, 16) && aligned(d_qk, 16), ENGRAM_E_ARG,
          "engram add_layer: wkv and qk must be non-NULL and 16-byte aligned");
    engram_ctx::Layer &L = ctx->layers[hash_index];
    L.set = true;
    L.tab = *table;
    L.wkv = d_wkv;
    L.wkv_q2k = nullptr;
    L.qk = d_qk;
    return ENGRAM_OK;
}

int32_t engram_ctx_set_wkv_q2k(engram_ctx *ctx, int32_t hash_index, const uint8_t *d_wkv_q2k)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram set_wkv_q2k: NULL context");
    CHECK(hash_index >= 0 && hash_index < ctx->nl, ENGRAM_E_ARG,
          "engram set_wkv_q2k: hash index %d outside 0..%d", hash_index, ctx->nl - 1);
    engram_ctx::Layer &L = ctx->layers[hash_index];
    CHECK(L.set, ENGRAM_E_STATE, "engram set_wkv_q2k: layer %d has no weights", hash_index);
    if (d_wkv_q2k) {
        const int64_t K = (int64_t)ctx->cols * ctx->cfg.head_dim;
        CHECK(K % 256 == 0 && K <= kQ2kWkvMaxK, ENGRAM_E_UNSUPPORTED,
              "engram set_wkv_q2k: K = %lld must be a multiple of 256 up to %lld", (long long)K,
              (long long)kQ2kWkvMaxK);
        CHECK(aligned(d_wkv_q2k, 4), ENGRAM_E_ARG, "engram set_wkv_q2k: blocks must be 4-byte aligned");
    }
    L.wkv_q2k = d_wkv_q2k;
    return ENGRAM_OK;
}

int32_t engram_reset(engram_ctx *ctx, void *stream)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram reset: NULL context");
    const Launch l = on(stream);
    int32_t rc = launch_fill_zero(
        ctx->history, sizeof(int64_t) * (size_t)(batch_of(&ctx->cfg) * ctx->cfg.max_seq), l);
    if (rc == ENGRAM_OK)
        rc = launch_fill_zero(ctx->err, 256, l);
    if (rc != ENGRAM_OK)
        return rc;
    ctx->pos = 0;
    ctx->step_open = false;
    ctx->step_T = 0;
    ctx->was_reset = true;
    return ENGRAM_OK;
}

int32_t engram_forward(engram_ctx *ctx, int32_t hash_index, const int32_t *d_ids, int64_t T,
                       float *d_h, void *stream)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram forward: NULL context");
    CHECK(hash_index >= 0 && hash_index < ctx->nl, ENGRAM_E_ARG,
          "engram forward: hash index %d outside 0..%d", hash_index, ctx->nl - 1);
    const engram_ctx::Layer &L = ctx->layers[hash_index];
    CHECK(L.set, ENGRAM_E_STATE, "engram: layer %d has no weights", hash_index);
    CHECK(T >= 1, ENGRAM_E_ARG, "engram forward: T = %lld", (long long)T);
    CHECK(T <= ctx->cfg.max_tokens, ENGRAM_E_RANGE, "engram: %lld tokens exceed the %lld workspace",
          (long long)T, (long long)ctx->cfg.max_tokens);
    CHECK(d_h && aligned(d_h, 16), ENGRAM_E_ARG, "engram forward: highway NULL or misaligned");
    if (hash_index == 0) {
        CHECK(d_ids, ENGRAM_E_ARG, "engram forward: NULL token ids");
        // (graph mode: the position lives on the device, which checks it)
        CHECK(ctx->graph_mode || ctx->pos + T <= ctx->cfg.max_seq, ENGRAM_E_RANGE,
              "engram hasher: %lld positions, %lld needed", (long long)ctx->cfg.max_seq,
              (long long)(ctx->pos + T));
    } else {
        CHECK(ctx->step_open, ENGRAM_E_STATE,
              "engram forward: layer %d before layer 0 opened a step", hash_index);
        CHECK(ctx->step_T == T, ENGRAM_E_STATE,
              "engram forward: layer %d got %lld tokens, the step has %lld", hash_index,
              (long long)T, (long long)ctx->step_T);
    }
    CHECK(ctx->was_reset, ENGRAM_E_STATE, "engram forward: the context needs engram_reset first");
    hipStream_t s = as_stream(stream);
    const engram_config &cfg = ctx->cfg;
    const int64_t B = batch_of(&cfg), M = B * T;   // tokens of the call, sequence-major
    int32_t rc;
    const bool one_launch = M == 1 && ctx->fused_decode && cfg.head_dim == 256 &&
                            ctx->cols <= kDecodeMaxCols;
    const bool one_launch_multi = T == 1 && B >= 2 && B <= kDecodeMultiMaxB &&
                                  ctx->fused_decode && !L.wkv_q2k && cfg.head_dim == 256 &&
                                  ctx->cols <= kDecodeMaxCols && ctx->nl * ctx->cols <= 64;
    CHECK(!ctx->graph_mode || one_launch || one_launch_multi, ENGRAM_E_STATE,
          "engram forward: graph mode runs single-token steps through the one-launch decode "
          "kernels only (T = %lld, %lld sequences)", (long long)T, (long long)B);
    // layer 0 opens a new step at the current position; the step (and the
    // position's advance) takes effect once the launch that hashes it is
    // enqueued, so a refused launch leaves no half-open step behind
    if (hash_index == 0) {
        ctx->step_open = false;
        ctx->step_start = ctx->pos;
    }
    // graph mode: the kernels read the step's position from the device word,
    // and the last layer's gate moves it on
    const DecodePos dpos{ctx->step_start, ctx->graph_mode ? ctx->d_pos : nullptr, cfg.max_seq};
    int64_t *advance = ctx->graph_mode && hash_index == ctx->nl - 1 ? ctx->d_pos : nullptr;
    // graph mode: a step refused on the device (past max_seq) gates nothing
    const int32_t *refused = ctx->graph_mode ? ctx->err : nullptr;
    // one decode token of one sequence: hash, gather and projection in one launch
    if (one_launch) {
        rc = staged(ctx, 2, s, [&](const Launch &l) {
            return launch_decode(ctx->consts, cfg.hash.d_token_map, d_ids, dpos, ctx->history,
                                 hash_index, hash_index == 0, L.tab, L.wkv, L.wkv_q2k, ctx->kv,
                                 ctx->kv_width, ctx->row_ids, ctx->rows, ctx->err, l);
        });
        if (rc != ENGRAM_OK)
            return rc;
        if (hash_index == 0)
            open_step(ctx, 1);
        return staged(ctx, 3, s, [&](const Launch &l) {
            return launch_gate(d_h, ctx->kv, L.qk, 1, cfg.hc, cfg.dim, cfg.eps, l, advance,
                               cfg.max_seq, refused);
        });
    }
    // one decode token of each of 2..4 sequences: the same, all tokens in one
    // pass over the weights
    if (one_launch_multi) {
        rc = staged(ctx, 2, s, [&](const Launch &l) {
            return launch_decode_multi(ctx->consts, cfg.hash.d_token_map, d_ids, dpos,
                                       ctx->history, cfg.max_seq, hash_index, hash_index == 0,
                                       L.tab, L.wkv, ctx->kv, ctx->kv_width, ctx->row_ids,
                                       ctx->rows, ctx->err, B, l);
        });
        if (rc != ENGRAM_OK)
            return rc;
        if (hash_index == 0)
            open_step(ctx, 1);
        return staged(ctx, 3, s, [&](const Launch &l) {
            return launch_gate(d_h, ctx->kv, L.qk, M, cfg.hc, cfg.dim, cfg.eps, l, advance,
                               cfg.max_seq, refused);
        });
    }
    if (hash_index == 0) {
        rc = staged(ctx, 0, s, [&](const Launch &l) {
            return launch_hash(ctx->consts, cfg.hash.d_token_map, d_ids, B, T, ctx->step_start,
                               ctx->history, cfg.max_seq, ctx->row_ids, ctx->err, l);
        });
        if (rc != ENGRAM_OK)
            return rc;
        open_step(ctx, T);
    }
    const int64_t K = (int64_t)ctx->cols * cfg.head_dim;
    rc = staged(ctx, 1, s, [&](const Launch &l) {
        return launch_gather(L.tab, ctx->row_ids + (int64_t)hash_index * ctx->cols, M, ctx->cols,
                             (int64_t)ctx->nl * ctx->cols, ctx->rows, ctx->err, l);
    });
    if (rc != ENGRAM_OK)
        return rc;
    rc = staged(ctx, 2, s, [&](const Launch &l) {
        if (M == 1 && L.wkv_q2k)
            return launch_gemv_q2k(ctx->rows, L.wkv_q2k, ctx->kv, K, ctx->kv_width, l);
        return dispatch_project(ctx->rows, L.wkv, ctx->kv, M, K, ctx->kv_width, l);
    });
    if (rc != ENGRAM_OK)
        return rc;
    return staged(ctx, 3, s, [&](const Launch &l) {
        return launch_gate(d_h, ctx->kv, L.qk, M, cfg.hc, cfg.dim, cfg.eps, l);
    });
}

int32_t engram_check(engram_ctx *ctx, void *stream)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram check: NULL context");
    hipError_t e = hipStreamSynchronize(as_stream(stream));
    CHECK(e == hipSuccess, ENGRAM_E_HIP, "engram check: %s", hipGetErrorString(e));
    int32_t word = 0;
    e = hipMemcpy(&word, ctx->err, sizeof word, hipMemcpyDeviceToHost);
    CHECK(e == hipSuccess, ENGRAM_E_HIP, "engram check: %s", hipGetErrorString(e));
    CHECK(word == 0, ENGRAM_E_DEVICE, "engram device error 0x%x:%s%s%s", word,
          (word & ENGRAM_DEVERR_TOKEN) ? " token id outside the vocabulary" : "",
          (word & ENGRAM_DEVERR_ROW) ? " row id outside the table" : "",
          (word & ENGRAM_DEVERR_POSITION) ? " a replayed step past max_seq" : "");
    return ENGRAM_OK;
}

int64_t engram_position(const engram_ctx *ctx) { return ctx ? ctx->pos : -1; }

int32_t engram_ctx_set_position(engram_ctx *ctx, int64_t pos, void *stream)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram set position: NULL context");
    CHECK(pos >= 0 && pos <= ctx->cfg.max_seq, ENGRAM_E_RANGE,
          "engram set position: %lld outside 0..%lld", (long long)pos,
          (long long)ctx->cfg.max_seq);
    const Launch l = on(stream);
    int32_t rc = launch_fill_zero(ctx->err, 256, l);     // error word (and device position)
    if (rc == ENGRAM_OK && ctx->graph_mode)
        rc = launch_set_word(ctx->d_pos, pos, l);
    if (rc != ENGRAM_OK)
        return rc;
    ctx->pos = pos;
    ctx->step_open = false;
    ctx->step_T = 0;
    ctx->was_reset = true;
    return ENGRAM_OK;
}

int32_t engram_ctx_buffers(const engram_ctx *ctx, int64_t **d_row_ids, uint16_t **d_rows,
                           uint16_t **d_kv, int32_t **d_err)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram buffers: NULL context");
    if (d_row_ids)
        *d_row_ids = ctx->row_ids;
    if (d_rows)
        *d_rows = ctx->rows;
    if (d_kv)
        *d_kv = ctx->kv;
    if (d_err)
        *d_err = ctx->err;
    return ENGRAM_OK;
}

int32_t engram_ctx_set_fused_decode(engram_ctx *ctx, int32_t enable)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram fused decode: NULL context");
    CHECK(enable || !ctx->graph_mode, ENGRAM_E_STATE,
          "engram fused decode: graph mode needs the one-launch kernels");
    ctx->fused_decode = enable != 0;
    return ENGRAM_OK;
}

int32_t engram_ctx_set_timing(engram_ctx *ctx, int32_t enable)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram timing: NULL context");
    CHECK(!(enable && ctx->graph_mode), ENGRAM_E_STATE,
          "engram timing: not in graph mode (its events cannot be captured)");
    ctx->timing = enable != 0;
    return ENGRAM_OK;
}

int32_t engram_ctx_set_graph_mode(engram_ctx *ctx, int32_t enable, void *stream)
{
    CHECK(ctx, ENGRAM_E_ARG, "engram graph mode: NULL context");
    CHECK(ctx->was_reset, ENGRAM_E_STATE, "engram graph mode: the context needs engram_reset first");
    if (enable) {
        CHECK(!ctx->timing, ENGRAM_E_STATE, "engram graph mode: stage timing is on");
        CHECK(ctx->fused_decode, ENGRAM_E_STATE, "engram graph mode: one-launch decode is off");
        if (!ctx->graph_mode) {
            const int32_t rc = launch_set_word(ctx->d_pos, ctx->pos, on(stream));
            if (rc != ENGRAM_OK)
                return rc;
        }
        ctx->graph_mode = true;
        return ENGRAM_OK;
    }
    if (ctx->graph_mode) {
        hipError_t e = hipStreamSynchronize(as_stream(stream));
        CHECK(e == hipSuccess, ENGRAM_E_HIP, "engram graph mode: %s", hipGetErrorString(e));
        int64_t p = 0;
        e = hipMemcpy(&p, ctx->d_pos, sizeof p, hipMemcpyDeviceToHost);
        CHECK(e == hipSuccess, ENGRAM_E_HIP, "engram graph mode: %s", hipGetErrorString(e));
        ctx->pos = p;
        ctx->graph_mode = false;
    }
    return ENGRAM_OK;
}

int32_t engram_ctx_timing(engram_ctx *ctx, double *ms_per_stage, int64_t *launches_per_stage)
{
    CHECK(ctx && ms_per_stage && launches_per_stage, ENGRAM_E_ARG, "engram timing: NULL pointer");
    for (int i = 0; i < 4; i++) {
        ms_per_stage[i] = 0.0;
        launches_per_stage[i] = 0;
    }
    int32_t rc = ENGRAM_OK;
    for (const TimingRec &r : ctx->recs) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
            rc = fail(ENGRAM_E_HIP, "engram timing: event query failed");
        ms_per_stage[r.stage] += ms;
        launches_per_stage[r.stage] += 1;
        ctx->pool.push_back(r.a);
        ctx->pool.push_back(r.b);
    }
    ctx->recs.clear();
    return rc;
}

void engram_ctx_destroy(engram_ctx *ctx)
{
    if (!ctx)
        return;
    for (const TimingRec &r : ctx->recs) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (hipEvent_t e : ctx->pool)
        (void)hipEventDestroy(e);
    delete ctx;
}

}  // extern "C"
