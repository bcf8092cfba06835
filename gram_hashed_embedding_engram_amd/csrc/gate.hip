// Stage 4: the gate, in place on the FP32 highway (metrale
// "deepseek_v41_ref/engram.rs", gate_and_add; atlascybernetics
// "spark_model/layers/engram_v41.rs", module doc stage 4 and
// EngramV41::upload_qk).
//
// One workgroup of four wavefronts per (token, stream) row: wavefront w
// takes the 256-wide chunks w, w+4, ... of the row, with every load of h,
// qk, the key and the value in flight at once and h held in registers from
// the sums to the update, so h is read once and written once.  The three
// sums (h.h, key.key, h.qk.key) are f32, reduced per lane, per wavefront,
// then over the four wavefronts in a fixed order, so the result does not
// depend on T or on the kernel variant.  A single token's hc rows thus
// spread over hc compute units instead of queueing on one.
#include "common.h"

namespace engram {
namespace {

// The gate of one (token, stream) row by one wavefront (metrale
// "deepseek_v41_ref/engram.rs", gate_and_add): the sigmoid of the signed
// square root of the scaled, doubly normalised h.qk.key product.
__device__ __forceinline__ float gate_value(float hh, float kk, float dot, float fdim,
                                            float inv_sqrt_dim, float eps)
{
    const float rstd = (1.0f / sqrtf(hh / fdim + eps)) * (1.0f / sqrtf(kk / fdim + eps));
    const float s = dot * rstd * inv_sqrt_dim;
    const float g = copysignf(sqrtf(fmaxf(fabsf(s), 1e-6f)), s);
    return 1.0f / (1.0f + expf(-g));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One 4-value piece of a gate row: the three f32 sums h.h, key.key and
// h.qk.key, each an explicit fma chain so every kernel that calls this
// rounds the same way.
__device__ __forceinline__ void gate_accum(const float4 &h, const float4 &q, const u32x2 &k,
                                           float &hh, float &kk, float &dot)
{
    const float kf[4] = {bf16_lo(k.x), bf16_hi(k.x), bf16_lo(k.y), bf16_hi(k.y)};
    const float hf[4] = {h.x, h.y, h.z, h.w};
    const float qf[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
        hh = fmaf(hf[e], hf[e], hh);
        kk = fmaf(kf[e], kf[e], kk);
        dot = fmaf(hf[e] * qf[e], kf[e], dot);
    }
}

__device__ __forceinline__ float4 gate_update(float4 h, float gate, const u32x2 &v)
{
    h.x = fmaf(gate, bf16_lo(v.x), h.x);
    h.y = fmaf(gate, bf16_hi(v.x), h.y);
    h.z = fmaf(gate, bf16_lo(v.y), h.z);
    h.w = fmaf(gate, bf16_hi(v.y), h.w);
    return h;
}

// The gate of one (token, stream) row by the four wavefronts of a workgroup
// (every thread of the workgroup calls it).  The row is dim = 256*nch
// values; wavefront w takes its chunks w, w+4, w+8, ... (at most MAXI of
// them) and lane l values 4l..4l+3 of each.  Every load (h, qk, key, value)
// is issued before any arithmetic and h stays in registers from the sums to
// the update.  Each lane sums its chunks in order, the wavefront reduces its
// lanes, and the four wavefront partials are added in order through LDS;
// that sequence does not depend on MAXI.
template <int MAXI>
__device__ __forceinline__ void gate_row(float *__restrict__ hp, const uint16_t *__restrict__ key,
                                         const float *__restrict__ q,
                                         const uint16_t *__restrict__ val, int nch, float eps,
                                         float fdim, float inv_sqrt_dim)
{
    __shared__ float s_part[4][3];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float4 hv[MAXI], qv[MAXI];
    u32x2 kv[MAXI], vv[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; i++) {
        const int idx = (w + 4 * i) * 256 + lane * 4;
        if (w + 4 * i < nch) {
            hv[i] = *(const float4 *)(hp + idx);
            qv[i] = *(const float4 *)(q + idx);
            kv[i] = *(const u32x2 *)(key + idx);
            vv[i] = *(const u32x2 *)(val + idx);
        }
    }
    float hh = 0.0f, kk = 0.0f, dot = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXI; i++)
        if (w + 4 * i < nch)
            gate_accum(hv[i], qv[i], kv[i], hh, kk, dot);
    hh = wave_sum(hh);
    kk = wave_sum(kk);
    dot = wave_sum(dot);
    if (lane == 0) {
        s_part[w][0] = hh;
        s_part[w][1] = kk;
        s_part[w][2] = dot;
    }
    __syncthreads();
    float t[3];
#pragma unroll
    for (int j = 0; j < 3; j++)
        t[j] = ((s_part[0][j] + s_part[1][j]) + s_part[2][j]) + s_part[3][j];
    const float gate = gate_value(t[0], t[1], t[2], fdim, inv_sqrt_dim, eps);
#pragma unroll
    for (int i = 0; i < MAXI; i++)
        if (w + 4 * i < nch)
            *(float4 *)(hp + (w + 4 * i) * 256 + lane * 4) = gate_update(hv[i], gate, vv[i]);
}

// The same row, with the same bits, for any nch: the chunks are taken in
// batches of 4 (h read again for the update).
__device__ __forceinline__ void gate_row_any(float *__restrict__ hp,
                                             const uint16_t *__restrict__ key,
                                             const float *__restrict__ q,
                                             const uint16_t *__restrict__ val, int nch, float eps,
                                             float fdim, float inv_sqrt_dim)
{
    __shared__ float s_part[4][3];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float hh = 0.0f, kk = 0.0f, dot = 0.0f;
    for (int i0 = 0; w + 4 * i0 < nch; i0 += 4) {
        float4 hv[4], qv[4];
        u32x2 kv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int ch = w + 4 * (i0 + i);
            if (ch < nch) {
                hv[i] = *(const float4 *)(hp + ch * 256 + lane * 4);
                qv[i] = *(const float4 *)(q + ch * 256 + lane * 4);
                kv[i] = *(const u32x2 *)(key + ch * 256 + lane * 4);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (w + 4 * (i0 + i) < nch)
                gate_accum(hv[i], qv[i], kv[i], hh, kk, dot);
    }
    hh = wave_sum(hh);
    kk = wave_sum(kk);
    dot = wave_sum(dot);
    if (lane == 0) {
        s_part[w][0] = hh;
        s_part[w][1] = kk;
        s_part[w][2] = dot;
    }
    __syncthreads();
    float t[3];
#pragma unroll
    for (int j = 0; j < 3; j++)
        t[j] = ((s_part[0][j] + s_part[1][j]) + s_part[2][j]) + s_part[3][j];
    const float gate = gate_value(t[0], t[1], t[2], fdim, inv_sqrt_dim, eps);
    for (int ch = w; ch < nch; ch += 4) {
        float *p = hp + ch * 256 + lane * 4;
        *(float4 *)p = gate_update(*(const float4 *)p, gate, *(const u32x2 *)(val + ch * 256 + lane * 4));
    }
}

constexpr int kGateMaxI = 8;   // chunks per wavefront held in registers: dim <= 8192

// Workgroup b -> row (token * hc + stream).  Workgroups are dispatched to
// the eight XCDs in turn, so b, b+8, b+16, ... share an L2: the hc rows of
// a token go to hc such workgroups, and the token's value row (and key
// rows' lines) are fetched from HBM once instead of once per stream.  The
// last T % 8 tokens keep the plain order.
__device__ __forceinline__ int64_t token_row(int64_t b, int64_t T, int hc)
{
    const int64_t grouped = (T & ~(int64_t)7) * hc;
    if (b >= grouped)
        return b;
    const int64_t s = b >> 3;
    const int64_t k = s / hc;
    const int c = (int)(s - k * hc);
    return ((k << 3) + (b & 7)) * hc + c;
}

// The step's position word, moved on by one (up to max_seq) once workgroup
// 0's row is done: the last layer of a replayed decode step.  No other
// thread of the launch reads it.
__device__ __forceinline__ void advance_step(int64_t *advance, int64_t max_seq)
{
    if (advance && blockIdx.x == 0 && threadIdx.x == 0) {
        const int64_t v = *advance;
        if (v < max_seq)
            *advance = v + 1;
    }
}

// Graph mode: a replayed step past max_seq (the step's first decode kernel
// set ENGRAM_DEVERR_POSITION in the error word, which an earlier launch
// wrote and nothing in this one does) leaves the highway as it was.
__device__ __forceinline__ bool step_refused(const int32_t *err)
{
    return err && (*err & ENGRAM_DEVERR_POSITION);
}

template <int MAXI>
__global__ __launch_bounds__(256) void gate_kernel(float *__restrict__ h,
                                                   const uint16_t *__restrict__ kv,
                                                   const float *__restrict__ qk, int64_t T,
                                                   int hc, int64_t dim, float eps, float fdim,
                                                   float inv_sqrt_dim, int64_t *advance,
                                                   int64_t max_seq, const int32_t *err)
{
    if (step_refused(err))
        return;
    const int64_t row = token_row(blockIdx.x, T, hc);
    const int64_t t = row / hc;
    const int c = (int)(row - t * hc);
    const uint16_t *kvt = kv + t * (hc + 1) * dim;
    gate_row<MAXI>(h + row * dim, kvt + (int64_t)c * dim, qk + (int64_t)c * dim,
                   kvt + (int64_t)hc * dim, (int)(dim >> 8), eps, fdim, inv_sqrt_dim);
    advance_step(advance, max_seq);
}

// Any multiple of 256 (h is read again for the update).
__global__ __launch_bounds__(256) void gate_kernel_any(float *__restrict__ h,
                                                       const uint16_t *__restrict__ kv,
                                                       const float *__restrict__ qk, int64_t T,
                                                       int hc, int64_t dim, float eps,
                                                       float fdim, float inv_sqrt_dim,
                                                       int64_t *advance, int64_t max_seq,
                                                       const int32_t *err)
{
    if (step_refused(err))
        return;
    const int64_t row = token_row(blockIdx.x, T, hc);
    const int64_t t = row / hc;
    const int c = (int)(row - t * hc);
    const uint16_t *kvt = kv + t * (hc + 1) * dim;
    gate_row_any(h + row * dim, kvt + (int64_t)c * dim, qk + (int64_t)c * dim,
                 kvt + (int64_t)hc * dim, (int)(dim >> 8), eps, fdim, inv_sqrt_dim);
    advance_step(advance, max_seq);
}

__global__ __launch_bounds__(256) void qk_kernel(const uint16_t *__restrict__ q,
                                                 const uint16_t *__restrict__ k,
                                                 float *__restrict__ qk, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        qk[i] = __uint_as_float((uint32_t)q[i] << 16) * __uint_as_float((uint32_t)k[i] << 16);
}

__global__ __launch_bounds__(64) void set_word_kernel(int64_t *__restrict__ p, int64_t v)
{
    if (threadIdx.x == 0)
        *p = v;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t *__restrict__ p, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

int32_t launch_gate(float *h, const uint16_t *kv, const float *qk, int64_t T, int32_t hc,
                    int64_t dim, float eps, const Launch &l, int64_t *advance, int64_t max_seq,
                    const int32_t *err)
{
    const int64_t rows = T * hc;
    if (rows == 0)
        return ENGRAM_OK;
    const dim3 grid((unsigned)rows), block(256);
    const float fdim = (float)dim;
    const float inv_sqrt_dim = powf(fdim, -0.5f);
    const int64_t maxi = (dim / 256 + 3) / 4;
#define ENGRAM_GATE_CASE(I_)                                                                   \
    case I_:                                                                                   \
        dispatch(gate_kernel<I_>, grid, block, l, true, true, h, kv, qk, T, (int)hc, dim, eps, \
                 fdim, inv_sqrt_dim, advance, max_seq, err);                                  \
        break;
    switch (maxi) {
        ENGRAM_GATE_CASE(1) ENGRAM_GATE_CASE(2) ENGRAM_GATE_CASE(3) ENGRAM_GATE_CASE(4)
        ENGRAM_GATE_CASE(5) ENGRAM_GATE_CASE(6) ENGRAM_GATE_CASE(7) ENGRAM_GATE_CASE(8)
    default:
        dispatch(gate_kernel_any, grid, block, l, true, true, h, kv, qk, T, (int)hc, dim, eps,
                 fdim, inv_sqrt_dim, advance, max_seq, err);
        break;
    }
#undef ENGRAM_GATE_CASE
    static_assert(kGateMaxI == 8, "dispatch covers 1..kGateMaxI");
    return launch_status("engram gate kernel");
}

int32_t launch_qk_product(const uint16_t *q, const uint16_t *k, float *qk, int64_t n,
                          const Launch &l)
{
    if (n == 0)
        return ENGRAM_OK;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    dispatch(qk_kernel, dim3((unsigned)blocks), dim3(256), l, true, true, q, k, qk, n);
    return launch_status("engram qk kernel");
}

int32_t launch_set_word(int64_t *p, int64_t v, const Launch &l)
{
    dispatch(set_word_kernel, dim3(1), dim3(64), l, true, true, p, v);
    return launch_status("engram set-word kernel");
}

int32_t launch_fill_zero(void *p, size_t bytes, const Launch &l)
{
    const int64_t words = (int64_t)(bytes / 4);
    if (words == 0)
        return ENGRAM_OK;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    dispatch(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), l, true, true, (uint32_t *)p,
             words);
    return launch_status("engram fill kernel");
}

}  // namespace engram
