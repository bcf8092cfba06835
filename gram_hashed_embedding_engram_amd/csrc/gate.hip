// Stage 4: the gate, in place on the FP32 highway (metrale
// "deepseek_v41_ref/engram.rs", gate_and_add; atlascybernetics
// "spark_model/layers/engram_v41.rs", module doc stage 4 and
// EngramV41::upload_qk).
//
// One wavefront per (token, stream).  A lane holds 4 consecutive highway
// values of each 256-wide chunk in registers (dim/64 values), so h is read
// once and written once; the three sums (h.h, key.key, h.qk.key) are f32
// partials reduced across the wave, the scalar gate is computed by every
// lane, and h += gate * value is written back with 16-byte stores.  The
// value row is shared by the hc streams of a token and is read from L2 after
// the first wave.  Widths above 4096 take a two-pass variant that re-reads h.
#include "common.h"

namespace engram {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float gate_value(float hh, float kk, float dot, float fdim,
                                            float inv_sqrt_dim, float eps)
{
    const float rstd = (1.0f / sqrtf(hh / fdim + eps)) * (1.0f / sqrtf(kk / fdim + eps));
    const float s = dot * rstd * inv_sqrt_dim;
    const float g = copysignf(sqrtf(fmaxf(fabsf(s), 1e-6f)), s);
    return 1.0f / (1.0f + expf(-g));
}

template <int NCH>
__global__ __launch_bounds__(256) void gate_kernel(float *__restrict__ h,
                                                   const uint16_t *__restrict__ kv,
                                                   const float *__restrict__ qk, int64_t T, int hc,
                                                   int64_t dim, float eps, float fdim,
                                                   float inv_sqrt_dim)
{
    const int64_t wid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wid >= T * hc)
        return;
    const int64_t t = wid / hc;
    const int c = (int)(wid - t * hc);
    float *hp = h + wid * dim;
    const uint16_t *key = kv + t * (hc + 1) * dim + (int64_t)c * dim;
    const uint16_t *val = kv + t * (hc + 1) * dim + (int64_t)hc * dim;
    const float *q = qk + (int64_t)c * dim;

    float4 hv[NCH];
    float hh = 0.0f, kk = 0.0f, dot = 0.0f;
#pragma unroll
    for (int ch = 0; ch < NCH; ch++) {
        const int64_t idx = (int64_t)ch * 256 + lane * 4;
        hv[ch] = *(const float4 *)(hp + idx);
        const u32x2 k2 = *(const u32x2 *)(key + idx);
        const float4 q4 = *(const float4 *)(q + idx);
        const float kf[4] = {bf16_lo(k2.x), bf16_hi(k2.x), bf16_lo(k2.y), bf16_hi(k2.y)};
        const float hf[4] = {hv[ch].x, hv[ch].y, hv[ch].z, hv[ch].w};
        const float qf[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            hh += hf[e] * hf[e];
            kk += kf[e] * kf[e];
            dot += hf[e] * qf[e] * kf[e];
        }
    }
    hh = wave_sum(hh);
    kk = wave_sum(kk);
    dot = wave_sum(dot);
    const float gate = gate_value(hh, kk, dot, fdim, inv_sqrt_dim, eps);
#pragma unroll
    for (int ch = 0; ch < NCH; ch++) {
        const int64_t idx = (int64_t)ch * 256 + lane * 4;
        const u32x2 v2 = *(const u32x2 *)(val + idx);
        float4 o = hv[ch];
        o.x += gate * bf16_lo(v2.x);
        o.y += gate * bf16_hi(v2.x);
        o.z += gate * bf16_lo(v2.y);
        o.w += gate * bf16_hi(v2.y);
        *(float4 *)(hp + idx) = o;
    }
}

// Any multiple of 256: first pass sums, second pass re-reads h and updates.
__global__ __launch_bounds__(256) void gate_kernel_2pass(float *__restrict__ h,
                                                         const uint16_t *__restrict__ kv,
                                                         const float *__restrict__ qk, int64_t T,
                                                         int hc, int64_t dim, float eps,
                                                         float fdim, float inv_sqrt_dim)
{
    const int64_t wid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wid >= T * hc)
        return;
    const int64_t t = wid / hc;
    const int c = (int)(wid - t * hc);
    float *hp = h + wid * dim;
    const uint16_t *key = kv + t * (hc + 1) * dim + (int64_t)c * dim;
    const uint16_t *val = kv + t * (hc + 1) * dim + (int64_t)hc * dim;
    const float *q = qk + (int64_t)c * dim;
    float hh = 0.0f, kk = 0.0f, dot = 0.0f;
    for (int64_t idx = lane * 4; idx < dim; idx += 256) {
        const float4 hv = *(const float4 *)(hp + idx);
        const u32x2 k2 = *(const u32x2 *)(key + idx);
        const float4 q4 = *(const float4 *)(q + idx);
        const float kf[4] = {bf16_lo(k2.x), bf16_hi(k2.x), bf16_lo(k2.y), bf16_hi(k2.y)};
        const float hf[4] = {hv.x, hv.y, hv.z, hv.w};
        const float qf[4] = {q4.x, q4.y, q4.z, q4.w};
        for (int e = 0; e < 4; e++) {
            hh += hf[e] * hf[e];
            kk += kf[e] * kf[e];
            dot += hf[e] * qf[e] * kf[e];
        }
    }
    hh = wave_sum(hh);
    kk = wave_sum(kk);
    dot = wave_sum(dot);
    const float gate = gate_value(hh, kk, dot, fdim, inv_sqrt_dim, eps);
    for (int64_t idx = lane * 4; idx < dim; idx += 256) {
        const u32x2 v2 = *(const u32x2 *)(val + idx);
        float4 o = *(const float4 *)(hp + idx);
        o.x += gate * bf16_lo(v2.x);
        o.y += gate * bf16_hi(v2.x);
        o.z += gate * bf16_lo(v2.y);
        o.w += gate * bf16_hi(v2.y);
        *(float4 *)(hp + idx) = o;
    }
}

__global__ __launch_bounds__(256) void qk_kernel(const uint16_t *__restrict__ q,
                                                 const uint16_t *__restrict__ k,
                                                 float *__restrict__ qk, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        qk[i] = __uint_as_float((uint32_t)q[i] << 16) * __uint_as_float((uint32_t)k[i] << 16);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t *__restrict__ p, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

int32_t launch_gate(float *h, const uint16_t *kv, const float *qk, int64_t T, int32_t hc,
                    int64_t dim, float eps, const Launch &l)
{
    const int64_t waves = T * hc;
    if (waves == 0)
        return ENGRAM_OK;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    const float fdim = (float)dim;
    const float inv_sqrt_dim = powf(fdim, -0.5f);
    const int64_t nch = dim / 256;
    const bool in_registers = nch == 1 || nch == 2 || nch == 4 || nch == 8 || nch == 16;
#define ENGRAM_GATE_CASE(N_)                                                              \
    case N_:                                                                              \
        dispatch(gate_kernel<N_>, grid, block, l, true, true, h, kv, qk, T, hc, dim, eps, fdim, \
                 inv_sqrt_dim);                                                          \
        break;
    if (in_registers) {
        switch (nch) {
            ENGRAM_GATE_CASE(1) ENGRAM_GATE_CASE(2) ENGRAM_GATE_CASE(4) ENGRAM_GATE_CASE(8)
            ENGRAM_GATE_CASE(16)
        default:
            break;
        }
    } else {
        dispatch(gate_kernel_2pass, grid, block, l, true, true, h, kv, qk, T, hc, dim, eps, fdim,
                 inv_sqrt_dim);
    }
#undef ENGRAM_GATE_CASE
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
