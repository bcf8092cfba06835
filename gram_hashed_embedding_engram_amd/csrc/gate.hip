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

constexpr int kGateMaxI = 8;   // chunks per wavefront held in registers: dim <= 8192

template <int MAXI>
__global__ __launch_bounds__(256) void gate_kernel(float *__restrict__ h,
                                                   const uint16_t *__restrict__ kv,
                                                   const float *__restrict__ qk, int hc,
                                                   int64_t dim, float eps, float fdim,
                                                   float inv_sqrt_dim)
{
    const int64_t row = blockIdx.x;
    const int64_t t = row / hc;
    const int c = (int)(row - t * hc);
    const uint16_t *kvt = kv + t * (hc + 1) * dim;
    gate_row<MAXI>(h + row * dim, kvt + (int64_t)c * dim, qk + (int64_t)c * dim,
                   kvt + (int64_t)hc * dim, (int)(dim >> 8), eps, fdim, inv_sqrt_dim);
}

// Any multiple of 256 (h is read again for the update).
__global__ __launch_bounds__(256) void gate_kernel_any(float *__restrict__ h,
                                                       const uint16_t *__restrict__ kv,
                                                       const float *__restrict__ qk, int hc,
                                                       int64_t dim, float eps, float fdim,
                                                       float inv_sqrt_dim)
{
    const int64_t row = blockIdx.x;
    const int64_t t = row / hc;
    const int c = (int)(row - t * hc);
    const uint16_t *kvt = kv + t * (hc + 1) * dim;
    gate_row_any(h + row * dim, kvt + (int64_t)c * dim, qk + (int64_t)c * dim,
                 kvt + (int64_t)hc * dim, (int)(dim >> 8), eps, fdim, inv_sqrt_dim);
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
    const int64_t rows = T * hc;
    if (rows == 0)
        return ENGRAM_OK;
    const dim3 grid((unsigned)rows), block(256);
    const float fdim = (float)dim;
    const float inv_sqrt_dim = powf(fdim, -0.5f);
    const int64_t maxi = (dim / 256 + 3) / 4;
#define ENGRAM_GATE_CASE(I_)                                                                   \
    case I_:                                                                                   \
        dispatch(gate_kernel<I_>, grid, block, l, true, true, h, kv, qk, (int)hc, dim, eps,    \
                 fdim, inv_sqrt_dim);                                                         \
        break;
    switch (maxi) {
        ENGRAM_GATE_CASE(1) ENGRAM_GATE_CASE(2) ENGRAM_GATE_CASE(3) ENGRAM_GATE_CASE(4)
        ENGRAM_GATE_CASE(5) ENGRAM_GATE_CASE(6) ENGRAM_GATE_CASE(7) ENGRAM_GATE_CASE(8)
    default:
        dispatch(gate_kernel_any, grid, block, l, true, true, h, kv, qk, (int)hc, dim, eps, fdim,
                 inv_sqrt_dim);
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
