// Stage 3 at one to four tokens: the wkv projection as an HBM-streaming GEMV
// (atlascybernetics "spark_model/layers/engram_v41.rs", EngramV41::gemv_k
// and module doc stage 3; metrale "deepseek_v41_ref/engram.rs",
// linear_bf16).  At a single token the projection reads every weight once
// and does two flops per weight, so its bound is HBM bandwidth, not the
// matrix cores.
//
// Layout: w [N][K] bf16, K contiguous.  One wavefront owns one output row at
// a time and reads it as K/512 coalesced 1 KiB loads (16 bytes a lane, all
// issued before the first is consumed, to keep many bytes in flight); the
// row then passes through the wavefront's 2 KiB LDS buffer into the
// sub-block order common.h fixes for one-token projections, so results equal
// those of the projection over Q2_K wkv blocks bit for bit.  The activations
// x [T][K] are loaded once per wave into registers in that order (lane l:
// chunks 2g, 2g+1 of sub-blocks g = l, l+64, ...).  Waves are persistent and
// take rows wave_id, wave_id + n_waves, ...  The per-lane f32 partial sums
// are reduced across the wave; the sum is rounded once to bf16.
#include "common.h"

namespace engram {
namespace {

constexpr int kGemvBlocksPerCu = 4;
constexpr int kGemvMultiThreads = 1024;

template <int NT, int NI>
__global__ __launch_bounds__(256) void gemv_kernel(const uint16_t *__restrict__ x,
                                                   const uint16_t *__restrict__ w,
                                                   uint16_t *__restrict__ y, int64_t K, int64_t N)
{
    constexpr int NS = (NI + 1) / 2;                 // 128-chunk segments of a row
    __shared__ u32x4 s_stage[4][128];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t kc = K >> 3;                       // 16-byte chunks per row
    const int n_sb = (int)(K >> 4);                  // 16-value sub-blocks per row
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;

    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 xr[NT][2 * NS];
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const u32x4 *xt = (const u32x4 *)(x + t * K);
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const int g = 64 * s + lane;
            xr[t][2 * s] = g < n_sb ? xt[2 * g] : zero;
            xr[t][2 * s + 1] = g < n_sb ? xt[2 * g + 1] : zero;
        }
    }

    u32x4 *stage = s_stage[wid];
    for (int64_t n = wave; n < N; n += n_waves) {
        const u32x4 *wr = (const u32x4 *)(w + n * K);
        u32x4 wv[NI];
#pragma unroll
        for (int i = 0; i < NI; i++) {
            const int64_t idx = (int64_t)i * 64 + lane;
            wv[i] = idx < kc ? __builtin_nontemporal_load(wr + idx) : zero;
        }
        float acc[NT], acc2[NT];
#pragma unroll
        for (int t = 0; t < NT; t++)
            acc[t] = acc2[t] = 0.0f;
        for_each_subblock<NI>(wv, stage, lane, n_sb, [&](int s, const u32x4 &a, const u32x4 &b) {
#pragma unroll
            for (int t = 0; t < NT; t++)
                subblock_dot(a, b, xr[t][2 * s], xr[t][2 * s + 1], acc[t], acc2[t]);
        });
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float s = wave_sum(acc[t] + acc2[t]);
            if (lane == t)
                y[t * N + n] = f32_to_bf16(s);
        }
    }
}

// The same projection for NT = 2..4 tokens in one pass over the weights: the
// tokens' activations [NT][K] sit in LDS (one 1024-thread workgroup per CU,
// so they are staged once per CU), and each row's sub-blocks meet every token
// in the one-token order above -- a token's outputs are bit for bit those of
// a one-token call.  At these T the arithmetic (NT v_dot2 a weight pair) is
// still small next to the weight stream.
template <int NT, int NI>
__global__ __launch_bounds__(kGemvMultiThreads) void gemv_multi_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
    int64_t K, int64_t N)
{
    constexpr int NW = kGemvMultiThreads / 64;
    constexpr int NX = (NT * NI * 64 + kGemvMultiThreads - 1) / kGemvMultiThreads;
    __shared__ u32x4 s_x[kGemvMultiMaxX / 8];
    __shared__ u32x4 s_stage[NW][128];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int kc = (int)(K >> 3), n_sb = (int)(K >> 4), nx = NT * kc;
    const int kcp = (kc + 127) & ~127;         // LDS slots a token (xslot layout)
    const int64_t wave = (int64_t)blockIdx.x * NW + wid;
    const int64_t n_waves = (int64_t)gridDim.x * NW;
    const u32x4 *x4 = (const u32x4 *)x;

    // the tokens' chunks (past the end: the last one again, not stored), then
    // this wavefront's first row, then the chunks into LDS: the wait for the
    // chunks leaves the row's loads in flight
    u32x4 xv[NX];
#pragma unroll
    for (int j = 0; j < NX; j++)
        xv[j] = x4[min(tid + j * kGemvMultiThreads, nx - 1)];
    const u32x4 *wr0 = (const u32x4 *)(w + min(wave, N - 1) * K);
    u32x4 wv[NI];
#pragma unroll
    for (int i = 0; i < NI; i++)
        wv[i] = __builtin_nontemporal_load(wr0 + min(i * 64 + lane, kc - 1));
#pragma unroll
    for (int j = 0; j < NX; j++) {
        const int i = tid + j * kGemvMultiThreads;      // chunk i % kc of token i / kc
        if (i < nx)
            s_x[(i / kc) * kcp + xslot(i % kc)] = xv[j];
    }
    __syncthreads();

    u32x4 *stage = s_stage[wid];
    for (int64_t n = wave; n < N; n += n_waves) {
        if (n != wave) {
            const u32x4 *wr = (const u32x4 *)(w + n * K);
#pragma unroll
            for (int i = 0; i < NI; i++)
                wv[i] = __builtin_nontemporal_load(wr + min(i * 64 + lane, kc - 1));
        }
        float acc[NT], acc2[NT];
#pragma unroll
        for (int t = 0; t < NT; t++)
            acc[t] = acc2[t] = 0.0f;
        for_each_subblock<NI>(wv, stage, lane, n_sb, [&](int s, const u32x4 &a, const u32x4 &b) {
#pragma unroll
            for (int t = 0; t < NT; t++)
                subblock_dot(a, b, s_x[t * kcp + 128 * s + lane], s_x[t * kcp + 128 * s + 64 + lane],
                             acc[t], acc2[t]);
        });
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float v = wave_sum(acc[t] + acc2[t]);
            if (lane == t)
                y[t * N + n] = f32_to_bf16(v);
        }
    }
}

template <int NT>
int32_t launch_multi(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t K, int64_t N,
                     const Launch &l)
{
    const int cus = device_cus();
    constexpr int NW = kGemvMultiThreads / 64;
    int64_t blocks = (N + NW - 1) / NW;
    if (blocks > cus)
        blocks = cus;
    const dim3 grid((unsigned)blocks), block(kGemvMultiThreads);
    const int64_t ni = (K + 511) / 512;
#define ENGRAM_GEMV_MULTI_CASE(NI_)                                                         \
    case NI_:                                                                               \
        dispatch(gemv_multi_kernel<NT, NI_>, grid, block, l, true, true, x, w, y, K, N);    \
        break;
    switch (ni) {
        ENGRAM_GEMV_MULTI_CASE(1) ENGRAM_GEMV_MULTI_CASE(2) ENGRAM_GEMV_MULTI_CASE(3)
        ENGRAM_GEMV_MULTI_CASE(4) ENGRAM_GEMV_MULTI_CASE(5) ENGRAM_GEMV_MULTI_CASE(6)
        ENGRAM_GEMV_MULTI_CASE(7) ENGRAM_GEMV_MULTI_CASE(8) ENGRAM_GEMV_MULTI_CASE(9)
        ENGRAM_GEMV_MULTI_CASE(10) ENGRAM_GEMV_MULTI_CASE(11) ENGRAM_GEMV_MULTI_CASE(12)
        ENGRAM_GEMV_MULTI_CASE(13) ENGRAM_GEMV_MULTI_CASE(14) ENGRAM_GEMV_MULTI_CASE(15)
        ENGRAM_GEMV_MULTI_CASE(16)
    default:
        return fail(ENGRAM_E_UNSUPPORTED, "engram gemv: K = %lld exceeds %lld", (long long)K,
                    (long long)kGemvMaxK);
    }
#undef ENGRAM_GEMV_MULTI_CASE
    return launch_status("engram gemv kernel");
}

template <int NT>
int32_t launch_nt(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t K, int64_t N,
                  const Launch &l, bool first, bool last)
{
    const int cus = device_cus();
    const int64_t ni = (K + 511) / 512;
    int64_t blocks = (N + 3) / 4;
    const int64_t cap = (int64_t)cus * kGemvBlocksPerCu;
    if (blocks > cap)
        blocks = cap;
    const dim3 grid((unsigned)blocks), block(256);
#define ENGRAM_GEMV_CASE(NI_)                                                               \
    case NI_:                                                                               \
        dispatch(gemv_kernel<NT, NI_>, grid, block, l, first, last, x, w, y, K, N);         \
        break;
    switch (ni) {
        ENGRAM_GEMV_CASE(1) ENGRAM_GEMV_CASE(2) ENGRAM_GEMV_CASE(3) ENGRAM_GEMV_CASE(4)
        ENGRAM_GEMV_CASE(5) ENGRAM_GEMV_CASE(6) ENGRAM_GEMV_CASE(7) ENGRAM_GEMV_CASE(8)
        ENGRAM_GEMV_CASE(9) ENGRAM_GEMV_CASE(10) ENGRAM_GEMV_CASE(11) ENGRAM_GEMV_CASE(12)
        ENGRAM_GEMV_CASE(13) ENGRAM_GEMV_CASE(14) ENGRAM_GEMV_CASE(15) ENGRAM_GEMV_CASE(16)
    default:
        return fail(ENGRAM_E_UNSUPPORTED, "engram gemv: K = %lld exceeds %lld", (long long)K,
                    (long long)kGemvMaxK);
    }
#undef ENGRAM_GEMV_CASE
    return launch_status("engram gemv kernel");
}

}  // namespace

bool gemv_multi_fits(int64_t T, int64_t K)
{
    return T >= 2 && T <= kGemvMultiMaxT && K <= kGemvMaxK &&
           T * ((K + 1023) / 1024) * 1024 <= kGemvMultiMaxX;
}

int32_t launch_gemv_multi(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t T,
                          int64_t K, int64_t N, const Launch &l)
{
    switch (T) {
    case 2: return launch_multi<2>(x, w, y, K, N, l);
    case 3: return launch_multi<3>(x, w, y, K, N, l);
    case 4: return launch_multi<4>(x, w, y, K, N, l);
    default:
        return fail(ENGRAM_E_UNSUPPORTED, "engram gemv: %lld tokens", (long long)T);
    }
}

int32_t launch_gemv(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t T, int64_t K,
                    int64_t N, const Launch &l)
{
    // two tokens share one pass over the weights; a third or fourth token
    // takes another pass
    for (int64_t t0 = 0; t0 < T; t0 += 2) {
        const int64_t nt = T - t0 >= 2 ? 2 : 1;
        const bool first = t0 == 0, last = t0 + nt >= T;
        const int32_t rc = nt == 2
                               ? launch_nt<2>(x + t0 * K, w, y + t0 * N, K, N, l, first, last)
                               : launch_nt<1>(x + t0 * K, w, y + t0 * N, K, N, l, first, last);
        if (rc != ENGRAM_OK)
            return rc;
    }
    return ENGRAM_OK;
}

}  // namespace engram
