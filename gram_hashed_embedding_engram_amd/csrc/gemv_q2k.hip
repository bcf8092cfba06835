// Stage 3 at one token with wkv shipped as Q2_K blocks (atlascybernetics
// "spark_model/layers/engram_v41.rs", EngramLayerWeights::wkv_q2k, read by
// the single-token projection in place of the bf16 expansion).
//
// y[n] = bf16(sum_k x[k] * w[n][k]) with w[n][k] the bf16 weight its Q2_K
// block decodes to.  Persistent wavefronts (four 256-thread workgroups per
// CU), one output row at a time: the next row's loads go out before this
// row's arithmetic, the row's dwords are staged in the wavefront's LDS
// buffer, and the row dot product is wkv_q2k.h's.  The activations of a
// lane's sub-blocks stay in registers for the whole launch.
#include "wkv_q2k.h"

namespace engram {
namespace {

constexpr int kQ2kBlocksPerCu = 4;

template <int NSB>
__global__ __launch_bounds__(256) void gemv_q2k_kernel(const uint16_t *__restrict__ x,
                                                       const uint8_t *__restrict__ w,
                                                       uint16_t *__restrict__ y, int64_t N, int K)
{
    constexpr int NLD = q2k_row_loads<NSB>();
    __shared__ uint32_t s_row[4][kQ2kWkvMaxRowDwords];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int n_sb = K >> 4, row_dwords = 21 * (K >> 8);
    const uint32_t *wd = (const uint32_t *)w;

    uint32_t r[NLD];
    q2k_row_load<NLD>(wd + min(wave, N - 1) * row_dwords, row_dwords, lane, r);

    uint32_t xr[NSB][8];
#pragma unroll
    for (int i = 0; i < NSB; i++) {
        const int g = lane + 64 * i;
        u32x4 a = {0u, 0u, 0u, 0u}, b = a;
        if (g < n_sb) {
            a = *(const u32x4 *)(x + 16 * g);
            b = *(const u32x4 *)(x + 16 * g + 8);
        }
        xr[i][0] = a.x; xr[i][1] = a.y; xr[i][2] = a.z; xr[i][3] = a.w;
        xr[i][4] = b.x; xr[i][5] = b.y; xr[i][6] = b.z; xr[i][7] = b.w;
    }

    for (int64_t n = wave; n < N; n += n_waves) {
        q2k_row_stage<NLD>(s_row[wid], r, row_dwords, lane);
        if (n + n_waves < N)
            q2k_row_load<NLD>(wd + (n + n_waves) * row_dwords, row_dwords, lane, r);
        const float s = wave_sum(q2k_row_dot<NSB>(s_row[wid], xr, n_sb, lane));
        if (lane == 0)
            y[n] = f32_to_bf16(s);
    }
}

}  // namespace

int32_t launch_gemv_q2k(const uint16_t *x, const uint8_t *w, uint16_t *y, int64_t K, int64_t N,
                        const Launch &l)
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    int64_t blocks = (N + 3) / 4;
    const int64_t cap = (int64_t)cus * kQ2kBlocksPerCu;
    if (blocks > cap)
        blocks = cap;
    const dim3 grid((unsigned)blocks), block(256);
    const int nsb = (int)((K + 1023) / 1024);
#define ENGRAM_GEMV_Q2K_CASE(S_)                                                                 \
    case S_:                                                                                     \
        dispatch(gemv_q2k_kernel<S_>, grid, block, l, true, true, x, w, y, N, (int)K);           \
        break;
    switch (nsb) {
        ENGRAM_GEMV_Q2K_CASE(1) ENGRAM_GEMV_Q2K_CASE(2) ENGRAM_GEMV_Q2K_CASE(3)
        ENGRAM_GEMV_Q2K_CASE(4) ENGRAM_GEMV_Q2K_CASE(5) ENGRAM_GEMV_Q2K_CASE(6)
        ENGRAM_GEMV_Q2K_CASE(7) ENGRAM_GEMV_Q2K_CASE(8)
    default:
        return fail(ENGRAM_E_UNSUPPORTED, "engram project_q2k: K = %lld above %d", (long long)K,
                    kQ2kMaxSubBlocks * 1024);
    }
#undef ENGRAM_GEMV_Q2K_CASE
    return launch_status("engram gemv_q2k kernel");
}

}  // namespace engram
