// Stage 3 at one token with wkv shipped as Q2_K blocks (atlascybernetics
// "spark_model/layers/engram_v41.rs", EngramLayerWeights::wkv_q2k: one
// token's projection reads these blocks instead of their bf16 expansion).
//
// y[n] = bf16(sum_k x[k] * w[n][k]) with w[n][k] the bf16 weight its Q2_K
// block decodes to.  Persistent wavefronts (two 1024-thread workgroups per
// CU), one output row at a time: the next row's loads go out before this
// row's arithmetic, the row's dwords are staged in the wavefront's LDS
// buffer, and the row dot product is wkv_q2k.h's, reading the token's
// activations from the workgroup's copy in LDS.
#include "wkv_q2k.h"

namespace engram {
namespace {

constexpr int kQ2kThreads = 1024;
constexpr int kQ2kBlocksPerCu = 2;

template <int NSB>
__global__ __launch_bounds__(kQ2kThreads, 8) void gemv_q2k_kernel(const uint16_t *__restrict__ x,
                                                               const uint8_t *__restrict__ w,
                                                               uint16_t *__restrict__ y, int64_t N,
                                                               int K)
{
    constexpr int NLD = q2k_row_loads<NSB>();
    __shared__ u32x4 s_x[kQ2kMaxSubBlocks * 128];
    __shared__ uint32_t s_row[kQ2kThreads / 64][kQ2kWkvMaxRowDwords];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + tid) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int n_sb = K >> 4, row_dwords = 21 * (K >> 8);
    const uint32_t *wd = (const uint32_t *)w;

    uint32_t r[NLD];
    q2k_row_load<NLD>(wd + min(wave, N - 1) * row_dwords, row_dwords, lane, r);

    // the token's activations, once per workgroup, into LDS
    for (int ch = tid; ch < (K >> 3); ch += kQ2kThreads)
        s_x[xslot(ch)] = ((const u32x4 *)x)[ch];
    __syncthreads();

    for (int64_t n = wave; n < N; n += n_waves) {
        q2k_row_stage<NLD>(s_row[wid], r, row_dwords, lane);
        if (n + n_waves < N)
            q2k_row_load<NLD>(wd + (n + n_waves) * row_dwords, row_dwords, lane, r);
        const float s = wave_sum(q2k_row_dot<NSB>(s_row[wid], s_x, n_sb, lane));
        if (lane == 0)
            y[n] = f32_to_bf16(s);
    }
}

}  // namespace

int32_t launch_gemv_q2k(const uint16_t *x, const uint8_t *w, uint16_t *y, int64_t K, int64_t N,
                        const Launch &l)
{
    const int cus = device_cus();
    int64_t blocks = (N + kQ2kThreads / 64 - 1) / (kQ2kThreads / 64);
    const int64_t cap = (int64_t)cus * kQ2kBlocksPerCu;
    if (blocks > cap)
        blocks = cap;
    const dim3 grid((unsigned)blocks), block(kQ2kThreads);
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
