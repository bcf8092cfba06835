// Stage 3 for a few tokens (5..128): the wkv projection as a bf16 MFMA GEMM
// with a short token dimension (atlascybernetics "spark_model/layers/
// engram_v41.rs", module doc stage 3; metrale "deepseek_v41_ref/engram.rs",
// linear_bf16) -- several sequences' decode tokens, short prompts.
//
// C[M][N] = A[M][K] * B[N][K]^T with A = the tokens (M <= 128), B = wkv.  At
// this M the GEMM is a single pass over wkv (252 MB at the decode shape), so
// the kernel is laid out like a weight stream: a workgroup per CU owns 16*RT
// consecutive output rows (RT <= 5) for all tokens and its wavefronts split
// K.  The matrix-core "A" operand is wkv (16 rows), "B" the tokens (16 per
// tile, MT tiles), so each lane's accumulator holds 4 consecutive outputs of
// one token (8-byte stores).
//
// A stream like this needs several wavefronts a SIMD to keep its loads in
// flight: with one (four a workgroup) it ran at about 4.9 TB/s, with three
// at about 6.0.  So a workgroup has twelve wavefronts for one or two token
// tiles and eight -- whose partial sums still fit in LDS -- for three or four.
// Five to eight token tiles (65..128 tokens) take four wavefronts with 80
// rows a workgroup: their accumulators need the AGPRs of a wavefront alone
// on its SIMD, and every workgroup reads all the tokens, so fewer, wider
// workgroups keep that traffic down (89 us at 128 tokens, against 166 us for
// the tiled GEMM, whose 64 workgroups leave most CUs idle).
#include "common.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Wavefront w of W takes the 64-value K segments w, w+W, w+2W, ... of the
// workgroup's 16*RT rows.  A segment of a 16-row tile arrives as two
// non-temporal loads of 8 rows x 128 contiguous bytes (whole cache lines:
// lane l takes row 8i + l/8, bytes 16*(l%8)), passes through the wavefront's
// own LDS buffer (rows padded to 144 bytes) and is read back in the MFMA
// layout (lane l: row l%16, values 8(l/16) .. of each 32-value step).  The W
// partial sums meet in LDS and are added in wavefront order.
constexpr int kFewSeg = 64;                        // K values a segment
constexpr int kFewRowBytes = 2 * kFewSeg + 16;     // LDS bytes a staged row
constexpr int kFewMaxRowTiles = 5;

template <int RT, int MT, int W>
__global__ __launch_bounds__(64 * W) void gemm_few_kernel(const uint16_t *__restrict__ A,
                                                          const uint16_t *__restrict__ B,
                                                          uint16_t *__restrict__ C, int M, int N,
                                                          int K)
{
    constexpr int STAGE_B = W * RT * 16 * kFewRowBytes;
    constexpr int RED_B = W * RT * MT * 64 * 16;
    static_assert(STAGE_B <= 160 * 1024 && RED_B <= 160 * 1024, "LDS");
    // the wavefronts' stage buffers, then (after a barrier) their partial sums
    __shared__ __attribute__((aligned(16))) uint8_t lds[STAGE_B > RED_B ? STAGE_B : RED_B];
    f32x4(*red)[RT][MT][64] = (f32x4(*)[RT][MT][64])lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, q = lane >> 4;
    const int n0 = blockIdx.x * 16 * RT;
    const int nseg = K / kFewSeg;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    uint8_t *stage = lds + w * (RT * 16 * kFewRowBytes);

    // load j of tile rt: rows past N read row N-1 (never stored); tokens past
    // M are zeros, not loaded
    const u32x4 *wrow[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int i = 0; i < 2; i++)
            wrow[rt][i] = (const u32x4 *)(B + (int64_t)min(n0 + 16 * rt + 8 * i + (lane >> 3),
                                                          N - 1) * K) + (lane & 7);
    const u32x4 *arow[MT];
    bool avalid[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
        const int m = 16 * mt + r16;
        avalid[mt] = m < M;
        arow[mt] = (const u32x4 *)(A + (int64_t)(m < M ? m : 0) * K + 8 * q);
    }
    f32x4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
            acc[rt][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int j = w; j < nseg; j += W) {
        u32x4 wb[RT][2], xb[2][MT];
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int i = 0; i < 2; i++)
                wb[rt][i] = __builtin_nontemporal_load(wrow[rt][i] + j * (kFewSeg / 8));
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
                xb[s][mt] = avalid[mt] ? arow[mt][4 * (2 * j + s)] : zero;
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int i = 0; i < 2; i++)
                *(u32x4 *)(stage + (16 * rt + 8 * i + (lane >> 3)) * kFewRowBytes +
                           16 * (lane & 7)) = wb[rt][i];
#pragma unroll
        for (int s = 0; s < 2; s++) {
            u32x4 af[RT];
#pragma unroll
            for (int rt = 0; rt < RT; rt++)
                af[rt] = *(const u32x4 *)(stage + (16 * rt + r16) * kFewRowBytes +
                                          16 * (4 * s + q));
#pragma unroll
            for (int rt = 0; rt < RT; rt++)
#pragma unroll
                for (int mt = 0; mt < MT; mt++)
                    acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, af[rt]), __builtin_bit_cast(bf16x8, xb[s][mt]),
                        acc[rt][mt], 0, 0, 0);
        }
    }

    __syncthreads();                  // every wavefront is done with its stage
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
            red[w][rt][mt][lane] = acc[rt][mt];
    __syncthreads();
    // accumulator e of lane l: output n = 16*rt + 4*(l/16) + e, token 16*mt + l%16
    for (int t = w; t < RT * MT; t += W) {
        const int rt = t / MT, mt = t - rt * MT;
        f32x4 v = red[0][rt][mt][lane];
#pragma unroll
        for (int u = 1; u < W; u++)
            v += red[u][rt][mt][lane];
        const int m = 16 * mt + r16;
        const int n = n0 + 16 * rt + 4 * q;
        if (m < M && n < N) {
            u32x2 o;
            o.x = pack_bf16x2(v.x, v.y);
            o.y = pack_bf16x2(v.z, v.w);
            *(u32x2 *)(C + (int64_t)m * N + n) = o;
        }
    }
}

}  // namespace

bool gemm_small_fits(int64_t M, int64_t K, int64_t N)
{
    return M >= 1 && M <= kGemmSmallMaxM && K % 1024 == 0 && N % 16 == 0;
}

int32_t launch_gemm_small(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M,
                          int64_t K, int64_t N, const Launch &l)
{
    const int cus = device_cus();
    // row tiles of 16 per workgroup: about one workgroup per CU, at most 5
    // (the LDS stage of twelve wavefronts); wider N takes more rounds
    const int64_t tiles = N / 16;
    int rt = (int)((tiles + cus - 1) / cus);
    if (rt > kFewMaxRowTiles)
        rt = kFewMaxRowTiles;
    const int mt = (int)((M + 15) / 16);
    if (mt > 4)
        rt = kFewMaxRowTiles;     // five to eight token tiles: one shape, 80 rows a workgroup
    // twelve wavefronts for one or two token tiles, eight (whose partial sums
    // still fit in LDS) for three or four
    const int waves = mt <= 2 ? 12 : mt <= 4 ? 8 : 4;
    const dim3 grid((unsigned)((tiles + rt - 1) / rt)), block(64 * waves);
#define ENGRAM_FEW_CASE(R_, T_, W_)                                                              \
    if (rt == R_ && mt == T_) {                                                                  \
        dispatch(gemm_few_kernel<R_, T_, W_>, grid, block, l, true, true, x, w, y, (int)M,       \
                 (int)N, (int)K);                                                                \
        return launch_status("engram few-token gemm kernel");                                   \
    }
#define ENGRAM_FEW_ROW(R_)                                                                       \
    ENGRAM_FEW_CASE(R_, 1, 12) ENGRAM_FEW_CASE(R_, 2, 12) ENGRAM_FEW_CASE(R_, 3, 8)               \
    ENGRAM_FEW_CASE(R_, 4, 8)
    ENGRAM_FEW_ROW(1) ENGRAM_FEW_ROW(2) ENGRAM_FEW_ROW(3) ENGRAM_FEW_ROW(4) ENGRAM_FEW_ROW(5)
    ENGRAM_FEW_CASE(5, 5, 4) ENGRAM_FEW_CASE(5, 6, 4) ENGRAM_FEW_CASE(5, 7, 4)
    ENGRAM_FEW_CASE(5, 8, 4)
#undef ENGRAM_FEW_ROW
#undef ENGRAM_FEW_CASE
    return fail(ENGRAM_E_UNSUPPORTED, "engram small gemm: %lld tokens", (long long)M);
}

}  // namespace engram
