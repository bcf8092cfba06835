// Stage 3 for a few tokens (2..64): the wkv projection as a bf16 MFMA GEMM
// with a short token dimension (atlascybernetics "spark_model/layers/
// engram_v41.rs", module doc stage 3; metrale "deepseek_v41_ref/engram.rs",
// linear_bf16) -- several sequences' decode tokens, short prompts.
//
// C[M][N] = A[M][K] * B[N][K]^T with A = the tokens (M <= 64), B = wkv.  At
// this M the GEMM is a single pass over wkv (252 MB at the decode shape), so
// the kernel is laid out like a weight stream: one 256-thread workgroup per
// CU owns 16*RT consecutive output rows (RT <= 6) for all tokens, its four
// wavefronts split K in four, and every lane streams its rows' weights
// straight from HBM into v_mfma_f32_16x16x32_bf16 operands, two batches of
// four K steps in flight.  The matrix-core "A" operand is wkv (16 rows), "B" the tokens (16
// per tile, MT tiles), so each lane's accumulator holds 4 consecutive outputs
// of one token (8-byte stores).
//
// K order: wavefront w takes K values [w*K/4, (w+1)*K/4) in steps of 32, and
// a step hands lane group q (lanes 16q..16q+15) values 8q..8q+7 of it, so
// one load instruction reads 64 contiguous bytes of each of 16 rows.  The
// four wavefronts' partial sums meet in LDS and are added in wavefront order.
// Up to 32 tokens (one or two token tiles) a twelve-wavefront variant below
// takes over, streaming whole cache lines through LDS (19% faster at 8-32
// tokens on the decode shape).
#include "common.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSteps = 4;         // K steps (32 values) per batch of loads
constexpr int kMaxRowTiles = 6;   // 16-row tiles per workgroup

template <int RT, int MT>
__global__ __launch_bounds__(256) void gemm_small_kernel(const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ B,
                                                         uint16_t *__restrict__ C, int M, int N,
                                                         int K)
{
    __shared__ f32x4 red[4][RT][MT][64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int n0 = blockIdx.x * 16 * RT;
    const int nsteps = K >> 7;                 // 32-value steps of this wavefront
    const int k0 = w * (K >> 2) + 8 * q;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // this lane's rows of wkv (clamped: tile rows past N read row N-1 and are
    // never stored) and of the tokens (past M: zeros, no load)
    const u32x4 *brow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
        brow[rt] = (const u32x4 *)(B + (int64_t)min(n0 + 16 * rt + r16, N - 1) * K + k0);
    const u32x4 *arow[MT];
    bool avalid[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
        const int m = 16 * mt + r16;
        avalid[mt] = m < M;
        arow[mt] = (const u32x4 *)(A + (int64_t)(m < M ? m : 0) * K + k0);
    }

    f32x4 acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
            acc[rt][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    u32x4 wb[2][kSteps][RT], xb[2][kSteps][MT];
    // a row's consecutive steps back to back: the second half of each cache
    // line is read right after the first
    auto load = [&](int set, int s0) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int s = 0; s < kSteps; s++)
                wb[set][s][rt] = brow[rt][4 * (s0 + s)];
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int s = 0; s < kSteps; s++)
                xb[set][s][mt] = avalid[mt] ? arow[mt][4 * (s0 + s)] : zero;
    };
    auto compute = [&](int set) {
#pragma unroll
        for (int s = 0; s < kSteps; s++)
#pragma unroll
            for (int rt = 0; rt < RT; rt++)
#pragma unroll
                for (int mt = 0; mt < MT; mt++)
                    acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, wb[set][s][rt]),
                        __builtin_bit_cast(bf16x8, xb[set][s][mt]), acc[rt][mt], 0, 0, 0);
    };

    // batches of kSteps steps, two in flight (nsteps is a multiple of 2*kSteps)
    load(0, 0);
    for (int s0 = 0; s0 < nsteps; s0 += 2 * kSteps) {
        load(1, s0 + kSteps);
        compute(0);
        if (s0 + 2 * kSteps < nsteps)
            load(0, s0 + 2 * kSteps);
        compute(1);
    }

    // ---- the four K quarters meet in LDS, added in wavefront order
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
            red[w][rt][mt][lane] = acc[rt][mt];
    __syncthreads();
    // accumulator e of lane l: output n = 16*rt + 4*(l/16) + e, token 16*mt + l%16
    for (int t = w; t < RT * MT; t += 4) {
        const int rt = t / MT, mt = t - rt * MT;
        const f32x4 v = ((red[0][rt][mt][lane] + red[1][rt][mt][lane]) + red[2][rt][mt][lane]) +
                        red[3][rt][mt][lane];
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

// At one or two 16-token tiles the kernel above runs one wavefront a SIMD and
// streams wkv at about 4.9 TB/s; this one keeps three a SIMD busy (twelve a
// workgroup) and reaches about 6.0.  Wavefront w takes the 64-value K
// segments w, w+12, w+24, ... of the workgroup's 16*RT rows.  A segment of a
// 16-row tile arrives as two non-temporal loads of 8 rows x 128 contiguous
// bytes (whole cache lines: lane l takes row 8i + l/8, bytes 16*(l%8)),
// passes through the wavefront's own LDS buffer (rows padded to 144 bytes)
// and is read back in the MFMA layout (lane l: row l%16, values 8(l/16) ..
// of each 32-value step).  The twelve partial sums meet in LDS and are added
// in wavefront order.
constexpr int kFewWaves = 12;
constexpr int kFewSeg = 64;                        // K values a segment
constexpr int kFewRowBytes = 2 * kFewSeg + 16;     // LDS bytes a staged row
constexpr int kFewMaxRowTiles = 5;

template <int RT, int MT>
__global__ __launch_bounds__(64 * kFewWaves) void gemm_few_kernel(const uint16_t *__restrict__ A,
                                                                  const uint16_t *__restrict__ B,
                                                                  uint16_t *__restrict__ C, int M,
                                                                  int N, int K)
{
    constexpr int STAGE_B = kFewWaves * RT * 16 * kFewRowBytes;
    constexpr int RED_B = kFewWaves * RT * MT * 64 * 16;
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

    for (int j = w; j < nseg; j += kFewWaves) {
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
    for (int t = w; t < RT * MT; t += kFewWaves) {
        const int rt = t / MT, mt = t - rt * MT;
        f32x4 v = red[0][rt][mt][lane];
#pragma unroll
        for (int u = 1; u < kFewWaves; u++)
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
    return M >= 1 && M <= kGemmSmallMaxM && K % (128 * 2 * kSteps) == 0 && N % 16 == 0;
}

int32_t launch_gemm_small(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M,
                          int64_t K, int64_t N, const Launch &l)
{
    const int cus = device_cus();
    // row tiles of 16 per workgroup: about one workgroup per CU (at most 6
    // tiles: beyond that the operand registers spill at four token tiles)
    const int64_t tiles = N / 16;
    int rt = (int)((tiles + cus - 1) / cus);
    if (rt > kMaxRowTiles)
        rt = kMaxRowTiles;
    const int mt = (int)((M + 15) / 16);
    if (mt <= 2 && rt <= kFewMaxRowTiles) {
        const dim3 grid((unsigned)((tiles + rt - 1) / rt)), block(64 * kFewWaves);
#define ENGRAM_FEW_CASE(R_, T_)                                                                  \
        if (rt == R_ && mt == T_) {                                                              \
            dispatch(gemm_few_kernel<R_, T_>, grid, block, l, true, true, x, w, y, (int)M,       \
                     (int)N, (int)K);                                                            \
            return launch_status("engram few-token gemm kernel");                               \
        }
        ENGRAM_FEW_CASE(1, 1) ENGRAM_FEW_CASE(1, 2) ENGRAM_FEW_CASE(2, 1) ENGRAM_FEW_CASE(2, 2)
        ENGRAM_FEW_CASE(3, 1) ENGRAM_FEW_CASE(3, 2) ENGRAM_FEW_CASE(4, 1) ENGRAM_FEW_CASE(4, 2)
        ENGRAM_FEW_CASE(5, 1) ENGRAM_FEW_CASE(5, 2)
#undef ENGRAM_FEW_CASE
    }
    const dim3 grid((unsigned)((tiles + rt - 1) / rt)), block(256);
#define ENGRAM_SMALL_CASE(R_, T_)                                                                \
    if (rt == R_ && mt == T_) {                                                                  \
        dispatch(gemm_small_kernel<R_, T_>, grid, block, l, true, true, x, w, y, (int)M, (int)N, \
                 (int)K);                                                                        \
        return launch_status("engram small gemm kernel");                                       \
    }
#define ENGRAM_SMALL_ROW(R_)                                                                     \
    ENGRAM_SMALL_CASE(R_, 1) ENGRAM_SMALL_CASE(R_, 2) ENGRAM_SMALL_CASE(R_, 3)                   \
    ENGRAM_SMALL_CASE(R_, 4)
    ENGRAM_SMALL_ROW(1) ENGRAM_SMALL_ROW(2) ENGRAM_SMALL_ROW(3) ENGRAM_SMALL_ROW(4)
    ENGRAM_SMALL_ROW(5) ENGRAM_SMALL_ROW(6)
#undef ENGRAM_SMALL_ROW
#undef ENGRAM_SMALL_CASE
    return fail(ENGRAM_E_UNSUPPORTED, "engram small gemm: %lld tokens", (long long)M);
}

}  // namespace engram
