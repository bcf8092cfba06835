// Stage 3 at many tokens: the wkv projection as a bf16 MFMA GEMM for gfx950
// (atlascybernetics "spark_model/layers/engram_v41.rs", module doc stage 3:
// [tokens, cols*head_dim] x wkv^T -> [tokens, dim*(hc+1)], a dense bf16 GEMM
// with f32 accumulation and bf16 output; metrale "deepseek_v41_ref/engram.rs",
// linear_bf16).
//
// C[M][N] = A[M][K] * B[N][K]^T: A = the gathered rows (tokens), B = wkv, both
// K-contiguous.
//
// Tiling: a 256-thread workgroup (4 wavefronts, one per SIMD) owns a 256x256
// output tile and walks K in steps of 64.  Each wavefront owns a 128x128
// quarter as 4x4 v_mfma_f32_32x32x16_bf16 blocks (256 f32 accumulators a
// lane).  The matrix-core "A" operand is fed from wkv and the "B" operand from
// the tokens, so each lane's accumulators hold 4 consecutive outputs of one
// token and leave as 8-byte stores.
//
// Data movement: the next K step is fetched from global memory into registers
// (16 bytes a load, 8 consecutive lanes covering one 128-byte row segment)
// while the matrix cores work on the current step from LDS; the registers are
// then written to the other half of a double-buffered LDS (2 x 64 KiB), one
// barrier per step.  Rows are stored in LDS as 8 chunks of 16 bytes with chunk
// c of row r at position c ^ ((r & 7) ^ ((r >> 3) & 1)), so the 16-byte
// fragment reads of 32 consecutive rows spread over all banks.
//
// Launch order: gfx950 dispatches consecutive workgroups to its 8 XCDs in
// turn, each XCD with its own L2.  The workgroup id is remapped so that each
// XCD works on one contiguous range of tiles, and that range is walked in
// groups of 4 token tiles per wkv tile, so the workgroups resident on one XCD
// share their A and B panels in that XCD's L2.
#include "common.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256;            // tokens per tile
constexpr int BN = 256;            // outputs per tile
constexpr int BK = 64;             // K per step
constexpr int KCH = BK / 8;        // 16-byte chunks per tile row
constexpr int GROUP_M = 4;         // token tiles walked per wkv tile
constexpr int XCDS = 8;

__device__ __forceinline__ int swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t *__restrict__ A,
                                                   const uint16_t *__restrict__ B,
                                                   uint16_t *__restrict__ C, int M, int N, int K,
                                                   int tiles_m, int tiles_n)
{
    __shared__ u32x4 sA[2][BM * KCH];
    __shared__ u32x4 sB[2][BN * KCH];

    // ---- tile of this workgroup: XCD-contiguous ranges, grouped raster
    const int G = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int xcd = b % XCDS, slot = b / XCDS;
    const int per = G / XCDS, rem = G % XCDS;
    const int L = xcd * per + min(xcd, rem) + slot;
    const int in_group = GROUP_M * tiles_n;
    const int first_m = (L / in_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (L % in_group) % gsize;
    const int tn = (L % in_group) / gsize;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    // ---- global -> register mapping: chunk (row = 32*j + tid/8, c = tid%8)
    const int lrow = tid >> 3, lc = tid & 7;
    const int kc = K >> 3;                          // 16-byte chunks per matrix row
    const u32x4 *A4 = (const u32x4 *)A;
    const u32x4 *B4 = (const u32x4 *)B;
    uint32_t aoff[8], boff[8];
    int sidx[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int row = 32 * j + lrow;
        const int am = min(m0 + row, M - 1), bn = min(n0 + row, N - 1);
        aoff[j] = (uint32_t)am * (uint32_t)kc + lc;
        boff[j] = (uint32_t)bn * (uint32_t)kc + lc;
        sidx[j] = row * KCH + (lc ^ swizzle(row));
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                acc[i][j][e] = 0.0f;

    u32x4 ra[8], rb[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        ra[j] = A4[aoff[j]];
        rb[j] = B4[boff[j]];
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
        sA[0][sidx[j]] = ra[j];
        sB[0][sidx[j]] = rb[j];
    }
    __syncthreads();

    // fragment rows of this lane: 32-row blocks, row within block = lane % 32
    const int fr = lane & 31, fhalf = lane >> 5;
    const int fsw = swizzle(fr);
    const int KT = K / BK;
    for (int kt = 0; kt < KT; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < KT) {
            const uint32_t adv = (uint32_t)(kt + 1) * KCH;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                ra[j] = A4[aoff[j] + adv];
                rb[j] = B4[boff[j] + adv];
            }
        }
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            const int ch = (2 * kk + fhalf) ^ fsw;
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int rn = wn * 128 + i * 32 + fr;
                fa[i] = __builtin_bit_cast(bf16x8, sB[cur][rn * KCH + ch]);
                const int rm = wm * 128 + i * 32 + fr;
                fb[i] = __builtin_bit_cast(bf16x8, sA[cur][rm * KCH + ch]);
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < KT) {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                sA[cur ^ 1][sidx[j]] = ra[j];
                sB[cur ^ 1][sidx[j]] = rb[j];
            }
        }
        __syncthreads();
    }

    // ---- epilogue: accumulator e of block (i, j) is output
    // n = 32i + 8(e/4) + 4(lane/32) + e%4 of this wave's 128 outputs, token
    // m = 32j + lane%32 of its 128 tokens; 4 consecutive n leave as 8 bytes
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int m = m0 + wm * 128 + j * 32 + fr;
        if (m >= M)
            continue;
        uint16_t *crow = C + (int64_t)m * N;
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int n = n0 + wn * 128 + i * 32 + g * 8 + fhalf * 4;
                if (n < N) {
                    u32x2 v;
                    v.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
                    v.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                    *(u32x2 *)(crow + n) = v;
                }
            }
        }
    }
}

}  // namespace

int32_t launch_gemm(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M, int64_t K,
                    int64_t N, hipStream_t s)
{
    if (M == 0)
        return ENGRAM_OK;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)tiles), dim3(256), 0, s, x, w, y, (int)M,
                       (int)N, (int)K, tiles_m, tiles_n);
    return launch_status("engram gemm kernel");
}

}  // namespace engram
