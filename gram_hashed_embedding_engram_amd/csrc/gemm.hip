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

typedef __attribute__((address_space(1))) const void *gptr_t;
typedef __attribute__((address_space(3))) void *lptr_t;

constexpr int TILE_SLOTS = (BM + BN) * KCH;   // 16-byte LDS slots per buffer (64 KiB)

__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t *__restrict__ A,
                                                   const uint16_t *__restrict__ B,
                                                   uint16_t *__restrict__ C, int M, int N, int K,
                                                   int tiles_m, int tiles_n)
{
    // [buffer][256 token rows, then 256 wkv rows][8 chunks]
    __shared__ u32x4 smem[2][TILE_SLOTS];

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

    // ---- loader: each wave fills 64 rows of the token tile and 64 rows of
    // the wkv tile, 8 rows (1 KiB) per direct-to-LDS load.  A load writes
    // lane l's 16 bytes to LDS slot l of its 64-slot block, so lane l takes
    // row 8j + l/8 of the block and the global chunk that belongs in LDS
    // slot l%8 of that row under the swizzle.
    const int lrow = lane >> 3, lslot = lane & 7;
    int aoff[8], boff[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int row = wave * 64 + 8 * j + lrow;
        const int chunk = lslot ^ swizzle(row);
        aoff[j] = min(m0 + row, M - 1) * K + chunk * 8;
        boff[j] = min(n0 + row, N - 1) * K + chunk * 8;
    }
    auto issue_loads = [&](int kt, int buf) {
        const int k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            __builtin_amdgcn_global_load_lds((gptr_t)(A + aoff[j] + k0),
                                             (lptr_t)&smem[buf][(wave * 64 + 8 * j) * KCH], 16,
                                             0, 0);
            __builtin_amdgcn_global_load_lds((gptr_t)(B + boff[j] + k0),
                                             (lptr_t)&smem[buf][(BM + wave * 64 + 8 * j) * KCH],
                                             16, 0, 0);
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                acc[i][j][e] = 0.0f;

    // fragment rows of this lane: 32-row blocks, row within block = lane % 32
    const int fr = lane & 31, fhalf = lane >> 5;
    const int fsw = swizzle(fr);
    auto read_frags = [&](int buf, int kk, bf16x8 *fa, bf16x8 *fb) {
        const int ch = (2 * kk + fhalf) ^ fsw;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            fa[i] = __builtin_bit_cast(bf16x8,
                                       smem[buf][(BM + wn * 128 + i * 32 + fr) * KCH + ch]);
            fb[i] = __builtin_bit_cast(bf16x8, smem[buf][(wm * 128 + i * 32 + fr) * KCH + ch]);
        }
    };

    // Pipeline of one K step (4 sub-steps of 16): the next step's tiles are
    // requested first (direct to the other LDS buffer); sub-step kk's 16 MFMAs
    // run while sub-step kk+1's fragments are read, one LDS read interleaved
    // after each MFMA; before the last sub-step the workgroup meets at the
    // barrier (the next tiles have landed, every wave is done with this
    // buffer) and the next step's first fragments are read behind the last
    // sub-step's MFMAs.
    issue_loads(0, 0);
    __syncthreads();
    bf16x8 fa[2][4], fb[2][4];
    read_frags(0, 0, fa[0], fb[0]);
    const int KT = K / BK;
    for (int kt = 0; kt < KT; kt++) {
        const int cur = kt & 1;
        // the last step reloads its own tile into the idle buffer instead of
        // branching, so the loop body stays one block the scheduler can
        // interleave (the extra tile is never read)
        issue_loads(min(kt + 1, KT - 1), cur ^ 1);
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            if (kk + 1 < BK / 16) {
                read_frags(cur, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
            } else {
                __syncthreads();
                read_frags(cur ^ 1, 0, fa[0], fb[0]);
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        fa[kk & 1][i], fb[kk & 1][j], acc[i][j], 0, 0, 0);
            if (kk == 0) {
#pragma unroll
                for (int r = 0; r < 8; r++) {
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global->LDS load
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                }
#pragma unroll
                for (int r = 0; r < 8; r++) {
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 8; r++) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }
            __builtin_amdgcn_sched_barrier(0);      // one sub-step per scheduling region
        }
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
                    int64_t N, const Launch &l)
{
    if (M == 0)
        return ENGRAM_OK;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    dispatch(gemm_kernel, dim3((unsigned)tiles), dim3(256), l, true, true, x, w, y, (int)M, (int)N,
             (int)K, tiles_m, tiles_n);
    return launch_status("engram gemm kernel");
}

}  // namespace engram
