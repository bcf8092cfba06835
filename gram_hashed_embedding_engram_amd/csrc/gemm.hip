// Stage 3 at many tokens: the wkv projection as a bf16 MFMA GEMM for gfx950
// (atlascybernetics "spark_model/layers/engram_v41.rs", module doc stage 3:
// [tokens, cols*head_dim] x wkv^T -> [tokens, dim*(hc+1)], a dense bf16 GEMM
// with f32 accumulation and bf16 output; metrale "deepseek_v41_ref/engram.rs",
// linear_bf16).
//
// C[M][N] = A[M][K] * B[N][K]^T: A = the gathered rows (tokens), B = wkv, both
// K-contiguous.
//
// Tiling: a 256-thread workgroup (4 wavefronts, one per SIMD) owns a 256-token
// x 320-output tile and walks K in tiles of 32.  Each wavefront owns a
// 128x160 quarter as 4x5 v_mfma_f32_32x32x16_bf16 blocks (320 f32
// accumulators a lane).  The bound is the rate at which operands reach a CU,
// so the tile is as large as the registers allow: 320 outputs take 10% fewer
// operand bytes per flop than 256 and still divide 20480 (4096 x 20480 is
// 1024 tiles, four full rounds of 256 CUs; 2048 tokens two).  The compiler
// keeps every MFMA accumulator in AGPRs, which hold 256 a lane, so the fifth
// output block of each wavefront (64 accumulators) is accumulated by MFMAs
// in their VGPR form, written out (mfma_vgpr).  The matrix-core "A" operand is
// fed from wkv and the "B" operand from the tokens, so each lane's
// accumulators hold 4 consecutive outputs of one token and leave as 8-byte
// stores.
//
// Data movement: global memory goes straight to LDS (buffer_load ... lds, 1
// KiB a load, no register staging) into a 4-stage ring of 36 KiB stages, so
// three K tiles are in flight while the matrix cores work on the fourth.
// Each tile's two 20-MFMA sub-steps are issued as groups of 2 MFMAs + 1 LDS
// fragment read of the next sub-step, with the next tile's 9 loads spread one
// per two groups; one workgroup barrier per tile.  Rows are stored in LDS as
// 4 chunks of 16 bytes with chunk c of row r at c ^ swizzle(r), so the
// 16-byte fragment reads of consecutive rows spread over all banks.
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256;            // tokens per tile
constexpr int NB = 5;              // 32-output MFMA blocks per wavefront
constexpr int BN = 64 * NB;        // outputs per tile (two wavefronts across)
constexpr int BK = 32;             // K per pipeline stage
constexpr int KCH = BK / 8;        // 16-byte chunks per tile row (4)
constexpr int NSTAGE = 4;          // LDS stages: NSTAGE-1 tiles in flight ahead of the one in use
constexpr int GROUP_M = 4;         // token tiles walked per wkv tile
constexpr int XCDS = 8;
constexpr int QN = 4 + NB;         // 1 KiB direct loads per wave per stage (4 token, NB wkv)
constexpr int NF = 4 + NB;         // MFMA fragments per wave per sub-step
constexpr int NG = 2 * NB;         // groups of 2 MFMAs per sub-step
constexpr int QA = (QN + 1) / 2;   // loads issued in a tile's first sub-step

typedef __attribute__((address_space(3))) void *lptr_t;

constexpr int STAGE_SLOTS = (BM + BN) * KCH;   // 16-byte LDS slots per stage (36 KiB)
static_assert(NSTAGE >= 3 && NSTAGE * STAGE_SLOTS * 16 <= 160 * 1024, "LDS stages");
static_assert(QA <= NB && QN - QA <= NB, "a tile's loads fit one per two groups");

// LDS position of 16-byte chunk c of tile row r: c ^ swizzle(r).  For any 16
// consecutive rows at one chunk, the rows sharing r % 4 (one 256-byte bank
// line) land on 4 different positions, and so do the rows sharing r % 2
// within any 8, so 16-byte fragment reads of consecutive rows hit distinct
// banks whether a pass serves 8 or 16 lanes.
__device__ __forceinline__ int swizzle(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }

// Wait until at most `pending` of this wave's global->LDS loads are still in
// flight (they complete in issue order) and its LDS reads are done, then
// meet the workgroup.  Written out because __syncthreads would also wait for
// the loads of the stages still being prefetched.
template <int PENDING>
__device__ __forceinline__ void stage_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(PENDING) : "memory");
}

// acc += a * b (32x32x16 bf16 MFMA) with acc in VGPRs.  The compiler knows
// nothing of this instruction's latency: the accumulator is touched only by
// this same MFMA (several MFMAs apart) until the epilogue, which first waits
// (mfma_vgpr_drain), and its operand registers are next overwritten more
// than a group of MFMAs later.
__device__ __forceinline__ void mfma_vgpr(f32x16 &acc, const bf16x8 &a, const bf16x8 &b)
{
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Wait states between the last mfma_vgpr and any other reader of its
// accumulators (a 16-pass MFMA result needs 18; 32 here).  The accumulators
// are operands, so no reader can be scheduled before the wait.
__device__ __forceinline__ void mfma_vgpr_drain(f32x16 (&acc)[4])
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
}

__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t *__restrict__ A,
                                                   const uint16_t *__restrict__ B,
                                                   uint16_t *__restrict__ C, int M, int N, int K,
                                                   int tiles_m, int tiles_n)
{
    // [stage][256 token rows, then 320 wkv rows][4 chunks]
    __shared__ u32x4 smem[NSTAGE][STAGE_SLOTS];

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

    // ---- loader: each wave fills 64 rows of the token tile and 80 rows of
    // the wkv tile, 16 rows (1 KiB) per direct-to-LDS buffer load.  A load
    // writes lane l's 16 bytes to LDS slot l of its 64-slot block, so lane l
    // takes row 16j + l/4 of the block and the global chunk that belongs in
    // slot l%4 of that row under the swizzle.  The buffer descriptors bound
    // each operand, so rows past M or N read as zeros; the K position of a
    // stage travels in the scalar offset.  (Buffer loads count only in the
    // vector-memory counter, so waiting for LDS reads never waits for them.)
    const __amdgpu_buffer_rsrc_t rsA =
        __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, (int)((uint32_t)M * K * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc((void *)B, 0, (int)((uint32_t)N * K * 2), 0x00020000);
    const int lrow = lane >> 2, lslot = lane & 3;
    uint32_t aoff[4], boff[NB];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int row = wave * 64 + 16 * j + lrow;
        aoff[j] = ((uint32_t)(m0 + row) * K + (lslot ^ swizzle(row)) * 8) * 2;
    }
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const int row = wave * 16 * NB + 16 * j + lrow;
        boff[j] = ((uint32_t)(n0 + row) * K + (lslot ^ swizzle(row)) * 8) * 2;
    }
    const int KT = K / BK;
    // one 1 KiB direct load: q < 4 -> token rows block q, q >= 4 -> wkv rows
    // block q-4
    auto load_one = [&](int kt, int q) {
        // past the end: reload the last tile (never read)
        const uint32_t kbytes = (uint32_t)min(kt, KT - 1) * BK * 2;
        const int st = kt % NSTAGE;
        if (q < 4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsA, (lptr_t)&smem[st][(wave * 64 + 16 * q) * KCH], 16, aoff[q], kbytes, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsB, (lptr_t)&smem[st][(BM + wave * 16 * NB + 16 * (q - 4)) * KCH], 16,
                boff[q - 4], kbytes, 0, 0);
    };

    // blocks i < NB-1 in AGPRs (the compiler's MFMA form), block NB-1 in VGPRs
    f32x16 acc[NB - 1][4], accv[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
#pragma unroll
        for (int e = 0; e < 16; e++)
            accv[j][e] = 0.0f;
#pragma unroll
        for (int i = 0; i < NB - 1; i++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                acc[i][j][e] = 0.0f;
    }

    // fragment rows of this lane: 32-row blocks, row within block = lane % 32
    const int fr = lane & 31, fhalf = lane >> 5;
    const int fsw = swizzle(fr);
    // fragment f of a sub-step: f < NB -> wkv rows block f ("A" operand),
    // f >= NB -> token rows block f-NB ("B" operand)
    auto read_one = [&](int st, int kk, int f) -> bf16x8 {
        const int ch = (2 * kk + fhalf) ^ fsw;
        const int row =
            f < NB ? BM + wn * 32 * NB + f * 32 + fr : wm * 128 + (f - NB) * 32 + fr;
        return __builtin_bit_cast(bf16x8, smem[st][row * KCH + ch]);
    };
    // group g of a sub-step: output blocks (g/2, 2(g%2)) and (g/2, 2(g%2)+1)
    auto mfma_pair = [&](int g, const bf16x8 (&f)[NF]) {
        const int i = g >> 1, j0 = 2 * (g & 1);
        if (i == NB - 1) {
            mfma_vgpr(accv[j0], f[i], f[NB + j0]);
            mfma_vgpr(accv[j0 + 1], f[i], f[NB + 1 + j0]);
        } else {
            acc[i][j0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], f[NB + j0], acc[i][j0],
                                                                 0, 0, 0);
            acc[i][j0 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], f[NB + 1 + j0],
                                                                     acc[i][j0 + 1], 0, 0, 0);
        }
    };

    // Pipeline.  Tiles kt+1..kt+NSTAGE-1 are in flight while tile kt is used.  A tile
    // is two sub-steps of 20 MFMAs.  Each sub-step is issued as 10 groups of
    // 2 MFMAs + 1 LDS read of the next sub-step's fragments (9 reads), with one
    // of the next tile's 9 direct loads in every other group: memory
    // instructions trickle between matrix-core instructions instead of
    // arriving in a burst that would stall the in-order issue of the MFMAs
    // behind them.  Before a tile's second sub-step the workgroup meets: tile
    // kt+1 has landed (the younger loads -- tiles kt+2.. and the first QA of
    // this tile's prefetch -- may still be pending) and every wave is done
    // with tile kt-1's stage, which this tile's prefetch overwrites.
    bf16x8 f0[NF], f1[NF];
#pragma unroll
    for (int t = 0; t < NSTAGE - 1; t++)
#pragma unroll
        for (int q = 0; q < QN; q++)
            load_one(t, q);
    stage_barrier<(NSTAGE - 2) * QN>();
#pragma unroll
    for (int f = 0; f < NF; f++)
        f0[f] = read_one(0, 0, f);
    for (int kt = 0; kt < KT; kt++) {
        const int st = kt % NSTAGE;
#pragma unroll
        for (int g = 0; g < NG; g++) {
            mfma_pair(g, f0);
            if (g < NF)
                f1[g] = read_one(st, 1, g);
            if ((g & 1) == 0 && (g >> 1) < QA)
                load_one(kt + NSTAGE - 1, g >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        stage_barrier<(NSTAGE - 3) * QN + QA>();
        __builtin_amdgcn_sched_barrier(0);
        const int nst = (kt + 1) % NSTAGE;
#pragma unroll
        for (int g = 0; g < NG; g++) {
            mfma_pair(g, f1);
            if (g < NF)
                f0[g] = read_one(nst, 0, g);
            if ((g & 1) == 0 && QA + (g >> 1) < QN)
                load_one(kt + NSTAGE - 1, QA + (g >> 1));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the trailing prefetches (reloads of the last tile) land before the
    // workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    mfma_vgpr_drain(accv);

    // ---- epilogue: accumulator e of block (i, j) is output
    // n = 32i + 8(e/4) + 4(lane/32) + e%4 of this wave's 160 outputs, token
    // m = 32j + lane%32 of its 128 tokens; 4 consecutive n leave as 8 bytes
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int m = m0 + wm * 128 + j * 32 + fr;
        if (m >= M)
            continue;
        uint16_t *crow = C + (int64_t)m * N;
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const f32x16 &a = i == NB - 1 ? accv[j] : acc[i < NB - 1 ? i : 0][j];
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int n = n0 + wn * 32 * NB + i * 32 + g * 8 + fhalf * 4;
                if (n < N) {
                    u32x2 v;
                    v.x = pack_bf16x2(a[4 * g], a[4 * g + 1]);
                    v.y = pack_bf16x2(a[4 * g + 2], a[4 * g + 3]);
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
