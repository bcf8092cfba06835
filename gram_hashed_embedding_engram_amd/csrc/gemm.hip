// Stage 3 at many tokens: the wkv projection as a bf16 MFMA GEMM for gfx950
// (atlascybernetics "spark_model/layers/engram_v41.rs", module doc stage 3:
// [tokens, cols*head_dim] x wkv^T -> [tokens, dim*(hc+1)], a dense bf16 GEMM
// with f32 accumulation and bf16 output; metrale "deepseek_v41_ref/engram.rs",
// linear_bf16).
//
// C[M][N] = A[M][K] * B[N][K]^T: A = the gathered rows (tokens), B = wkv, both
// K-contiguous.
//
// Tiling: a 512-thread workgroup owns a 256-token x 320-output tile and walks
// K in tiles of 32.  Its eight wavefronts sit two to a SIMD, and each owns a
// 128-token x 80-output piece as 8 x 5 blocks of v_mfma_f32_16x16x32_bf16
// (160 f32 accumulators a lane).  On gfx950 the 16x16x32 form sustains a
// higher rate than the 32x32x16 one, and the two wavefronts of a SIMD keep
// the matrix core fed while either of them waits.  The two wavefronts of a
// SIMD take turns (ping-pong): while one issues the 40 MFMAs of its current
// K tile from registers, the other reads its 13 operand fragments of the next
// K tile from LDS and issues its share of the global loads.  A workgroup
// barrier ends every phase, so group 0 (wavefronts 0-3) always runs one
// phase ahead of group 1 (wavefronts 4-7).  The 256x320 tile is as large as
// the registers of two wavefronts a SIMD allow.  320 outputs divide 20480,
// and 4096 x 20480 makes 1024 tiles, four full rounds of 256 CUs.  For a few
// hundred tokens, whose 256-token tiles would leave CUs idle, the same kernel
// runs with 128-token tiles (four token blocks a wavefront instead of eight).
//
// Data movement: global memory goes straight to LDS (buffer_load ... lds, 1
// KiB a load, no register staging) into a 4-stage ring of 36 KiB stages, so
// three K tiles are in flight while the fourth is read.  Group 0 loads the
// 256 token rows of a stage (four loads a wavefront) and group 1 the 320 wkv
// rows (five).  Each wavefront waits only for its own loads (s_waitcnt
// vmcnt, which counts in issue order) before the barrier that hands a stage
// to its readers.  Rows are stored in LDS as 4 chunks of 16 bytes, with chunk
// c of row r at c ^ swizzle(r), so the 16-byte fragment reads of 16
// consecutive rows spread over all banks.
//
// Launch order: gfx950 dispatches consecutive workgroups to its 8 XCDs in
// turn, each XCD with its own L2.  The workgroup id is remapped so that each
// XCD works on one contiguous range of tiles, walked in groups of 8 token
// tiles per wkv tile.  The 32 workgroups resident on one XCD then share
// their token and wkv panels in that XCD's L2.
#include "common.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 320;            // outputs per tile
constexpr int BK = 32;             // K per stage
constexpr int KCH = BK / 8;        // 16-byte chunks per tile row (4)
constexpr int NSTAGE = 4;          // LDS stages
constexpr int AHEAD = NSTAGE - 1;  // K tiles in flight ahead of the one being read
constexpr int GROUP_M = 8;         // token tiles walked per wkv tile
constexpr int XCDS = 8;
constexpr int WB = 5;              // 16-output MFMA blocks per wavefront (80 outputs)
constexpr int LW = BN / 16 / 4;    // 1 KiB wkv-row loads per group-1 wavefront per stage (5)

// The token side of a tile, for TB 16-token MFMA blocks per wavefront: 256
// tokens a tile at TB = 8 (the prefill tile), 128 at TB = 4 (twice the tiles
// for a few hundred tokens, whose 256-token tiles leave CUs idle).
template <int TB>
struct TokenSide {
    static constexpr int BM = 32 * TB;                 // tokens per tile
    static constexpr int NF = TB + WB;                 // fragments per wavefront per K tile
    static constexpr int LT = BM / 16 / 4;             // token-row loads per group-0 wavefront
    static constexpr int STAGE_SLOTS = (BM + BN) * KCH;   // 16-byte LDS slots per stage
    static_assert(NSTAGE * STAGE_SLOTS * 16 <= 160 * 1024, "LDS stages");
    static_assert(LT <= LW, "per-wavefront load offsets sized for the larger share");
};

typedef __attribute__((address_space(3))) void *lptr_t;

// LDS position of 16-byte chunk c of tile row r: c ^ swizzle(r).  Among any
// 16 consecutive rows read at one chunk, the rows that share a 256-byte bank
// line land on 4 different positions, and so do those that share r % 2
// within any 8, so a 16-byte fragment read hits distinct banks whether a
// pass serves 8 or 16 lanes.
__device__ __forceinline__ int swizzle(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }

// Wait until at most N of this wavefront's vector-memory loads are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_loads()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for this wavefront's LDS reads.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Meet the workgroup, with nothing moved across by the scheduler.
__device__ __forceinline__ void phase_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int TB>
__global__ __launch_bounds__(512) void gemm_kernel(const uint16_t *__restrict__ A,
                                                   const uint16_t *__restrict__ B,
                                                   uint16_t *__restrict__ C, int M, int N, int K,
                                                   int tiles_m, int tiles_n)
{
    constexpr int BM = TokenSide<TB>::BM, NF = TokenSide<TB>::NF, LT = TokenSide<TB>::LT;
    constexpr int STAGE_SLOTS = TokenSide<TB>::STAGE_SLOTS;
    // [stage][BM token rows, then 320 wkv rows][4 chunks]
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

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, simd = wave & 3;      // wavefronts s and s+4 share SIMD s
    const int th = simd & 1;                          // token half of the tile
    const int oq = (simd >> 1) | (grp << 1);          // output quarter of the tile

    // ---- loader: a 1 KiB direct-to-LDS buffer load fills 16 rows x 64 bytes;
    // lane l takes row 16j + l/4 and the global chunk that belongs in slot
    // l%4 of that row under the swizzle.  The buffer descriptors bound each
    // operand, so rows past M or N read as zeros; the K position of a stage
    // travels in the scalar offset.
    const __amdgpu_buffer_rsrc_t rsA =
        __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, (int)((uint32_t)M * K * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc((void *)B, 0, (int)((uint32_t)N * K * 2), 0x00020000);
    const int lrow = lane >> 2, lslot = lane & 3;
    uint32_t goff[LW];
    int lbase[LW];
#pragma unroll
    for (int j = 0; j < LW; j++) {
        if (grp == 0) {               // token rows (BM/4)s .. (BM/4)s + BM/4-1
            const int row = simd * (BM / 4) + 16 * j + lrow;
            goff[j] = ((uint32_t)(m0 + row) * K + (lslot ^ swizzle(row)) * 8) * 2;
            lbase[j] = (simd * (BM / 4) + 16 * j) * KCH;
        } else {                      // wkv rows 80s .. 80s+79
            const int row = simd * 80 + 16 * j + lrow;
            goff[j] = ((uint32_t)(n0 + row) * K + (lslot ^ swizzle(row)) * 8) * 2;
            lbase[j] = (BM + simd * 80 + 16 * j) * KCH;
        }
    }
    const int KT = K / BK;
    // this wavefront's loads of K tile kt (past the end: the last tile again,
    // into a stage nobody reads any more)
    auto issue = [&](int kt) {
        const uint32_t kbytes = (uint32_t)min(kt, KT - 1) * BK * 2;
        const int st = kt % NSTAGE;
        if (grp == 0) {
#pragma unroll
            for (int j = 0; j < LT; j++)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lptr_t)&smem[st][lbase[j]], 16,
                                                         goff[j], kbytes, 0, 0);
        } else {
#pragma unroll
            for (int j = 0; j < LW; j++)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lptr_t)&smem[st][lbase[j]], 16,
                                                         goff[j], kbytes, 0, 0);
        }
    };

    f32x4 acc[WB][TB];
#pragma unroll
    for (int i = 0; i < WB; i++)
#pragma unroll
        for (int j = 0; j < TB; j++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                acc[i][j][e] = 0.0f;

    // fragment f of a K tile: f < WB -> wkv rows block f (the MFMA "A"
    // operand), f >= WB -> token rows block f-WB ("B"); lane l holds row l%16
    // of the block, K values 8(l/16) .. 8(l/16)+7 of the tile
    const int fr = lane & 15, fch = lane >> 4;
    bf16x8 frag[NF];
    auto read_tile = [&](int st) {
#pragma unroll
        for (int f = 0; f < NF; f++) {
            const int row = f < WB ? BM + oq * 80 + f * 16 + fr : th * (BM / 2) + (f - WB) * 16 + fr;
            frag[f] = __builtin_bit_cast(bf16x8, smem[st][row * KCH + (fch ^ swizzle(row))]);
        }
    };
    auto compute = [&]() {
#pragma unroll
        for (int i = 0; i < WB; i++)
#pragma unroll
            for (int j = 0; j < TB; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag[i], frag[WB + j],
                                                                    acc[i][j], 0, 0, 0);
    };

    // ---- pipeline.  Phase p of group 0 is phase p-1 of group 1; a K tile
    // is read by group 0 in one phase and by group 1 in the next.  Tile kt's
    // loads go out in the memory phases of tile kt-AHEAD (group 0's token
    // rows, then group 1's wkv rows) into stage kt % NSTAGE, which last held
    // tile kt-NSTAGE; group 1 read that tile in the phase before group 0's
    // memory phase of tile kt-AHEAD, a barrier earlier.  Before the barrier
    // that ends a phase, each wavefront waits for its own loads of the next
    // tile anyone reads:
    //   group 0 after reading tile k: nothing new (tile k's loads are done);
    //   group 0 after computing k: tile k+1 -> AHEAD-1 tiles of loads may pend;
    //   group 1 after reading k: tile k+1 (which group 0 reads next);
    //   group 1 after computing k-1: tile k (which it reads next).
#pragma unroll
    for (int t = 0; t < AHEAD; t++)
        issue(t);
    if (grp == 0)
        wait_loads<LT * (AHEAD - 1)>();
    else
        wait_loads<LW * (AHEAD - 1)>();
    phase_barrier();
    if (grp == 1)
        phase_barrier();              // group 1 runs one phase behind
    for (int kt = 0; kt < KT; kt++) {
        // memory phase: this wavefront's fragments of tile kt, its loads of
        // tile kt+AHEAD
        read_tile(kt % NSTAGE);
        issue(kt + AHEAD);
        wait_lds();
        if (grp == 1)
            wait_loads<LW * (AHEAD - 1)>();
        phase_barrier();
        // compute phase
        compute();
        if (grp == 0)
            wait_loads<LT * (AHEAD - 1)>();
        else
            wait_loads<LW * (AHEAD - 1)>();
        phase_barrier();
    }
    if (grp == 0)
        phase_barrier();              // every wavefront meets the same number of barriers
    // the trailing loads (reloads of the last tile) land before the
    // workgroup's LDS is released
    wait_loads<0>();

    // ---- epilogue: accumulator e of block (i, j) is output 16i + 4(lane/16)
    // + e of this wavefront's 80, token 16j + lane%16 of its 128: 4
    // consecutive outputs leave as 8 bytes (N is a multiple of 16, so the 4
    // are all in range or all past it)
#pragma unroll
    for (int j = 0; j < TB; j++) {
        const int m = m0 + th * (BM / 2) + j * 16 + fr;
        if (m >= M)
            continue;
        uint16_t *crow = C + (int64_t)m * N;
#pragma unroll
        for (int i = 0; i < WB; i++) {
            const int n = n0 + oq * 80 + i * 16 + fch * 4;
            if (n < N) {
                u32x2 v;
                v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                *(u32x2 *)(crow + n) = v;
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
    const int tiles_n = (int)((N + BN - 1) / BN);
    // 128-token tiles when 256-token ones would leave CUs idle and the
    // smaller ones still fit in one round (each output adds the same products
    // in the same order either way)
    const int cus = device_cus();
    const int64_t w8 = ((M + 255) / 256) * tiles_n, w4 = ((M + 127) / 128) * tiles_n;
    if (w8 < cus && w4 <= cus) {
        const int tiles_m = (int)((M + 127) / 128);
        dispatch(gemm_kernel<4>, dim3((unsigned)(tiles_m * tiles_n)), dim3(512), l, true, true,
                 x, w, y, (int)M, (int)N, (int)K, tiles_m, tiles_n);
    } else {
        const int tiles_m = (int)((M + 255) / 256);
        dispatch(gemm_kernel<8>, dim3((unsigned)((int64_t)tiles_m * tiles_n)), dim3(512), l, true,
                 true, x, w, y, (int)M, (int)N, (int)K, tiles_m, tiles_n);
    }
    return launch_status("engram gemm kernel");
}

}  // namespace engram
