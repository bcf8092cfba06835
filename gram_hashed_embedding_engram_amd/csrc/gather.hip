// Stage 2: gather the hashed rows from an HBM-resident table and dequantise
// them to bf16 (atlascybernetics "spark_model/layers/engram_v41.rs", module
// doc stage 2 and rows_from_q2k; metrale "deepseek_v41_ref/engram.rs",
// regen_table and embed_rows).
//
// Output row r = t*cols + c holds table row ids[t*id_stride + c]; the rows of
// one token are contiguous, so the output is the [T, cols*head_dim] input of
// the projection.  Without ids the Q2_K kernel expands blocks 0..T-1 in order
// (the bf16 expansion of a weight matrix shipped as Q2_K blocks).
//
// Q2_K (84-byte blocks, only 4-byte aligned): a workgroup takes 64 rows at a
// time.  It first stages the 64 blocks in LDS with one coalesced dword load
// per (row, dword) -- 21 dwords a block -- spread over all 256 threads, then
// each half-wave expands one row from LDS: lane i writes values 8i..8i+7 as
// one 16-byte store, so a row leaves as one 512-byte coalesced write.  The
// rows are written once and next read by another kernel, so the stores are
// non-temporal (streamed out rather than kept in the caches: on the 5.9 GB
// table at 16 384 tokens the kernel went from 57-60 us to 45-46 us).
//
// Block layout (GGML k-quant; the pages give the size only): bytes 0..15
// scale/min nibbles of the 16 sub-blocks of 16 values, bytes 16..79 the 2-bit
// quants, bytes 80..83 fp16 d and dmin.  Value e uses quant byte
// 32*(e/128) + e%32 at bit 2*((e%128)/32) and sub-block e/16; for lane i
// (values 8i..8i+7) that is 8 consecutive quant bytes at 32*(i/16) + 8*(i%4),
// shift 2*((i%16)/4), sub-block i/2.  y = d*scale*q - dmin*min: both products
// are exact in f32, so the single subtraction and the bf16 rounding fix the
// result bit for bit.
//
// e4m3 (16-byte aligned rows): a thread expands 16 codes of one row with one
// 16-byte load and one scale, writing two 16-byte stores.  e4m3 times a
// power-of-two scale is exact in bf16.
#include "common.h"

namespace engram {
namespace {

constexpr int kQ2kRows = 64;          // rows staged per workgroup iteration
constexpr int kQ2kDwords = 21;        // 84 bytes

__global__ __launch_bounds__(256) void gather_q2k_kernel(const uint8_t *__restrict__ table,
                                                         int64_t n_table_rows,
                                                         const int64_t *__restrict__ ids,
                                                         int64_t id_stride, int32_t cols,
                                                         int64_t total_rows,
                                                         uint16_t *__restrict__ out,
                                                         int32_t *__restrict__ err)
{
    __shared__ uint32_t blk[kQ2kRows * kQ2kDwords];
    __shared__ int64_t row_off[kQ2kRows];
    const int tid = threadIdx.x;

    for (int64_t base = (int64_t)blockIdx.x * kQ2kRows; base < total_rows;
         base += (int64_t)gridDim.x * kQ2kRows) {
        if (tid < kQ2kRows) {
            const int64_t r = base + tid;
            int64_t off = -1;
            if (r < total_rows) {
                const int64_t t = r / cols;
                const int64_t c = r - t * cols;
                const int64_t id = ids ? ids[t * id_stride + c] : r;
                if (id >= 0 && id < n_table_rows)
                    off = id * ENGRAM_Q2K_ROW_BYTES;
                else if (err)
                    atomicOr(err, ENGRAM_DEVERR_ROW);
            }
            row_off[tid] = off;
        }
        __syncthreads();
        for (int w = tid; w < kQ2kRows * kQ2kDwords; w += 256) {
            const int rr = w / kQ2kDwords;
            const int d = w - rr * kQ2kDwords;
            const int64_t off = row_off[rr];
            blk[w] = off >= 0 ? *(const uint32_t *)(table + off + 4 * d) : 0u;
        }
        __syncthreads();

        const int i = tid & 31;               // lane within the row: values 8i..8i+7
        for (int rr = tid >> 5; rr < kQ2kRows; rr += 8) {
            const int64_t r = base + rr;
            if (r >= total_rows)
                break;
            u32x4 o = q2k_dequant8(blk + rr * kQ2kDwords, i);
            if (row_off[rr] < 0)
                o = u32x4{0u, 0u, 0u, 0u};
            __builtin_nontemporal_store(o, (u32x4 *)(out + r * 256 + 8 * i));
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void gather_e4m3_kernel(const uint8_t *__restrict__ codes,
                                                          const float *__restrict__ scales,
                                                          int64_t n_table_rows, int32_t head_dim,
                                                          int32_t scale_block,
                                                          const int64_t *__restrict__ ids,
                                                          int64_t id_stride, int32_t cols,
                                                          int64_t total_rows,
                                                          uint16_t *__restrict__ out,
                                                          int32_t *__restrict__ err)
{
    const int chunks = head_dim >> 4;      // 16 codes per thread
    const int nb = head_dim / scale_block;
    const int64_t total = total_rows * chunks;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = g / chunks;
        const int ch = (int)(g - r * chunks);
        const int64_t t = r / cols;
        const int64_t c = r - t * cols;
        const int64_t id = ids[t * id_stride + c];
        u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = o0;
        if (id >= 0 && id < n_table_rows) {
            const u32x4 v = *(const u32x4 *)(codes + id * head_dim + 16 * ch);
            const float s = scales[id * nb + (16 * ch) / scale_block];
            o0 = e4m3_dequant8(v.x, v.y, s);
            o1 = e4m3_dequant8(v.z, v.w, s);
        } else if (err && ch == 0) {
            atomicOr(err, ENGRAM_DEVERR_ROW);
        }
        u32x4 *dst = (u32x4 *)(out + r * head_dim + 16 * ch);
        __builtin_nontemporal_store(o0, dst);
        __builtin_nontemporal_store(o1, dst + 1);
    }
}

}  // namespace

int32_t launch_gather(const engram_table &tab, const int64_t *row_ids, int64_t T, int32_t cols,
                      int64_t id_stride, uint16_t *rows, int32_t *err, const Launch &l)
{
    const int64_t total_rows = T * cols;
    if (total_rows == 0)
        return ENGRAM_OK;
    if (tab.fmt == ENGRAM_FMT_Q2K) {
        int64_t blocks = (total_rows + kQ2kRows - 1) / kQ2kRows;
        if (blocks > 16384)
            blocks = 16384;
        dispatch(gather_q2k_kernel, dim3((unsigned)blocks), dim3(256), l, true, true, tab.d_data,
                 tab.n_rows, row_ids, id_stride, cols, total_rows, rows, err);
    } else {
        const int64_t threads = total_rows * (tab.head_dim / 16);
        int64_t blocks = (threads + 255) / 256;
        if (blocks > 16384)
            blocks = 16384;
        dispatch(gather_e4m3_kernel, dim3((unsigned)blocks), dim3(256), l, true, true, tab.d_data,
                 tab.d_scales, tab.n_rows, tab.head_dim, tab.scale_block, row_ids, id_stride, cols,
                 total_rows, rows, err);
    }
    return launch_status("engram gather kernel");
}

int32_t launch_dequant_q2k(const uint8_t *blocks, int64_t n_blocks, uint16_t *out,
                           const Launch &l)
{
    if (n_blocks == 0)
        return ENGRAM_OK;
    int64_t grid = (n_blocks + kQ2kRows - 1) / kQ2kRows;
    if (grid > 16384)
        grid = 16384;
    dispatch(gather_q2k_kernel, dim3((unsigned)grid), dim3(256), l, true, true, blocks, n_blocks,
             (const int64_t *)nullptr, (int64_t)1, (int32_t)1, n_blocks, out, (int32_t *)nullptr);
    return launch_status("engram dequant kernel");
}

}  // namespace engram
