// A yardstick for the streaming projections: a kernel that does nothing but
// stream a buffer from memory, in the decode projection's access pattern
// (each wavefront reads 12 KiB rows -- one wkv row at 24 columns -- as twelve
// 1 KiB non-temporal loads, the next row's loads issued as soon as the
// current row has been consumed).  Its rate over an HBM-resident buffer is
// the practical ceiling of a read stream on the device, against which the
// decode kernels' rate is judged; it is not a step of the engram method.
//
// The data is XOR-folded so the loads are live: wavefront w of the fixed
// grid stores its fold in sink word w, so the XOR of the sink words is the
// XOR of every 32-bit word read.
#include "common.h"

namespace engram {
namespace {

constexpr int kCalibRowChunks = 12;      // 16-byte chunks per lane per row
constexpr int kCalibBlocks = ENGRAM_STREAM_SINK_WORDS / 4;   // 8 a CU on 256 CUs
static_assert(kCalibRowChunks * 1024 == ENGRAM_STREAM_ROW_BYTES, "row size");

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p,
                                                          int64_t n_rows,
                                                          uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    constexpr int64_t kRow = kCalibRowChunks * 64;
    u32x4 v[kCalibRowChunks];
    // rows past the end are clamped to the last row: loaded, never folded
    const u32x4 *row = p + min(wave, n_rows - 1) * kRow;
#pragma unroll
    for (int i = 0; i < kCalibRowChunks; i++)
        v[i] = __builtin_nontemporal_load(row + i * 64 + lane);
    uint32_t acc = 0u;
    for (int64_t r = wave; r < n_rows; r += n_waves) {
#pragma unroll
        for (int i = 0; i < kCalibRowChunks; i++)
            acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
        row = p + min(r + n_waves, n_rows - 1) * kRow;
#pragma unroll
        for (int i = 0; i < kCalibRowChunks; i++)
            v[i] = __builtin_nontemporal_load(row + i * 64 + lane);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if (lane == 0)
        sink[wave] = acc;
}

}  // namespace

int32_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, const Launch &l)
{
    const int64_t n_rows = bytes / (kCalibRowChunks * 1024);
    if (n_rows == 0)
        return ENGRAM_OK;
    dispatch(stream_read_kernel, dim3(kCalibBlocks), dim3(256), l, true, true,
             (const u32x4 *)src, n_rows, sink);
    return launch_status("engram stream-read kernel");
}

}  // namespace engram
