// Stage 1: the n-gram hash (atlascybernetics "spark_model/layers/engram_v41.rs",
// EngramHasher::hash; metrale "deepseek_v41_ref/engram.rs",
// NgramHashState::forward), data-parallel on the GPU.
//
// One thread per (sequence, token, layer, head) for B sequences at one
// common position (NgramHashState's batch rows, each with its own cache).
// Each thread rebuilds its token's window of compressed ids: a position
// inside this call is read through the token map from the call's own ids, a
// position before it from its sequence's history row, so no thread reads a
// history entry another thread of the same launch writes.  The first thread
// of each token records the token's compressed id in the history for later
// calls.
//
// Arithmetic: the window hash is kept in uint64 (wrapping multiply and XOR
// are the two's-complement i64 operations of the pages); the remainder is
// taken as signed i64 and moved into [0, prime) (Euclidean remainder).
#include "common.h"

namespace engram {
namespace {

__global__ __launch_bounds__(256) void hash_kernel(const HashConsts c,
                                                   const int64_t *__restrict__ token_map,
                                                   const int32_t *__restrict__ ids_all, int64_t B,
                                                   int64_t T, int64_t start_pos,
                                                   int64_t *__restrict__ history_all,
                                                   int64_t hist_stride,
                                                   int64_t *__restrict__ row_ids,
                                                   int32_t *__restrict__ err)
{
    const int64_t per_token = (int64_t)c.nl * c.nh;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= B * T * per_token)
        return;
    const int64_t bt = gid / per_token;              // token b*T + j of the call
    const int r = (int)(gid - bt * per_token);
    const int l = r / c.nh, head = r - l * c.nh;
    const int64_t b = bt / T, j = bt - b * T;
    const int32_t *ids = ids_all + b * T;
    int64_t *history = history_all + b * hist_stride;
    const int64_t pos = start_pos + j;

    // the window, newest first, with the sticky pad rule
    int64_t tok[ENGRAM_MAX_NGRAM];
    bool blocked = false, bad_own = false;
    int64_t own = 0;
#pragma unroll
    for (int k = 0; k < ENGRAM_MAX_NGRAM; k++) {
        if (k < c.ng) {
            const int64_t q = pos - k;
            int64_t src = 0;
            if (q < 0) {
                blocked = true;
            } else {
                if (q >= start_pos) {
                    const int32_t id = ids[q - start_pos];
                    if (id < 0 || (int64_t)id >= c.vocab) {
                        src = -1;                // reported, then hashed as unmapped
                        if (k == 0)
                            bad_own = true;
                    } else {
                        src = token_map[id];
                    }
                } else {
                    src = history[q];
                }
                if (src == -1)
                    blocked = true;
            }
            if (k == 0)
                own = src;
            tok[k] = blocked ? c.pad_id : src;
        }
    }
    if (l == 0 && head == 0) {
        history[pos] = own;
        if (bad_own && err)
            atomicOr(err, ENGRAM_DEVERR_TOKEN);
    }

    const int64_t *m = c.mult + l * c.ng;
    uint64_t rolling = (uint64_t)tok[0] * (uint64_t)m[0];
    int64_t *out = row_ids + (bt * c.nl + l) * c.cols;
#pragma unroll
    for (int i = 1; i < ENGRAM_MAX_NGRAM; i++) {
        if (i < c.ng) {
            rolling ^= (uint64_t)tok[i] * (uint64_t)m[i];
            const int col = (i - 1) * c.nh + head;
            const int slot = l * c.cols + col;
            out[col] = rem_euclid((int64_t)rolling, c.prime[slot]) + c.offset[slot];
        }
    }
}

}  // namespace

int32_t launch_hash(const HashConsts &c, const int64_t *token_map, const int32_t *ids, int64_t B,
                    int64_t T, int64_t start_pos, int64_t *history, int64_t hist_stride,
                    int64_t *row_ids, int32_t *err, const Launch &l)
{
    const int64_t threads = B * T * c.nl * c.nh;
    if (threads == 0)
        return ENGRAM_OK;
    const int64_t blocks = (threads + 255) / 256;
    dispatch(hash_kernel, dim3((unsigned)blocks), dim3(256), l, true, true, c, token_map, ids, B,
             T, start_pos, history, hist_stride, row_ids, err);
    return launch_status("engram hash kernel");
}

}  // namespace engram
