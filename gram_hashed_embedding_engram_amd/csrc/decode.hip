// Decode step of one engram layer in one launch: hash of the token's n-gram
// window (atlascybernetics "spark_model/layers/engram_v41.rs",
// EngramHasher::hash), gather + dequant of its cols table rows
// (rows_from_q2k; metrale "deepseek_v41_ref/engram.rs", regen_table and
// embed_rows) and the wkv projection at one token (EngramV41::gemv_k;
// linear_bf16).
//
// At one token the layer is one pass over wkv (252 MB at the decode shape);
// hashing 24 ids and dequantising 24 rows is a few microseconds of latency.
// Fused, that latency hides under the weight stream: every thread first reads
// its hash constants, every wavefront then puts its first wkv row in flight,
// and its workgroup hashes the token (one thread per (layer, column)),
// stages the needed 84-byte Q2_K blocks in LDS through the scalar cache (the
// token, its look-back and the blocks are scalar loads, which do not wait
// behind the weight loads in flight), expands them once per workgroup into
// the token's bf16 activations (12 KiB of LDS), which the wavefronts read back
// per row (registers hold only the weight row in flight, so four workgroups
// stay resident per CU).  The projection loop is the GEMV's: one wavefront
// per output row at a time, K/512 non-temporal 1 KiB loads in flight, the
// row brought into the one-token sub-block order of common.h through the
// wavefront's 2 KiB LDS buffer, one f32 wave sum, one bf16 rounding, the
// store issued after the next row's loads.  Workgroup 0 also writes the step's row ids, the dequantised rows
// and the history entry, so the workspace holds what the separate stages
// would have left there.
//
// With wkv registered as Q2_K blocks the projection loop is wkv_q2k.h's row
// dot product instead (41 MB a layer instead of 252 MB), reading the
// activations from LDS per sub-block.  With an e4m3 table (256-byte rows, too
// large to stage through scalar registers) the table loads are vector loads
// issued ahead of the first weight row, so waiting for them leaves the row in
// flight.  The several-sequence kernel below does the same for 2-4 tokens,
// one per sequence, in one pass over wkv.
//
// The step's position is a kernel argument, or -- for steps replayed from a
// captured graph -- a device word that the step's last gate advances
// (step_pos); either way it is checked against the history's length.
//
// The gate stays a launch of its own.  It needs every kv row, and doing it
// in the last workgroup to finish was measured slower: the completion count
// and the device-wide visibility of kv cost about 4 us per launch, and four
// gate rows on one compute unit take twice as long as the gate kernel's
// four workgroups.
#include "wkv_q2k.h"

namespace engram {
namespace {

constexpr int kDecodeBlocksPerCu = 4;
constexpr int kMaxChunks = kDecodeMaxCols * 32;   // 8-value chunks of the activations

// Everything a decode launch needs besides the hash constants and wkv.
struct DecodeArgs {
    const int64_t *token_map;
    const int32_t *ids;
    int64_t pos;
    int64_t *history;
    int32_t layer, first_layer;
    const uint8_t *table;
    const float *scales;
    int64_t n_rows;
    int32_t scale_block, reserved;
    uint16_t *y;
    int64_t N;
    int64_t *row_ids;
    uint16_t *rows;
    int32_t *err;
    int64_t hist_stride;     // history entries per sequence (several sequences)
    const int64_t *pos_word; // non-null: the step's position is read here (graph replay)
    int64_t max_seq;         // history entries a sequence, for that position's check
};

// A load of a value that no thread writes during the launch, through the
// scalar cache (constant address space; the address must be the same in every
// lane).  Vector loads complete in issue order, so a vector load issued after
// the weight row's loads cannot be waited for without waiting for the row;
// scalar loads have their own counter and do not queue behind it.
template <class T>
__device__ __forceinline__ T cload(const T *p)
{
    return *(const __attribute__((address_space(4))) T *)p;
}

__device__ __forceinline__ int64_t uniform64(int64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The step's position: the kernel argument, or -- for a replayed graph --
// the device word the previous step's last gate advanced.  A position past
// the history is reported (ok = false) and clamped, so reads stay in bounds
// and nothing is written there.
__device__ __forceinline__ int64_t step_pos(const DecodeArgs &a, bool &ok)
{
    if (!a.pos_word) {
        ok = true;
        return a.pos;
    }
    const int64_t p = cload(a.pos_word);
    ok = p >= 0 && p < a.max_seq;
    return ok ? p : (p < 0 ? 0 : a.max_seq - 1);
}

// The hash constants of the slot thread tid computes (layer tid / cols,
// column tid % cols).  Indexed per thread, they arrive by vector loads, so a
// decode kernel reads them first, before its first weight row: the wait for
// them then leaves the row's loads in flight.
struct SlotConsts {
    int64_t m[ENGRAM_MAX_NGRAM];
    int64_t prime, offset;
};

__device__ __forceinline__ SlotConsts slot_consts(const HashConsts &c)
{
    SlotConsts sc;
    const int slot = min((int)threadIdx.x, c.nl * c.cols - 1);
    const int l = slot / c.cols;
#pragma unroll
    for (int k = 0; k < ENGRAM_MAX_NGRAM; k++)      // in bounds: l*ng + k < MAX_LAYERS*MAX_NGRAM
        sc.m[k] = c.mult[l * c.ng + k];
    sc.prime = c.prime[slot];
    sc.offset = c.offset[slot];
    return sc;
}

// Hash of the token and gather + dequant of this layer's cols rows into the
// activations s_x by the NT threads of a workgroup (every workgroup;
// workgroup 0 also writes the row ids, the history entry and the dequantised
// rows).  Ends with s_x complete, chunk c at slot xslot(c).  The token, its
// look-back and (Q2_K) the table blocks come through the scalar cache, so
// nothing here waits for the weight loads the kernel issued before the call.
// e4m3 rows (256 bytes and their scales) are too large to stage through
// scalar registers: their vector loads go out first and the kernel's first
// weight row right after them (issue_row, called here for e4m3 tables only),
// so waiting for the table leaves the row in flight.
template <int FMT, int NT, class IssueRow>
__device__ __forceinline__ void decode_prologue(const HashConsts &c, const DecodeArgs &a,
                                                const SlotConsts &sc, int64_t *s_id,
                                                uint32_t *s_blk, u32x4 *s_x, IssueRow &&issue_row)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, and known so
    const int cols = c.cols;
    const int64_t kc = (int64_t)cols * 32;
    bool pos_ok;
    const int64_t pos = step_pos(a, pos_ok);
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // ---- the token's compressed id and its look-back (win[k]: k positions
    // back; -1 = unmapped or before the sequence start), the same in every thread
    int64_t win[ENGRAM_MAX_NGRAM];
    bool bad = false;
    if (a.first_layer) {
        const int32_t t = cload(a.ids);
        bad = t < 0 || (int64_t)t >= c.vocab;
        const int64_t mapped = cload(a.token_map + (bad ? 0 : t));
        win[0] = bad ? -1 : mapped;          // reported, then hashed as unmapped
    } else {
        win[0] = cload(a.history + pos);
    }
#pragma unroll
    for (int k = 1; k < ENGRAM_MAX_NGRAM; k++) {
        win[k] = -1;
        if (k < c.ng) {
            const int64_t q = pos - k;
            const int64_t v = cload(a.history + (q >= 0 ? q : 0));
            win[k] = q >= 0 ? v : -1;
        }
    }

    // ---- hash: thread (l, col) computes layer l's id of column col; every
    // workgroup needs its own layer's, workgroup 0 of the first layer writes all
    if (tid < c.nl * cols) {
        const int l = tid / cols, col = tid - l * cols;
        if (l == a.layer || (blockIdx.x == 0 && a.first_layer)) {
            const int ngram = col / c.nh + 2;     // column (n-2)*n_heads + head
            bool blocked = win[0] == -1;
            uint64_t r = (uint64_t)(blocked ? c.pad_id : win[0]) * (uint64_t)sc.m[0];
#pragma unroll
            for (int k = 1; k < ENGRAM_MAX_NGRAM; k++) {
                if (k < ngram) {
                    blocked = blocked || win[k] == -1;
                    r ^= (uint64_t)(blocked ? c.pad_id : win[k]) * (uint64_t)sc.m[k];
                }
            }
            const int slot = l * cols + col;
            const int64_t id = rem_euclid((int64_t)r, sc.prime) + sc.offset;
            if (blockIdx.x == 0) {
                a.row_ids[slot] = id;
                if (tid == 0 && a.first_layer) {
                    if (pos_ok)
                        a.history[pos] = win[0];
                    if (bad && a.err)
                        atomicOr(a.err, ENGRAM_DEVERR_TOKEN);
                    if (!pos_ok && a.err)
                        atomicOr(a.err, ENGRAM_DEVERR_POSITION);
                }
            }
            if (l == a.layer) {
                const bool in_table = id >= 0 && id < a.n_rows;
                if (!in_table && blockIdx.x == 0 && a.err)
                    atomicOr(a.err, ENGRAM_DEVERR_ROW);
                s_id[col] = in_table ? id : -1;
            }
        }
    }
    __syncthreads();

    // ---- gather + dequant of the cols rows into the activations in LDS
    if (FMT == ENGRAM_FMT_Q2K) {
        // wavefront w stages blocks w, w + NW, ...: a batch of kBatch blocks'
        // 21 dwords at a time by scalar loads (all issued before the first is
        // used: one memory round trip a batch), into lanes 0..20, then LDS.
        // A missing block (id -1) reads block 0 and stores zeros.  Three
        // blocks take 63 SGPRs: the 1024-thread kernel (at most two blocks a
        // wavefront, fewer SGPRs at its occupancy) batches two.
        constexpr int NW = NT / 64, kBatch = NW >= 16 ? 2 : 3;
        for (int r0 = wid; r0 < cols; r0 += kBatch * NW) {
            int64_t id[kBatch];
            const uint32_t *blk[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; b++) {
                const int r = r0 + b * NW;
                id[b] = r < cols ? uniform64(s_id[r]) : -1;
                blk[b] = (const uint32_t *)(a.table + (id[b] >= 0 ? id[b] : 0) *
                                                          ENGRAM_Q2K_ROW_BYTES);
            }
            uint32_t d[kBatch][21];
#pragma unroll
            for (int b = 0; b < kBatch; b++)
#pragma unroll
                for (int j = 0; j < 21; j++)
                    d[b][j] = cload(blk[b] + j);
#pragma unroll
            for (int b = 0; b < kBatch; b++) {
                uint32_t v = 0u;
#pragma unroll
                for (int j = 0; j < 21; j++)      // dword j into lane j (v_writelane)
                    asm("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(d[b][j]), "i"(j));
                const int r = r0 + b * NW;
                if (r < cols && lane < 21)
                    s_blk[r * 21 + lane] = id[b] >= 0 ? v : 0u;
            }
        }
        __syncthreads();
        for (int ch = tid; ch < kc; ch += NT) {
            const int r = ch >> 5;
            s_x[xslot(ch)] = s_id[r] >= 0 ? q2k_dequant8(s_blk + r * 21, ch & 31) : zero;
        }
    } else {
        // this thread's chunks tid, tid + NT, ...: every load unconditional
        // (past kc: the last chunk again; a missing row: row 0), all issued
        // before the weight row
        constexpr int NCH = (kMaxChunks + NT - 1) / NT;
        const int nb = 256 / a.scale_block;
        uint32_t w0[NCH], w1[NCH];
        float sv[NCH];
        bool live[NCH];
#pragma unroll
        for (int j = 0; j < NCH; j++) {
            const int ch = min(tid + j * NT, (int)kc - 1), r = ch >> 5, sub = ch & 31;
            const int64_t id = s_id[r];
            live[j] = tid + j * NT < kc && id >= 0;
            const int64_t idc = id >= 0 ? id : 0;
            const uint32_t *b = (const uint32_t *)(a.table + idc * 256 + 8 * sub);
            w0[j] = b[0];
            w1[j] = b[1];
            sv[j] = a.scales[idc * nb + (8 * sub) / a.scale_block];
        }
        __builtin_amdgcn_sched_barrier(0);      // the table loads stay ahead of the row's
        issue_row();
#pragma unroll
        for (int j = 0; j < NCH; j++)
            if (tid + j * NT < kc)
                s_x[xslot(tid + j * NT)] = live[j] ? e4m3_dequant8(w0[j], w1[j], sv[j]) : zero;
    }
    __syncthreads();
    if (blockIdx.x == 0)
        for (int ch = tid; ch < kc; ch += NT)
            ((u32x4 *)a.rows)[ch] = s_x[xslot(ch)];
}

template <int FMT, int NI>
__global__ __launch_bounds__(256) void decode_kernel(const HashConsts c, const DecodeArgs a,
                                                     const uint16_t *__restrict__ w)
{
    __shared__ int64_t s_id[kDecodeMaxCols];
    __shared__ uint32_t s_blk[kDecodeMaxCols * 21];
    __shared__ u32x4 s_x[kMaxChunks];
    __shared__ u32x4 s_stage[4][128];
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t K = (int64_t)c.cols * 256, kc = K >> 3, N = a.N;
    const int n_sb = c.cols * 16;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + tid) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    uint16_t *__restrict__ y = a.y;

    // ---- this thread's hash constants, then the first wkv row of this
    // wavefront (past the row's end, lanes load its last chunk again: loads
    // are unconditional, and the staged order never reads those chunks) --
    // with an e4m3 table, inside the prologue right after the table loads
    const SlotConsts sc = slot_consts(c);
    u32x4 wv[NI];
    auto issue_row = [&] {
        const u32x4 *wr = (const u32x4 *)(w + min(wave, N - 1) * K);
#pragma unroll
        for (int i = 0; i < NI; i++)
            wv[i] = __builtin_nontemporal_load(wr + min((int64_t)i * 64 + lane, kc - 1));
    };
    if constexpr (FMT == ENGRAM_FMT_Q2K)
        issue_row();

    decode_prologue<FMT, 256>(c, a, sc, s_id, s_blk, s_x, issue_row);

    // ---- projection: rows wave, wave + n_waves, ...  A row's result is
    // stored after the next row's loads are issued, so the loop's wait for
    // those loads does not also wait for the store.
    int64_t prev_n = -1;
    uint16_t prev_v = 0;
    for (int64_t n = wave; n < N; n += n_waves) {
        if (n != wave) {
            const u32x4 *wr = (const u32x4 *)(w + n * K);
#pragma unroll
            for (int i = 0; i < NI; i++)
                wv[i] = __builtin_nontemporal_load(wr + min((int64_t)i * 64 + lane, kc - 1));
        }
        if (lane == 0 && prev_n >= 0)
            y[prev_n] = prev_v;
        // the activations stay in LDS: registers hold only the weight row in
        // flight
        float acc = 0.0f, acc2 = 0.0f;
        for_each_subblock<NI>(wv, s_stage[tid >> 6], lane, n_sb,
                              [&](int s, const u32x4 &wa, const u32x4 &wb) {
                                  subblock_dot(wa, wb, s_x[128 * s + lane],
                                               s_x[128 * s + 64 + lane], acc, acc2);
                              });
        prev_v = f32_to_bf16(wave_sum(acc + acc2));
        prev_n = n;
    }
    if (lane == 0 && prev_n >= 0)
        y[prev_n] = prev_v;
}

// The same layer step with wkv as Q2_K blocks [N][K/256][84].  Here the
// projection is bound by the vector ALUs, so the prologue's arithmetic
// counts: a 1024-thread workgroup runs it once for sixteen wavefronts, and
// two workgroups share a CU (eight wavefronts a SIMD).
constexpr int kQ2kwThreads = 1024;
constexpr int kQ2kwBlocksPerCu = 2;

template <int FMT, int NSB>
__global__ __launch_bounds__(kQ2kwThreads, 8) void decode_q2kw_kernel(const HashConsts c,
                                                                   const DecodeArgs a,
                                                                   const uint8_t *__restrict__ wq)
{
    constexpr int NLD = q2k_row_loads<NSB>();
    __shared__ int64_t s_id[kDecodeMaxCols];
    __shared__ uint32_t s_blk[kDecodeMaxCols * 21];
    __shared__ u32x4 s_x[kMaxChunks];
    __shared__ uint32_t s_row[kQ2kwThreads / 64][kQ2kWkvMaxRowDwords];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int K = c.cols * 256, n_sb = K >> 4, row_dwords = 21 * (K >> 8);
    const int64_t N = a.N;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + tid) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const uint32_t *wd = (const uint32_t *)wq;

    // ---- this thread's hash constants, then the first row's blocks (with
    // an e4m3 table: inside the prologue, after the table loads)
    const SlotConsts sc = slot_consts(c);
    uint32_t r[NLD];
    auto issue_row = [&] {
        q2k_row_load<NLD>(wd + min(wave, N - 1) * row_dwords, row_dwords, lane, r);
    };
    if constexpr (FMT == ENGRAM_FMT_Q2K)
        issue_row();

    decode_prologue<FMT, kQ2kwThreads>(c, a, sc, s_id, s_blk, s_x, issue_row);

    // ---- projection, one row per wavefront at a time
    for (int64_t n = wave; n < N; n += n_waves) {
        q2k_row_stage<NLD>(s_row[wid], r, row_dwords, lane);
        if (n + n_waves < N)
            q2k_row_load<NLD>(wd + (n + n_waves) * row_dwords, row_dwords, lane, r);
        const float s = wave_sum(q2k_row_dot<NSB>(s_row[wid], s_x, n_sb, lane));
        if (lane == 0)
            a.y[n] = f32_to_bf16(s);
    }
}

// The same decode step for NB = 2..4 sequences that advance together (one
// token each, all at position a.pos, sequence b's history at history +
// b*hist_stride): one launch hashes, gathers and dequantises the NB tokens
// and projects them in one pass over wkv, every token in the one-token order
// (its kv equals a one-sequence step's bit for bit).  One 1024-thread
// workgroup per CU.  Wavefront b < NB hashes sequence b -- lane = slot (layer
// lane / cols, column lane % cols), so at most 64 slots -- with the token,
// its look-back and the hash constants as scalar loads (no vector load waits
// behind the weight row in flight).  All 16 wavefronts then stage the NB*cols
// Q2_K blocks through the scalar cache, and the workgroup expands them into
// the NB tokens' activations in LDS.
constexpr int kDecodeMultiThreads = 1024;

template <int FMT, int NB, int NI>
__global__ __launch_bounds__(kDecodeMultiThreads) void decode_multi_kernel(
    const HashConsts c, const DecodeArgs a, const uint16_t *__restrict__ w)
{
    constexpr int NW = kDecodeMultiThreads / 64;
    __shared__ int64_t s_id[NB * kDecodeMaxCols];
    __shared__ uint32_t s_blk[NB * kDecodeMaxCols * 21];
    __shared__ u32x4 s_x[NB * kMaxChunks];
    __shared__ u32x4 s_stage[NW][128];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cols = c.cols, nslots = c.nl * cols;
    const int64_t K = (int64_t)cols * 256, N = a.N;
    const int kc = cols * 32, kcp = (kc + 127) & ~127, n_sb = cols * 16;
    const int64_t wave = (int64_t)blockIdx.x * NW + wid;
    const int64_t n_waves = (int64_t)gridDim.x * NW;
    bool pos_ok;
    const int64_t pos = step_pos(a, pos_ok);
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // ---- this lane's hash slot constants (slot = lane: layer slot / cols,
    // column slot % cols), then the first wkv row of this wavefront (past
    // the row's end: its last chunk again).  The constants are taken right
    // after the row's loads are issued, in every wavefront: their loads stay
    // ahead of the row's, and the wait for them leaves the row in flight.
    const int slot = min(lane, nslots - 1);
    const int sl = slot / cols;
    int64_t m[ENGRAM_MAX_NGRAM];
#pragma unroll
    for (int k = 0; k < ENGRAM_MAX_NGRAM; k++)      // in bounds: l*ng + k < MAX_LAYERS*MAX_NGRAM
        m[k] = c.mult[sl * c.ng + k];
    const int64_t prime = c.prime[slot], offset = c.offset[slot];
    const u32x4 *wr0 = (const u32x4 *)(w + min(wave, N - 1) * K);
    u32x4 wv[NI];
#pragma unroll
    for (int i = 0; i < NI; i++)
        wv[i] = __builtin_nontemporal_load(wr0 + min(i * 64 + lane, kc - 1));
    asm volatile("" ::"v"(prime), "v"(offset), "v"(m[0]), "v"(m[1]), "v"(m[2]), "v"(m[3]),
                 "v"(m[4]), "v"(m[5]), "v"(m[6]), "v"(m[7]));

    // ---- hash of sequence b = wid
    if (wid < NB) {
        const int b = wid;
        int64_t *hist = a.history + (int64_t)b * a.hist_stride;
        int64_t win[ENGRAM_MAX_NGRAM];
        bool bad = false;
        if (a.first_layer) {
            const int32_t t = cload(a.ids + b);
            bad = t < 0 || (int64_t)t >= c.vocab;
            const int64_t mapped = cload(a.token_map + (bad ? 0 : t));
            win[0] = bad ? -1 : mapped;          // reported, then hashed as unmapped
        } else {
            win[0] = cload(hist + pos);
        }
#pragma unroll
        for (int k = 1; k < ENGRAM_MAX_NGRAM; k++) {
            win[k] = -1;
            if (k < c.ng) {
                const int64_t q = pos - k;
                const int64_t v = cload(hist + (q >= 0 ? q : 0));
                win[k] = q >= 0 ? v : -1;
            }
        }
        const int l = sl, col = slot - l * cols;
        if (lane < nslots && (l == a.layer || (blockIdx.x == 0 && a.first_layer))) {
            const int ngram = col / c.nh + 2;     // column (n-2)*n_heads + head
            bool blocked = win[0] == -1;
            uint64_t r = (uint64_t)(blocked ? c.pad_id : win[0]) * (uint64_t)m[0];
#pragma unroll
            for (int k = 1; k < ENGRAM_MAX_NGRAM; k++) {
                if (k < ngram) {
                    blocked = blocked || win[k] == -1;
                    r ^= (uint64_t)(blocked ? c.pad_id : win[k]) * (uint64_t)m[k];
                }
            }
            const int64_t id = rem_euclid((int64_t)r, prime) + offset;
            if (blockIdx.x == 0) {
                a.row_ids[(int64_t)b * nslots + slot] = id;
                if (lane == 0 && a.first_layer) {
                    if (pos_ok)
                        hist[pos] = win[0];
                    if (bad && a.err)
                        atomicOr(a.err, ENGRAM_DEVERR_TOKEN);
                    if (!pos_ok && a.err)
                        atomicOr(a.err, ENGRAM_DEVERR_POSITION);
                }
            }
            if (l == a.layer) {
                const bool in_table = id >= 0 && id < a.n_rows;
                if (!in_table && blockIdx.x == 0 && a.err)
                    atomicOr(a.err, ENGRAM_DEVERR_ROW);
                s_id[b * cols + col] = in_table ? id : -1;
            }
        }
    }
    __syncthreads();

    // ---- gather + dequant of the NB*cols rows into the activations
    const int nrows = NB * cols;
    if (FMT == ENGRAM_FMT_Q2K) {
        constexpr int kBatch = 2;      // 42 SGPRs of blocks a round trip
        for (int r0 = wid; r0 < nrows; r0 += kBatch * NW) {
            int64_t id[kBatch];
            const uint32_t *blk[kBatch];
#pragma unroll
            for (int bb = 0; bb < kBatch; bb++) {
                const int r = r0 + bb * NW;
                id[bb] = r < nrows ? uniform64(s_id[r]) : -1;
                blk[bb] = (const uint32_t *)(a.table + (id[bb] >= 0 ? id[bb] : 0) *
                                                           ENGRAM_Q2K_ROW_BYTES);
            }
            uint32_t d[kBatch][21];
#pragma unroll
            for (int bb = 0; bb < kBatch; bb++)
#pragma unroll
                for (int j = 0; j < 21; j++)
                    d[bb][j] = cload(blk[bb] + j);
#pragma unroll
            for (int bb = 0; bb < kBatch; bb++) {
                uint32_t v = 0u;
#pragma unroll
                for (int j = 0; j < 21; j++)      // dword j into lane j (v_writelane)
                    asm("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(d[bb][j]), "i"(j));
                const int r = r0 + bb * NW;
                if (r < nrows && lane < 21)
                    s_blk[r * 21 + lane] = id[bb] >= 0 ? v : 0u;
            }
        }
        __syncthreads();
        for (int ch = tid; ch < NB * kc; ch += kDecodeMultiThreads) {
            const int b = ch / kc, chl = ch - b * kc, r = b * cols + (chl >> 5);
            s_x[b * kcp + xslot(chl)] = s_id[r] >= 0 ? q2k_dequant8(s_blk + r * 21, chl & 31) : zero;
        }
    } else {
        const int nb = 256 / a.scale_block;
        for (int ch = tid; ch < NB * kc; ch += kDecodeMultiThreads) {
            const int b = ch / kc, chl = ch - b * kc, sub = chl & 31;
            const int64_t id = s_id[b * cols + (chl >> 5)];
            u32x4 o = zero;
            if (id >= 0) {
                const uint32_t *p = (const uint32_t *)(a.table + id * 256 + 8 * sub);
                o = e4m3_dequant8(p[0], p[1], a.scales[id * nb + (8 * sub) / a.scale_block]);
            }
            s_x[b * kcp + xslot(chl)] = o;
        }
    }
    __syncthreads();
    if (blockIdx.x == 0)
        for (int ch = tid; ch < NB * kc; ch += kDecodeMultiThreads) {
            const int b = ch / kc, chl = ch - b * kc;
            ((u32x4 *)a.rows)[(int64_t)b * kc + chl] = s_x[b * kcp + xslot(chl)];
        }

    // ---- projection: rows wave, wave + n_waves, ..., all NB tokens at once
    u32x4 *stage = s_stage[wid];
    for (int64_t n = wave; n < N; n += n_waves) {
        if (n != wave) {
            const u32x4 *wr = (const u32x4 *)(w + n * K);
#pragma unroll
            for (int i = 0; i < NI; i++)
                wv[i] = __builtin_nontemporal_load(wr + min(i * 64 + lane, kc - 1));
        }
        float acc[NB], acc2[NB];
#pragma unroll
        for (int t = 0; t < NB; t++)
            acc[t] = acc2[t] = 0.0f;
        for_each_subblock<NI>(wv, stage, lane, n_sb, [&](int s, const u32x4 &wa, const u32x4 &wb) {
#pragma unroll
            for (int t = 0; t < NB; t++)
                subblock_dot(wa, wb, s_x[t * kcp + 128 * s + lane],
                             s_x[t * kcp + 128 * s + 64 + lane], acc[t], acc2[t]);
        });
#pragma unroll
        for (int t = 0; t < NB; t++) {
            const float v = wave_sum(acc[t] + acc2[t]);
            if (lane == t)
                a.y[t * N + n] = f32_to_bf16(v);
        }
    }
}

}  // namespace

int32_t launch_decode_multi(const HashConsts &c, const int64_t *token_map, const int32_t *ids,
                            const DecodePos &pos, int64_t *history, int64_t hist_stride, int32_t layer,
                            bool first_layer, const engram_table &tab, const uint16_t *w,
                            uint16_t *y, int64_t N, int64_t *row_ids, uint16_t *rows,
                            int32_t *err, int64_t B, const Launch &l)
{
    const int cus = device_cus();
    const DecodeArgs a{token_map, ids,    pos.pos,  history, layer, first_layer ? 1 : 0,
                       tab.d_data, tab.d_scales, tab.n_rows, tab.scale_block, 0, y, N,
                       row_ids, rows, err, hist_stride, pos.word, pos.max_seq};
    const int ni = (c.cols * 256 + 511) / 512;
    int64_t blocks = (N + 15) / 16;
    if (blocks > cus)
        blocks = cus;
    const dim3 grid((unsigned)blocks), block(kDecodeMultiThreads);
    const bool q2k = tab.fmt == ENGRAM_FMT_Q2K;
#define ENGRAM_DM_CASE(B_, NI_)                                                                  \
    if (B == B_ && ni == NI_) {                                                                  \
        if (q2k)                                                                                 \
            dispatch(decode_multi_kernel<ENGRAM_FMT_Q2K, B_, NI_>, grid, block, l, true, true, c, \
                     a, w);                                                                      \
        else                                                                                     \
            dispatch(decode_multi_kernel<ENGRAM_FMT_E4M3, B_, NI_>, grid, block, l, true, true,   \
                     c, a, w);                                                                   \
        return launch_status("engram decode kernel");                                           \
    }
#define ENGRAM_DM_ROW(B_)                                                                        \
    ENGRAM_DM_CASE(B_, 1) ENGRAM_DM_CASE(B_, 2) ENGRAM_DM_CASE(B_, 3) ENGRAM_DM_CASE(B_, 4)      \
    ENGRAM_DM_CASE(B_, 5) ENGRAM_DM_CASE(B_, 6) ENGRAM_DM_CASE(B_, 7) ENGRAM_DM_CASE(B_, 8)      \
    ENGRAM_DM_CASE(B_, 9) ENGRAM_DM_CASE(B_, 10) ENGRAM_DM_CASE(B_, 11) ENGRAM_DM_CASE(B_, 12)   \
    ENGRAM_DM_CASE(B_, 13) ENGRAM_DM_CASE(B_, 14) ENGRAM_DM_CASE(B_, 15) ENGRAM_DM_CASE(B_, 16)
    ENGRAM_DM_ROW(2) ENGRAM_DM_ROW(3) ENGRAM_DM_ROW(4)
#undef ENGRAM_DM_ROW
#undef ENGRAM_DM_CASE
    return fail(ENGRAM_E_UNSUPPORTED, "engram decode: %lld sequences, %d columns", (long long)B,
                c.cols);
}

int32_t launch_decode(const HashConsts &c, const int64_t *token_map, const int32_t *ids,
                      const DecodePos &pos, int64_t *history, int32_t layer, bool first_layer,
                      const engram_table &tab, const uint16_t *w, const uint8_t *w_q2k,
                      uint16_t *y, int64_t N, int64_t *row_ids, uint16_t *rows, int32_t *err,
                      const Launch &l)
{
    const int cus = device_cus();
    const DecodeArgs a{token_map, ids,    pos.pos,  history, layer, first_layer ? 1 : 0,
                       tab.d_data, tab.d_scales, tab.n_rows, tab.scale_block, 0, y, N,
                       row_ids, rows, err, 0, pos.word, pos.max_seq};
    const int64_t K = (int64_t)c.cols * 256;
    int64_t blocks = (N + 3) / 4;
    const int64_t cap = (int64_t)cus * kDecodeBlocksPerCu;
    if (blocks > cap)
        blocks = cap;
    const dim3 grid((unsigned)blocks), block(256);
    const bool q2k_table = tab.fmt == ENGRAM_FMT_Q2K;
    if (w_q2k) {
        const int nsb = (int)((K + 1023) / 1024);
        int64_t qblocks = (N + kQ2kwThreads / 64 - 1) / (kQ2kwThreads / 64);
        if (qblocks > (int64_t)cus * kQ2kwBlocksPerCu)
            qblocks = (int64_t)cus * kQ2kwBlocksPerCu;
        const dim3 qgrid((unsigned)qblocks), qblock(kQ2kwThreads);
#define ENGRAM_DECODE_Q2KW_CASE(S_)                                                              \
    case S_:                                                                                     \
        if (q2k_table)                                                                           \
            dispatch(decode_q2kw_kernel<ENGRAM_FMT_Q2K, S_>, qgrid, qblock, l, true, true, c, a, \
                     w_q2k);                                                                     \
        else                                                                                     \
            dispatch(decode_q2kw_kernel<ENGRAM_FMT_E4M3, S_>, qgrid, qblock, l, true, true, c,   \
                     a, w_q2k);                                                                  \
        break;
        switch (nsb) {
            ENGRAM_DECODE_Q2KW_CASE(1) ENGRAM_DECODE_Q2KW_CASE(2) ENGRAM_DECODE_Q2KW_CASE(3)
            ENGRAM_DECODE_Q2KW_CASE(4) ENGRAM_DECODE_Q2KW_CASE(5) ENGRAM_DECODE_Q2KW_CASE(6)
            ENGRAM_DECODE_Q2KW_CASE(7) ENGRAM_DECODE_Q2KW_CASE(8)
        default:
            return fail(ENGRAM_E_UNSUPPORTED, "engram decode: %lld columns exceed %lld",
                        (long long)c.cols, (long long)kDecodeMaxCols);
        }
#undef ENGRAM_DECODE_Q2KW_CASE
        return launch_status("engram decode kernel");
    }
    const int64_t ni = (K + 511) / 512;
#define ENGRAM_DECODE_CASE(NI_)                                                                  \
    case NI_:                                                                                    \
        if (q2k_table)                                                                           \
            dispatch(decode_kernel<ENGRAM_FMT_Q2K, NI_>, grid, block, l, true, true, c, a, w);   \
        else                                                                                     \
            dispatch(decode_kernel<ENGRAM_FMT_E4M3, NI_>, grid, block, l, true, true, c, a, w);  \
        break;
    switch (ni) {
        ENGRAM_DECODE_CASE(1) ENGRAM_DECODE_CASE(2) ENGRAM_DECODE_CASE(3) ENGRAM_DECODE_CASE(4)
        ENGRAM_DECODE_CASE(5) ENGRAM_DECODE_CASE(6) ENGRAM_DECODE_CASE(7) ENGRAM_DECODE_CASE(8)
        ENGRAM_DECODE_CASE(9) ENGRAM_DECODE_CASE(10) ENGRAM_DECODE_CASE(11) ENGRAM_DECODE_CASE(12)
        ENGRAM_DECODE_CASE(13) ENGRAM_DECODE_CASE(14) ENGRAM_DECODE_CASE(15) ENGRAM_DECODE_CASE(16)
    default:
        return fail(ENGRAM_E_UNSUPPORTED, "engram decode: %lld columns exceed %lld",
                    (long long)c.cols, (long long)kDecodeMaxCols);
    }
#undef ENGRAM_DECODE_CASE
    return launch_status("engram decode kernel");
}

}  // namespace engram
