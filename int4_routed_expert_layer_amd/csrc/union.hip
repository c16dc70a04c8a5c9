// union.hip -- Union step: batch-union deduplication of the selected
// experts, and the work list of the grouped expert GEMMs.
//
// The README ("Mai aspettare il disco due volte") and the getting-started
// page (step Union) describe batch positions reading each unique expert only
// once.  The canonical output here: union_ids ascending, counts[E], offsets =
// exclusive prefix sum of counts, and gather = the entries t*k+j ordered by
// (expert, token) -- a stable counting sort -- so each expert's tokens form
// one contiguous run of rows for the expert FFNs.
//
// One block (256 threads for up to 256 experts, else 1024) does the whole
// batch: an LDS histogram (integer atomics, order-free), two block scans
// (offsets, compaction of the union), then the gather in chunks of one entry
// per thread, where each entry's rank among
// equal experts comes from wave ballots (match-any over the id bits) plus
// per-wave counts in LDS.  Everything is integer, so results are exact and
// independent of scheduling.
#include "dev_common.h"

namespace coli {
namespace {

constexpr int kThreads = 1024;

// NT threads handle up to NT experts.
template <int NT>
__global__ __launch_bounds__(NT) void union_kernel(
    const int32_t *__restrict__ idx, int n_ent, int n_experts,
    int32_t *__restrict__ n_union, int32_t *__restrict__ union_ids,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ gather, int32_t *__restrict__ err) {
    constexpr int kThreads = NT;
    constexpr int kWaves = NT / 64;
    __shared__ int s_cnt[NT];
    __shared__ int s_off[NT];
    __shared__ int s_base[NT];
    __shared__ unsigned short s_wc[kWaves][NT];
    __shared__ int s_tmp[kWaves + 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    s_cnt[tid] = 0;
    s_base[tid] = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s_wc[w][tid] = 0;
    __syncthreads();

    bool bad = false;
    for (int i = tid; i < n_ent; i += kThreads) {
        const int e = idx[i];
        if (e >= 0 && e < n_experts)
            atomicAdd(&s_cnt[e], 1);
        else
            bad = true;
    }
    if (bad) atomicOr(err, 1);
    __syncthreads();

    const int c = tid < n_experts ? s_cnt[tid] : 0;
    int total = 0;
    const int excl = dev::block_exclusive_scan<NT>(c, s_tmp, &total);
    if (tid < n_experts) {
        counts[tid] = c;
        offsets[tid] = excl;
        s_off[tid] = excl;
    }
    if (tid == 0) offsets[n_experts] = total;
    const int flag = (tid < n_experts && c > 0) ? 1 : 0;
    int nu = 0;
    const int pos = dev::block_exclusive_scan<NT>(flag, s_tmp, &nu);
    if (flag) union_ids[pos] = tid;
    if (tid == 0) *n_union = nu;
    __syncthreads();

    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < n_ent; c0 += kThreads) {
        const int i = c0 + tid;
        int e = i < n_ent ? idx[i] : -1;
        if (e >= n_experts) e = -1;
        uint64_t peers = __ballot(e >= 0);
#pragma unroll
        for (int b = 0; b < 10; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & lt_mask);
        if (e >= 0 && rank == 0) s_wc[wave][e] = static_cast<unsigned short>(__popcll(peers));
        __syncthreads();
        if (e >= 0) {
            int before = 0;
            for (int w = 0; w < wave; ++w) before += s_wc[w][e];
            gather[s_off[e] + s_base[e] + before + rank] = i;
        }
        __syncthreads();
        if (tid < n_experts) {
            int tot = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                tot += s_wc[w][tid];
                s_wc[w][tid] = 0;
            }
            s_base[tid] += tot;
        }
        __syncthreads();
    }
}

// Work chunks for the grouped GEMMs: each union expert (and the shared
// expert, placed after them) is cut into runs of at most kChunkRows rows.
__global__ __launch_bounds__(kThreads) void plan_kernel(FwdArgs a,
                                                        ChunkDesc *__restrict__ chunks,
                                                        int32_t *__restrict__ n_chunks) {
    __shared__ int s_tmp[kThreads / 64 + 1];
    const int tid = threadIdx.x;
    const int nu = *a.n_union;
    int e = 0, m = 0, row0 = 0;
    if (tid < nu) {
        e = a.union_ids[tid];
        m = a.counts[e];
        row0 = a.offsets[e];
    } else if (tid == nu && a.has_shared) {
        e = a.n_experts;
        m = a.n_tok;
        row0 = a.n_tok * a.k;
    }
    const int nch = (m + kChunkRows - 1) / kChunkRows;
    int total = 0;
    const int first = dev::block_exclusive_scan<kThreads>(nch, s_tmp, &total);
    for (int c = 0; c < nch; ++c) {
        ChunkDesc d;
        d.expert = e;
        d.row0 = row0 + c * kChunkRows;
        d.rows = min(kChunkRows, m - c * kChunkRows);
        d.pad = 0;
        chunks[first + c] = d;
    }
    if (tid == 0) *n_chunks = total;
}

}  // namespace

hipError_t launch_union(const int32_t *idx, int n_tok, int k, int n_experts,
                        int32_t *n_union, int32_t *union_ids, int32_t *counts,
                        int32_t *offsets, int32_t *gather, int32_t *err,
                        hipStream_t s) {
    if (n_experts <= 256)
        launch(union_kernel<256>, 1, 256, 0, s, idx, n_tok * k, n_experts, n_union, union_ids,
                                            counts, offsets, gather, err);
    else
        launch(union_kernel<1024>, 1, 1024, 0, s, idx, n_tok * k, n_experts, n_union, union_ids,
                                              counts, offsets, gather, err);
    return hipGetLastError();
}

hipError_t launch_plan(const FwdArgs &a, ChunkDesc *chunks, int32_t *n_chunks,
                       hipStream_t s) {
    launch(plan_kernel, 1, kThreads, 0, s, a, chunks, n_chunks);
    return hipGetLastError();
}

int max_work_chunks(int n_tok, int k, int n_experts, int has_shared) {
    const int rows = n_tok * k + (has_shared ? n_tok : 0);
    const int experts = (n_tok * k < n_experts ? n_tok * k : n_experts) + (has_shared ? 1 : 0);
    return rows / kChunkRows + experts + 1;
}

}  // namespace coli
