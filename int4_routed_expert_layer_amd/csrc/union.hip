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
// The batch's n = n_tok*k entries are cut into slabs of whole 256-entry
// chunks, one workgroup per slab, in two launches:
//  * rank: each workgroup gives every entry of its slab its stable rank among
//    the slab's entries of the same expert (chunk by chunk: wave ballots
//    matching the id bits give the rank inside a wave, per-wave counts in LDS
//    the waves before it, a per-expert running base the chunks before it) and
//    publishes its per-expert counts.  The last workgroup to finish sums the
//    counts over slabs in slab order, which gives counts, offsets, the union
//    and each slab's per-expert base.
//  * scatter: entry i of expert e in slab b goes to
//    gather[offsets[e] + base[b][e] + rank[i]].
// Up to 2048 entries the same ranking runs in a single workgroup and one
// launch does everything (union_small_kernel), together with the grouped
// work list and the fp16 copy of x when a layer call asks for them.
// Everything is integer and every sum has a fixed order or is order-free, so
// the results are exact and independent of scheduling.
#include "dev_common.h"

namespace coli {
namespace {

constexpr int kThreads = 1024;

constexpr int kUT = 256;                 // threads per union workgroup
constexpr int kUWaves = kUT / 64;

// Stable rank of every entry of [i0, i1) among the earlier entries of the
// range with the same expert, chunk by chunk: wave ballots matching the id
// bits give the rank inside a wave, per-wave counts in LDS the waves before
// it, and s_base[e] (zero on entry, the count of e in the range on exit) the
// chunks before it.  put(i, rank) receives each valid entry's rank.  Ids
// outside [0, E) are left out; returns true in a thread that saw one.  All
// kUT threads must call it.
template <class Put>
__device__ bool rank_entries(const int32_t *__restrict__ idx, int i0, int i1, int E, int *s_base,
                             unsigned short (*s_wc)[kMaxExperts], Put put) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    bool bad = false;
    int nxt = i0 + tid < i1 ? idx[i0 + tid] : -1;
    for (int c0 = i0; c0 < i1; c0 += kUT) {
        const int i = c0 + tid;
        int e = nxt;
        nxt = i + kUT < i1 ? idx[i + kUT] : -1;
        if (i < i1 && (e < 0 || e >= E)) bad = true;
        if (e >= E) e = -1;
        uint64_t peers = __ballot(e >= 0);
#pragma unroll
        for (int bit = 0; bit < 10; ++bit) {
            const bool on = (e >> bit) & 1;
            const uint64_t m = __ballot(on);
            peers &= on ? m : ~m;
        }
        const int r = __popcll(peers & lt_mask);
        const bool leader = e >= 0 && r == 0;
        const int cnt = __popcll(peers);
        if (leader) s_wc[wave][e] = static_cast<unsigned short>(cnt);
        __syncthreads();
        if (e >= 0) {
            int before = 0;
            for (int w = 0; w < wave; ++w) before += s_wc[w][e];
            put(i, s_base[e] + before + r);
        }
        __syncthreads();
        if (leader) {
            atomicAdd(&s_base[e], cnt);  // integer adds: order-free
            s_wc[wave][e] = 0;
        }
        __syncthreads();
    }
    return bad;
}

__global__ __launch_bounds__(kUT) void union_rank_kernel(
    const int32_t *__restrict__ idx, int n_ent, int slab, int n_experts,
    int32_t *__restrict__ rank_out, int32_t *__restrict__ blk, int32_t *__restrict__ counter,
    int32_t *__restrict__ n_union, int32_t *__restrict__ union_ids,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ err) {
    __shared__ int s_base[kMaxExperts];
    __shared__ unsigned short s_wc[kUWaves][kMaxExperts];
    __shared__ int s_tmp[kUWaves + 1];
    const int tid = threadIdx.x;
    const int E = n_experts, b = blockIdx.x, nb = gridDim.x;

    for (int e = tid; e < E; e += kUT) {
        s_base[e] = 0;
#pragma unroll
        for (int w = 0; w < kUWaves; ++w) s_wc[w][e] = 0;
    }
    __syncthreads();

    const int i0 = b * slab, i1 = min(n_ent, i0 + slab);
    const bool bad = rank_entries(idx, i0, i1, E, s_base, s_wc, [&](int i, int r) { rank_out[i] = r; });
    if (bad) atomicOr(err, 1);
    for (int e = tid; e < E; e += kUT) dev::store_coherent(&blk[b * E + e], s_base[e]);
    if (!dev::arrive_last(counter, nb)) return;

    // Last workgroup: per-expert sums over slabs in slab order (blk becomes
    // each slab's exclusive base), then offsets and the union over experts.
    int carry_off = 0, carry_u = 0;
    for (int e0 = 0; e0 < E; e0 += kUT) {
        const int e = e0 + tid;
        int c = 0;
        if (e < E) {
            for (int q0 = 0; q0 < nb; q0 += 16) {
                int v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    v[j] = q0 + j < nb ? dev::load_coherent(&blk[(q0 + j) * E + e]) : 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (q0 + j < nb) blk[(q0 + j) * E + e] = c;
                    c += v[j];
                }
            }
        }
        int tot = 0;
        const int ex = dev::block_exclusive_scan<kUT>(c, s_tmp, &tot);
        if (e < E) {
            counts[e] = c;
            offsets[e] = carry_off + ex;
        }
        carry_off += tot;
        const int f = (e < E && c > 0) ? 1 : 0;
        int nu = 0;
        const int pos = dev::block_exclusive_scan<kUT>(f, s_tmp, &nu);
        if (f) union_ids[carry_u + pos] = e;
        carry_u += nu;
    }
    if (tid == 0) {
        offsets[E] = carry_off;
        *n_union = carry_u;
    }
}

__global__ __launch_bounds__(kUT) void union_scatter_kernel(
    const int32_t *__restrict__ idx, int n_ent, int slab, int n_experts,
    const int32_t *__restrict__ rank, const int32_t *__restrict__ blk,
    const int32_t *__restrict__ offsets, int32_t *__restrict__ gather) {
    const int i = blockIdx.x * kUT + threadIdx.x;
    if (i >= n_ent) return;
    const int e = idx[i];
    if (e < 0 || e >= n_experts) return;
    gather[offsets[e] + blk[(i / slab) * n_experts + e] + rank[i]] = i;
}

// Work chunks for the grouped GEMMs: each union expert (and the shared
// expert, placed after them) is cut into runs of at most a.chunk_rows rows.
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
    const int cr = a.chunk_rows;
    const int nch = (m + cr - 1) / cr;
    int total = 0;
    const int first = dev::block_exclusive_scan<kThreads>(nch, s_tmp, &total);
    for (int c = 0; c < nch; ++c) {
        ChunkDesc d;
        d.expert = e;
        d.row0 = row0 + c * cr;
        d.rows = min(cr, m - c * cr);
        d.pad = 0;
        chunks[first + c] = d;
    }
    if (tid == 0) *n_chunks = total;
}

// Calls of at most kUnionSmallEntries entries: the whole union in one
// workgroup (block 0).  The ranks stay in LDS, counts, offsets and the union
// come from the same workgroup without a hand-off between workgroups, and
// the scatter follows; with a work list requested (`chunks` non-NULL: the
// grouped strategy of a layer call) the same workgroup then cuts it as
// plan_kernel does, and the launch's other workgroups make the fp16 copy of
// x (n8 groups of 8).  One launch instead of four; the outputs are those of
// the two-launch union, bit for bit (the same stable counting sort).
__global__ __launch_bounds__(kUT) void union_small_kernel(
    const int32_t *__restrict__ idx, int n_ent, int n_experts, int32_t *__restrict__ n_union,
    int32_t *__restrict__ union_ids, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ gather, FwdArgs a, ChunkDesc *__restrict__ chunks, int32_t *__restrict__ n_chunks,
    size_t n8) {
    if (blockIdx.x > 0) {
        dev::to_half8(a.x, a.act_bf16, static_cast<size_t>(blockIdx.x - 1) * kUT + threadIdx.x, n8, a.xh, a.err);
        return;
    }
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_uid[kMaxExperts];
    __shared__ unsigned short s_wc[kUWaves][kMaxExperts];
    __shared__ int s_rank[kUnionSmallEntries];
    __shared__ int s_tmp[kUWaves + 1];
    const int tid = threadIdx.x;
    const int E = n_experts;
    for (int e = tid; e < E; e += kUT) {
        s_cnt[e] = 0;
#pragma unroll
        for (int w = 0; w < kUWaves; ++w) s_wc[w][e] = 0;
    }
    __syncthreads();
    const bool bad = rank_entries(idx, 0, n_ent, E, s_cnt, s_wc, [&](int i, int r) { s_rank[i] = r; });
    if (bad) atomicOr(a.err, kErrExpertId);

    // Counts, offsets and the union, over experts in ascending order.
    int carry_off = 0, carry_u = 0;
    for (int e0 = 0; e0 < E; e0 += kUT) {
        const int e = e0 + tid;
        const int c = e < E ? s_cnt[e] : 0;
        int tot = 0;
        const int ex = dev::block_exclusive_scan<kUT>(c, s_tmp, &tot);
        if (e < E) {
            counts[e] = c;
            offsets[e] = carry_off + ex;
            s_off[e] = carry_off + ex;
        }
        carry_off += tot;
        const int f = c > 0 ? 1 : 0;
        int nu = 0;
        const int pos = dev::block_exclusive_scan<kUT>(f, s_tmp, &nu);
        if (f) {
            union_ids[carry_u + pos] = e;
            s_uid[carry_u + pos] = e;
        }
        carry_u += nu;
    }
    if (tid == 0) {
        offsets[E] = carry_off;
        *n_union = carry_u;
    }
    __syncthreads();
    for (int i = tid; i < n_ent; i += kUT) {
        const int e = idx[i];
        if (e >= 0 && e < E) gather[s_off[e] + s_rank[i]] = i;
    }
    if (!chunks) return;

    // The grouped work list: union experts, then the shared one, cut into
    // runs of at most a.chunk_rows rows.
    const int units = carry_u + (a.has_shared ? 1 : 0);
    const int cr = a.chunk_rows;
    int carry_c = 0;
    for (int u0 = 0; u0 < units; u0 += kUT) {
        const int u = u0 + tid;
        int e = 0, m = 0, row0 = 0;
        if (u < carry_u) {
            e = s_uid[u];
            m = s_cnt[e];
            row0 = s_off[e];
        } else if (u == carry_u && a.has_shared) {
            e = E;
            m = a.n_tok;
            row0 = a.n_tok * a.k;
        }
        const int nch = (m + cr - 1) / cr;
        int tot = 0;
        const int first = carry_c + dev::block_exclusive_scan<kUT>(nch, s_tmp, &tot);
        for (int c = 0; c < nch; ++c) {
            ChunkDesc d;
            d.expert = e;
            d.row0 = row0 + c * cr;
            d.rows = min(cr, m - c * cr);
            d.pad = 0;
            chunks[first + c] = d;
        }
        carry_c += tot;
    }
    if (tid == 0) *n_chunks = carry_c;
}

}  // namespace

UnionSplit union_split(int n_tok, int k) {
    const int n = n_tok * k;
    const int per = (n + kUnionMaxBlocks - 1) / kUnionMaxBlocks;
    UnionSplit u;
    u.slab = ((per + kUT - 1) / kUT) * kUT;
    if (u.slab < kUT) u.slab = kUT;
    u.nb = n > 0 ? (n + u.slab - 1) / u.slab : 1;
    return u;
}

hipError_t launch_union_rank(const int32_t *idx, int n_tok, int k, int n_experts, UnionScratch ws,
                             int32_t *n_union, int32_t *union_ids, int32_t *counts, int32_t *offsets,
                             int32_t *err, hipStream_t s) {
    const UnionSplit u = union_split(n_tok, k);
    launch(union_rank_kernel, u.nb, kUT, 0, s, idx, n_tok * k, u.slab, n_experts, ws.rank, ws.blk,
           ws.counter, n_union, union_ids, counts, offsets, err);
    return hipGetLastError();
}

hipError_t launch_union_scatter(const int32_t *idx, int n_tok, int k, int n_experts, UnionScratch ws,
                                const int32_t *offsets, int32_t *gather, hipStream_t s) {
    const int n = n_tok * k;
    if (n == 0) return hipSuccess;
    const UnionSplit u = union_split(n_tok, k);
    launch(union_scatter_kernel, (n + kUT - 1) / kUT, kUT, 0, s, idx, n, u.slab, n_experts, ws.rank,
           ws.blk, offsets, gather);
    return hipGetLastError();
}

hipError_t launch_plan(const FwdArgs &a, ChunkDesc *chunks, int32_t *n_chunks,
                       hipStream_t s) {
    launch(plan_kernel, 1, kThreads, 0, s, a, chunks, n_chunks);
    return hipGetLastError();
}

hipError_t launch_union_small(const int32_t *idx, int n_tok, int k, int n_experts, int32_t *n_union,
                              int32_t *union_ids, int32_t *counts, int32_t *offsets, int32_t *gather,
                              const FwdArgs &a, ChunkDesc *chunks, int32_t *n_chunks, hipStream_t s) {
    const int n = n_tok * k;
    if (n > kUnionSmallEntries) return hipErrorInvalidValue;
    const size_t n8 = chunks ? static_cast<size_t>(a.n_tok) * a.hidden / 8 : 0;
    const unsigned grid = 1 + static_cast<unsigned>((n8 + kUT - 1) / kUT);
    launch(union_small_kernel, grid, kUT, 0, s, idx, n, n_experts, n_union, union_ids, counts, offsets, gather, a,
           chunks, n_chunks, n8);
    return hipGetLastError();
}

int max_work_chunks(int n_tok, int k, int n_experts, int has_shared, int chunk_rows) {
    const int rows = n_tok * k + (has_shared ? n_tok : 0);
    const int experts = (n_tok * k < n_experts ? n_tok * k : n_experts) + (has_shared ? 1 : 0);
    return rows / chunk_rows + experts + 1;
}

int work_list_capacity(int max_tokens, int k, int n_experts, int has_shared) {
    const int small = max_tokens < kSmallChunkMaxTok ? max_tokens : kSmallChunkMaxTok;
    return std::max(max_work_chunks(max_tokens, k, n_experts, has_shared, chunk_rows_for(max_tokens)),
                    max_work_chunks(small, k, n_experts, has_shared, kSmallChunkRows));
}

}  // namespace coli
