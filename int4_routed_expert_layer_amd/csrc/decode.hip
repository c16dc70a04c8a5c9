// decode.hip -- front half of a small-batch layer call in one launch:
//   * router blocks: one wave per expert computes its logit for every token
//     in the fixed summation order (identical bits to the standalone router
//     kernel);
//   * shared-expert blocks: the always-on shared expert does not depend on
//     routing, so its gate/up panels stream from HBM while the router runs;
//   * the last router block to finish (arrival counter) selects the top-k of
//     every token and builds the union, so the routed gate/up kernel can
//     start right after this launch.
// Top-k, keys (logit desc, id asc), unique per expert: one token -- each
// wave ranks its 64 candidates, the k best of each wave are the only
// possible winners, and ranking those 4k finalists gives the slots; two to
// four tokens -- one wave per token takes k rounds of a wave-wide max.
// Union: an LDS histogram, one block scan, and an in-order rank for the
// gather (one token needs no scan at all).
#include "dev_gemv.h"

#pragma clang fp contract(off)

namespace coli {
namespace {

constexpr int kFrontThreads = 256;
constexpr int kFrontMaxExperts = 256;
constexpr int kFrontGateUpGroup = 4;   // shared gate/up chunks per register buffer
// Tokens per shared gate/up block: three or four tokens are split over two
// blocks per panel (two tokens each), which halves the per-block dot-product
// work on the front's critical path; each token's arithmetic is the same as
// in a four-token block.
template <int NT>
constexpr int front_shared_tokens() { return NT == 4 ? 2 : NT; }

template <int NT, bool BF16>
__device__ __forceinline__ void wave_router(const FwdArgs &a, const FrontArgs &f, int e) {
    const int lane = threadIdx.x & 63;
    const int H = a.hidden, E = a.n_experts;
    const float b = f.bias ? f.bias[e] : 0.0f;   // scalar load, in flight during the row
    const float *wrow = f.wt + static_cast<size_t>(e) * H + lane;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
    constexpr int U = NT == 1 ? 32 : 16;
    const int steps = H / 64;
    int j0 = 0;
    for (; j0 + U <= steps; j0 += U) {
        float wv[U], xv[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (j0 + u) * 64 + lane;
            wv[u] = wrow[(j0 + u) * 64];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const size_t idx = static_cast<size_t>(min(t, a.n_tok - 1)) * H + k;
                xv[u][t] = BF16 ? dev::bf16_bits_to_f32(static_cast<const uint16_t *>(a.x)[idx])
                                : static_cast<const float *>(a.x)[idx];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(xv[u][t], wv[u], acc[t]);
    }
    for (; j0 < steps; ++j0) {
        const int k = j0 * 64 + lane;
        const float wv = wrow[j0 * 64];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const size_t idx = static_cast<size_t>(min(t, a.n_tok - 1)) * H + k;
            const float xv = BF16 ? dev::bf16_bits_to_f32(static_cast<const uint16_t *>(a.x)[idx])
                                  : static_cast<const float *>(a.x)[idx];
            acc[t] = __builtin_fmaf(xv, wv, acc[t]);
        }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = acc[t] + __shfl_down(acc[t], s, 64);
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t < a.n_tok) dev::store_coherent(f.logits + static_cast<size_t>(t) * E + e, acc[t] + b);
    }
}

// Unit descriptors past the n_union routed units: the shared expert's (rows
// n_tok k .. n_tok k + n_tok - 1 of the hidden buffer), then units past the
// last one (m = -1) up to f.n_units.
// tsh is the shared expert's blob (loaded early, off the selection's path).
__device__ __forceinline__ void write_tail_units(const FwdArgs &a, const FrontArgs &f, int n_union,
                                                 const uint8_t *tsh, int tid) {
    if (!f.units) return;
    for (int u = n_union + tid; u < f.n_units; u += kFrontThreads) {
        const bool shared = u == n_union && a.has_shared;
        f.units[u] = shared ? UnitDesc{tsh, a.n_tok * a.k, a.n_tok, a.n_experts, 0, 0}
                            : UnitDesc{nullptr, 0, -1, 0, 0, 0};
    }
}

// One token: top-k by ranks within waves and among the finalists, weights in
// rank order; its union needs no scans, as the k selected experts are
// distinct: expert e has count 1 if selected, offset = number of selected
// experts below e, and its single entry is the slot that chose it.
__device__ void select_one_token(const FwdArgs &a, const FrontArgs &f) {
    __shared__ uint64_t s_key[kFrontMaxExperts];
    __shared__ uint64_t s_fin[4 * kMaxTopK];
    __shared__ float s_sig[kMaxTopK];
    __shared__ int s_sel[kMaxTopK];
    const int tid = threadIdx.x, wave = tid >> 6;
    const int E = a.n_experts, k = a.k;
    // Blob pointers for the unit descriptors, in flight with the logits.
    const uint8_t *tbl = f.units && tid < E ? a.table[tid] : nullptr;
    const uint8_t *tsh = f.units && a.has_shared ? a.table[E] : nullptr;
    const uint32_t low = 0xFFFFFFFFu - static_cast<uint32_t>(tid);
    uint64_t key = low;
    if (tid < E) key |= static_cast<uint64_t>(dev::float_key(dev::load_coherent(f.logits + tid))) << 32;
    s_key[tid] = key;
    __syncthreads();
    int r = 0;
    for (int j = 0; j < 64; ++j) r += s_key[64 * wave + j] > key ? 1 : 0;
    if (r < k) s_fin[wave * k + r] = key;
    __syncthreads();
    if (tid < 4 * k) {
        const uint64_t fk = s_fin[tid];
        int R = 0;
        for (int j = 0; j < 4 * k; ++j) R += s_fin[j] > fk ? 1 : 0;
        if (R < k) {
            const uint32_t kh = static_cast<uint32_t>(fk >> 32);
            const float l = __uint_as_float((kh & 0x80000000u) ? (kh & 0x7fffffffu) : ~kh);
            s_sel[R] = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(fk));
            s_sig[R] = 1.0f / (1.0f + expf(-l));
        }
    }
    __syncthreads();
    if (tid < k) {
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) sum = sum + s_sig[j];
        f.topk_idx[tid] = s_sel[tid];
        f.topk_w[tid] = s_sig[tid] / sum;
    }
    if (tid < E) {
        int below = 0, slot = -1;
        for (int j = 0; j < k; ++j) {
            const int id = s_sel[j];
            below += id < tid ? 1 : 0;
            slot = id == tid ? j : slot;
        }
        f.counts[tid] = slot >= 0 ? 1 : 0;
        f.offsets[tid] = below;
        if (slot >= 0) {
            f.union_ids[below] = tid;
            f.gather[below] = slot;
            if (f.units) f.units[below] = UnitDesc{tbl, below, 1, tid, 0, 0};
        }
    }
    if (tid == 0) {
        f.offsets[E] = k;
        *f.n_union = k;
    }
    write_tail_units(a, f, k, tsh, tid);
}

// Two to kFrontMaxTok tokens: wave t selects token t's experts (lane l holds
// the keys of experts l, l + 64, ...; k rounds of a wave-wide max, the same
// selection and weights as the standalone top-k), then the union with one
// block scan of counts and union flags packed together.
__device__ void select_few_tokens(const FwdArgs &a, const FrontArgs &f) {
    __shared__ int s_idx[kFrontMaxTok * kMaxTopK];
    __shared__ int s_cnt[kFrontMaxExperts];
    __shared__ int s_off[kFrontMaxExperts];
    __shared__ int s_tmp[kFrontThreads / 64 + 1];
    constexpr int kEpl = kFrontMaxExperts / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.n_experts, k = a.k, n_tok = a.n_tok;
    const uint8_t *tbl = f.units && tid < E ? a.table[tid] : nullptr;
    const uint8_t *tsh = f.units && a.has_shared ? a.table[E] : nullptr;
    if (wave < n_tok) {
        const int t = wave;
        uint64_t key[kEpl];
#pragma unroll
        for (int j = 0; j < kEpl; ++j) {
            const int e = lane + 64 * j;
            key[j] = e < E ? (static_cast<uint64_t>(dev::float_key(dev::load_coherent(f.logits + t * E + e))) << 32) |
                                 (0xFFFFFFFFu - static_cast<uint32_t>(e))
                           : 0ull;
        }
        int my_e = 0;
        float my_sig = 0.0f, sum = 0.0f;
        for (int r = 0; r < k; ++r) {
            uint64_t best = key[0];
#pragma unroll
            for (int j = 1; j < kEpl; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const uint64_t other = __shfl_xor(best, o, 64);
                best = other > best ? other : best;
            }
            const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
#pragma unroll
            for (int j = 0; j < kEpl; ++j)
                if (lane + 64 * j == e) key[j] = 0ull;
            const uint32_t kh = static_cast<uint32_t>(best >> 32);
            const float l = __uint_as_float((kh & 0x80000000u) ? (kh & 0x7fffffffu) : ~kh);
            const float sg = 1.0f / (1.0f + expf(-l));
            sum = sum + sg;
            if (lane == r) {
                my_e = e;
                my_sig = sg;
            }
        }
        if (lane < k) {
            s_idx[t * k + lane] = my_e;
            f.topk_idx[t * k + lane] = my_e;
            f.topk_w[t * k + lane] = my_sig / sum;
        }
    }
    s_cnt[tid] = 0;
    __syncthreads();
    const int n_ent = n_tok * k;
    if (tid < n_ent) atomicAdd(&s_cnt[s_idx[tid]], 1);
    __syncthreads();
    // counts (< 2^16) in the low half, union flags in the high half: one scan
    // gives both the offsets and the union positions.
    const int c = tid < E ? s_cnt[tid] : 0;
    int total = 0;
    const int excl = dev::block_exclusive_scan<kFrontThreads>(c | ((c > 0 ? 1 : 0) << 16), s_tmp, &total);
    if (tid < E) {
        f.counts[tid] = c;
        f.offsets[tid] = excl & 0xFFFF;
        s_off[tid] = excl & 0xFFFF;
        if (c > 0) {
            f.union_ids[excl >> 16] = tid;
            if (f.units) f.units[excl >> 16] = UnitDesc{tbl, excl & 0xFFFF, c, tid, 0, 0};
        }
    }
    if (tid == 0) {
        f.offsets[E] = total & 0xFFFF;
        *f.n_union = total >> 16;
    }
    write_tail_units(a, f, total >> 16, tsh, tid);
    __syncthreads();
    if (tid < n_ent) {
        const int e = s_idx[tid];
        int before = 0;
        for (int i = 0; i < tid; ++i) before += s_idx[i] == e ? 1 : 0;
        f.gather[s_off[e] + before] = tid;
    }
}

template <class F, int NT, bool BF16>
__global__ __launch_bounds__(kFrontThreads) void decode_front_kernel(FwdArgs a, FrontArgs f, int router_blocks) {
    extern __shared__ __align__(16) uint8_t lds[];
    if (static_cast<int>(blockIdx.x) >= router_blocks) {
        constexpr int ST = front_shared_tokens<NT>();
        const int P = a.inter / kPanel;
        const int b = blockIdx.x - router_blocks, p = b % P, m0 = ST * (b / P);
        const int m = min(ST, a.n_tok - m0);
        // One block per CU here: a deeper load pipeline than the routed kernel.
        if (m > 0)
            dev::gateup_panel<F, ST, kFrontGateUpGroup>(a, dev::PlainRows{a}, a.table[a.n_experts],
                                                         a.n_tok * a.k + m0, m, p, lds, dev::lds_address(lds));
        return;
    }
    if (blockIdx.x == 0 && f.next_counters)
        for (int i = threadIdx.x; i < f.n_next; i += kFrontThreads) dev::store_coherent(f.next_counters + i, 0);
    const int e = static_cast<int>(blockIdx.x) * 4 + dev::wave_id();   // uniform per wave
    if (e < a.n_experts) wave_router<NT, BF16>(a, f, e);
    if (dev::arrive_last(f.counter, router_blocks)) {
        if (a.n_tok == 1) select_one_token(a, f);
        else select_few_tokens(a, f);
    }
}

template <class F, int NT>
hipError_t launch_t(const FwdArgs &a, const FrontArgs &f, size_t lds, hipStream_t s) {
    const int router_blocks = (a.n_experts + 3) / 4;
    const int grid = router_blocks + (a.has_shared ? a.inter / kPanel * (NT / front_shared_tokens<NT>()) : 0);
    if (a.act_bf16)
        launch(decode_front_kernel<F, NT, true>, grid, kFrontThreads, lds, s, a, f, router_blocks);
    else
        launch(decode_front_kernel<F, NT, false>, grid, kFrontThreads, lds, s, a, f, router_blocks);
    return hipGetLastError();
}

template <class F>
hipError_t launch_nt(const FwdArgs &a, const FrontArgs &f, int nt, size_t lds, hipStream_t s) {
    if (nt == 1) return launch_t<F, 1>(a, f, lds, s);
    if (nt == 2) return launch_t<F, 2>(a, f, lds, s);
    return launch_t<F, 4>(a, f, lds, s);
}

}  // namespace

hipError_t launch_decode_front(const FwdArgs &a, const FrontArgs &f, size_t max_lds, hipStream_t s) {
    if (a.n_tok < 1 || a.n_tok > kFrontMaxTok || a.n_experts > kFrontMaxExperts) return hipErrorInvalidValue;
    const int nt = a.n_tok == 1 ? 1 : (a.n_tok == 2 ? 2 : 4);
    const size_t lds = a.has_shared ? dev::gateup_lds_bytes(nt == 4 ? front_shared_tokens<4>() : nt, a.hidden) : 0;
    if (lds > max_lds) return hipErrorInvalidValue;
    hipError_t e = hipSuccess;
    dev::dispatch_format(a.lay.group, a.lay.bits,
                         [&](auto fmt) { e = launch_nt<decltype(fmt)>(a, f, nt, lds, s); });
    return e;
}

}  // namespace coli
