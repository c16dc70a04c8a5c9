// route.hip -- Route step: router logits in one fixed fp32 summation order,
// then per-token top-k with (logit desc, expert id asc) ordering and
// sigmoid-renormalised weights.
//
// The Colibri getting-started page ("トークンごとの処理経路", step Route) only
// says the router picks the experts each token activates.  The logit is
// defined here as 64 interleaved fmaf chains (chain l accumulates reduction
// indices l, l+64, l+128, ... in ascending order) folded by a fixed tree
// (s = 32, 16, ..., 1: p[i] = p[i] + p[i+s]) plus the bias.  A 64-lane wave
// realises exactly that order: lane l owns chain l, and the tree is six
// shuffle-down steps.  Because every float operation and its order is fixed,
// the logits, and therefore the selected experts, are reproducible bit for
// bit by any implementation of the same definition.
#include "dev_common.h"

#pragma clang fp contract(off)

namespace coli {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <bool BF16>
__device__ __forceinline__ float load_x(const void *x, size_t i) {
    if (BF16) return bf16_to_f32(static_cast<const uint16_t *>(x)[i]);
    return static_cast<const float *>(x)[i];
}

// One 64-thread block per tile of TB tokens x TE experts.  wt is the router
// weight transposed to [E x H] so lane l reads 64 consecutive floats.
// COHERENT: the logits are written past this XCD's caches, for a workgroup
// of the same launch to read (router_topk_kernel).
template <int TB, int TE, bool BF16, int UNROLL, bool COHERENT = false>
__device__ __forceinline__ void router_tile(
    const void *__restrict__ x, const float *__restrict__ wt,
    const float *__restrict__ bias, int n_tok, int hidden, int n_experts,
    float *__restrict__ logits, int tile) {
    const int tiles_e = (n_experts + TE - 1) / TE;
    const int te = tile % tiles_e;
    const int tt = tile / tiles_e;
    const int t0 = tt * TB, e0 = te * TE;
    const int lane = threadIdx.x & 63;

    const float *wrow[TE];
#pragma unroll
    for (int i = 0; i < TE; ++i) {
        int e = min(e0 + i, n_experts - 1);
        wrow[i] = wt + static_cast<size_t>(e) * hidden + lane;
    }
    size_t xoff[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b)
        xoff[b] = static_cast<size_t>(min(t0 + b, n_tok - 1)) * hidden + lane;

    float acc[TB][TE];
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int i = 0; i < TE; ++i) acc[b][i] = 0.0f;

    // Loads of a whole batch are issued before its FMAs; the chain order of
    // every accumulator stays k = lane, lane+64, ... ascending.
    const int steps = hidden / 64;
    int j0 = 0;
    for (; j0 + UNROLL <= steps; j0 += UNROLL) {
        float xv[UNROLL][TB], wv[UNROLL][TE];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int k = (j0 + u) * 64;
#pragma unroll
            for (int b = 0; b < TB; ++b) xv[u][b] = load_x<BF16>(x, xoff[b] + k);
#pragma unroll
            for (int i = 0; i < TE; ++i) wv[u][i] = wrow[i][k];
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int b = 0; b < TB; ++b)
#pragma unroll
                for (int i = 0; i < TE; ++i)
                    acc[b][i] = __builtin_fmaf(xv[u][b], wv[u][i], acc[b][i]);
    }
    for (; j0 < steps; ++j0) {
        const int k = j0 * 64;
        float xv[TB], wv[TE];
#pragma unroll
        for (int b = 0; b < TB; ++b) xv[b] = load_x<BF16>(x, xoff[b] + k);
#pragma unroll
        for (int i = 0; i < TE; ++i) wv[i] = wrow[i][k];
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int i = 0; i < TE; ++i) acc[b][i] = __builtin_fmaf(xv[b], wv[i], acc[b][i]);
    }
    // Fixed tree: after step s, lanes i < s hold p[i] + p[i+s].
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1)
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int i = 0; i < TE; ++i)
                acc[b][i] = acc[b][i] + __shfl_down(acc[b][i], s, 64);
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int i = 0; i < TE; ++i) {
                const int t = t0 + b, e = e0 + i;
                if (t < n_tok && e < n_experts) {
                    float *dst = logits + static_cast<size_t>(t) * n_experts + e;
                    const float v = acc[b][i] + (bias ? bias[e] : 0.0f);
                    if (COHERENT) dev::store_coherent(dst, v);
                    else *dst = v;
                }
            }
    }
}

template <int TB, int TE, bool BF16, int UNROLL>
__global__ __launch_bounds__(64) void router_logits_kernel(
    const void *__restrict__ x, const float *__restrict__ wt,
    const float *__restrict__ bias, int n_tok, int hidden, int n_experts,
    float *__restrict__ logits) {
    router_tile<TB, TE, BF16, UNROLL>(x, wt, bias, n_tok, hidden, n_experts, logits, blockIdx.x);
}

// Top-k by repeated selection, one wave per token: lane l holds the keys of
// experts l, l+64, ...; each of k rounds takes the largest remaining key
// (logit descending, then expert id ascending) by a wave max and removes it,
// so round r yields the expert of rank r.  A key is the order-preserving
// unsigned image of the logit (-0 and +0 equal) in the high word and the
// complemented id in the low word; 0 marks a removed or absent expert.  The
// weights are sigmoid(logit) divided by the sum of the k sigmoids, added in
// rank order.
__device__ __forceinline__ uint32_t logit_key(float f) {
    const uint32_t b = __float_as_uint(f + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One wave: the k selected experts and weights of token t from its row of
// logits.  COHERENT: the row was written by other workgroups of the same
// launch (read past the caches of this workgroup's XCD).
template <int EPL, bool COHERENT>
__device__ __forceinline__ void topk_token(const float *row, int n_experts, int k, size_t t,
                                           int32_t *__restrict__ idx, float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    uint64_t key[EPL];
    // Coherent reads as buffer loads with the sc1 policy (past this XCD's
    // caches), all in flight together, not one atomic load after another.
    const dev::rsrc_t rrow = dev::make_rsrc(row, static_cast<uint32_t>(n_experts) * 4);
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        float v = 0.0f;
        if (COHERENT) v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rrow, 4 * e, 0, 16));
        else if (e < n_experts) v = row[e];
        key[j] = e < n_experts
                     ? (static_cast<uint64_t>(logit_key(v)) << 32) | (0xffffffffu - static_cast<uint32_t>(e))
                     : 0ull;
    }
    int my_e = 0;
    float my_sig = 0.0f, sum = 0.0f;
    for (int r = 0; r < k; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const uint64_t other = __shfl_xor(best, o, 64);
            best = other > best ? other : best;
        }
        const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (lane + 64 * j == e) key[j] = 0ull;
        const float sg = 1.0f / (1.0f + expf(-key_logit(static_cast<uint32_t>(best >> 32))));
        sum = sum + sg;
        if (lane == r) {
            my_e = e;
            my_sig = sg;
        }
    }
    if (lane < k) {
        idx[t * k + lane] = my_e;
        w[t * k + lane] = my_sig / sum;
    }
}

template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits,
                                                   int n_tok, int n_experts, int k,
                                                   int32_t *__restrict__ idx,
                                                   float *__restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_tok) return;  // uniform per wave
    topk_token<EPL, false>(logits + static_cast<size_t>(t) * n_experts, n_experts, k, static_cast<size_t>(t),
                           idx, w);
}

// Batches the fused router and top-k launch serves: the 4 x 2 tile range of
// launch_router_logits (3 to 128 tokens).
constexpr int kRouteTopkMinTok = 3;
constexpr int kRouteTopkMaxTok = 128;
constexpr int kRouteTopkBlocks = kRouteTopkMaxTok / 4;   // token blocks, one arrival counter each
// Each counter on a 128-byte line of its own: the tile blocks' device-scope
// atomics on one line serialise (16 counters packed in one line made the
// launch 60 us at 64 tokens).
constexpr int kRouteTopkStride = 32;

// Router and top-k in one launch (batches of at most kRouteTopkMaxTok
// tokens): every tile's block hands its logits over (coherent stores) and
// arrives at its token block's counter; the last of the block's tiles_e
// tiles to arrive selects the experts of those TB tokens, one token after
// another, with topk_kernel's code -- the same logits, keys and sums, so the
// same bits as the two launches.
template <int TB, int TE, bool BF16, int UNROLL, int EPL>
__global__ __launch_bounds__(64 * TB) void router_topk_kernel(
    const void *__restrict__ x, const float *__restrict__ wt, const float *__restrict__ bias, int n_tok,
    int hidden, int n_experts, int k, float *__restrict__ logits, int32_t *__restrict__ counters,
    int32_t *__restrict__ idx, float *__restrict__ w) {
    // TB waves per workgroup, wave j on tile j of the workgroup's run of TB
    // consecutive expert tiles of one token block (tiles past the last are idle).
    const int tiles_e = (n_experts + TE - 1) / TE;
    const int groups_e = (tiles_e + TB - 1) / TB;
    const int tt = blockIdx.x / groups_e, ge = blockIdx.x % groups_e;
    const int wave = dev::wave_id();
    const int te = ge * TB + wave;
    if (te < tiles_e) router_tile<TB, TE, BF16, UNROLL, true>(x, wt, bias, n_tok, hidden, n_experts, logits, tt * tiles_e + te);
    if (!dev::arrive_last(counters + tt * kRouteTopkStride, groups_e)) return;
    // The last workgroup of the token block: wave j selects for token j.
    const int t = tt * TB + wave;
    if (t < n_tok)
        topk_token<EPL, true>(logits + static_cast<size_t>(t) * n_experts, n_experts, k, static_cast<size_t>(t), idx, w);
}

template <int TB, int TE, int UNROLL>
hipError_t launch_logits_t(const void *x, int act_bf16, const float *wt,
                           const float *bias, int n_tok, int hidden,
                           int n_experts, float *logits, hipStream_t s) {
    const int tiles = ((n_tok + TB - 1) / TB) * ((n_experts + TE - 1) / TE);
    if (act_bf16)
        launch(router_logits_kernel<TB, TE, true, UNROLL>, tiles, 64, 0, s,
            x, wt, bias, n_tok, hidden, n_experts, logits);
    else
        launch(router_logits_kernel<TB, TE, false, UNROLL>, tiles, 64, 0, s,
            x, wt, bias, n_tok, hidden, n_experts, logits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router_logits(const void *x, int act_bf16, const float *wt,
                                const float *bias, int n_tok, int hidden,
                                int n_experts, float *logits, hipStream_t s) {
    if (n_tok <= 0) return hipSuccess;
    if (n_tok <= 2)
        return launch_logits_t<1, 1, 32>(x, act_bf16, wt, bias, n_tok, hidden,
                                         n_experts, logits, s);
    // Up to 128 tokens, small tiles: more waves, each with a shorter load chain
    // (at 64 tokens 21 us instead of 38 us with the 8 x 8 tiles).
    if (n_tok <= 128)
        return launch_logits_t<4, 2, 8>(x, act_bf16, wt, bias, n_tok, hidden,
                                        n_experts, logits, s);
    return launch_logits_t<8, 8, 4>(x, act_bf16, wt, bias, n_tok, hidden,
                                    n_experts, logits, s);
}

template <int EPL>
void launch_router_topk_as(const void *x, int act_bf16, const float *wt, const float *bias, int n_tok, int hidden,
                           int n_experts, int k, float *logits, int32_t *counters, int32_t *idx, float *w,
                           hipStream_t s) {
    const int blocks = ((n_tok + 3) / 4) * ((((n_experts + 1) / 2) + 3) / 4);
    if (act_bf16)
        launch(router_topk_kernel<4, 2, true, 8, EPL>, blocks, 256, 0, s, x, wt, bias, n_tok, hidden, n_experts, k,
               logits, counters, idx, w);
    else
        launch(router_topk_kernel<4, 2, false, 8, EPL>, blocks, 256, 0, s, x, wt, bias, n_tok, hidden, n_experts, k,
               logits, counters, idx, w);
}

// hipErrorNotSupported (nothing launched) for batch sizes outside the fused
// range; `counters` holds route_topk_counters() ints, zero at rest.
int route_topk_counters() { return kRouteTopkBlocks * kRouteTopkStride; }

hipError_t launch_router_topk(const void *x, int act_bf16, const float *wt, const float *bias, int n_tok, int hidden,
                              int n_experts, int k, float *logits, int32_t *counters, int32_t *idx, float *w,
                              hipStream_t s) {
    if (n_tok < kRouteTopkMinTok || n_tok > kRouteTopkMaxTok) return hipErrorNotSupported;
    if (!counters) return hipErrorInvalidValue;
    if (n_experts <= 64) launch_router_topk_as<1>(x, act_bf16, wt, bias, n_tok, hidden, n_experts, k, logits, counters, idx, w, s);
    else if (n_experts <= 128) launch_router_topk_as<2>(x, act_bf16, wt, bias, n_tok, hidden, n_experts, k, logits, counters, idx, w, s);
    else if (n_experts <= 256) launch_router_topk_as<4>(x, act_bf16, wt, bias, n_tok, hidden, n_experts, k, logits, counters, idx, w, s);
    else if (n_experts <= 512) launch_router_topk_as<8>(x, act_bf16, wt, bias, n_tok, hidden, n_experts, k, logits, counters, idx, w, s);
    else launch_router_topk_as<16>(x, act_bf16, wt, bias, n_tok, hidden, n_experts, k, logits, counters, idx, w, s);
    return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int n_tok, int n_experts, int k,
                       int32_t *idx, float *w, hipStream_t s) {
    if (n_tok <= 0) return hipSuccess;
    const int blocks = (n_tok + 3) / 4;
    if (n_experts <= 64)
        launch(topk_kernel<1>, blocks, 256, 0, s, logits, n_tok, n_experts, k, idx, w);
    else if (n_experts <= 128)
        launch(topk_kernel<2>, blocks, 256, 0, s, logits, n_tok, n_experts, k, idx, w);
    else if (n_experts <= 256)
        launch(topk_kernel<4>, blocks, 256, 0, s, logits, n_tok, n_experts, k, idx, w);
    else if (n_experts <= 512)
        launch(topk_kernel<8>, blocks, 256, 0, s, logits, n_tok, n_experts, k, idx, w);
    else
        launch(topk_kernel<16>, blocks, 256, 0, s, logits, n_tok, n_experts, k, idx, w);
    return hipGetLastError();
}

}  // namespace coli
