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
#include "internal.h"

#pragma clang fp contract(off)

namespace coli {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// One 64-thread block per tile of TB tokens x TE experts.  wt is the router
// weight transposed to [E x H] so lane l reads 64 consecutive floats.
template <int TB, int TE, bool BF16, int UNROLL>
__global__ __launch_bounds__(64) void router_logits_kernel(
    const void *__restrict__ x, const float *__restrict__ wt,
    const float *__restrict__ bias, int n_tok, int hidden, int n_experts,
    float *__restrict__ logits) {
    const int tiles_e = (n_experts + TE - 1) / TE;
    const int te = blockIdx.x % tiles_e;
    const int tt = blockIdx.x / tiles_e;
    const int t0 = tt * TB, e0 = te * TE;
    const int lane = threadIdx.x;

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

    const int steps = hidden / 64;
    for (int j0 = 0; j0 < steps; j0 += UNROLL) {
        float xv[UNROLL][TB], wv[UNROLL][TE];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int k = (j0 + u) * 64;
            const bool ok = (j0 + u) < steps;
#pragma unroll
            for (int b = 0; b < TB; ++b) {
                if (BF16)
                    xv[u][b] = ok ? bf16_to_f32(static_cast<const uint16_t *>(x)[xoff[b] + k]) : 0.0f;
                else
                    xv[u][b] = ok ? static_cast<const float *>(x)[xoff[b] + k] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < TE; ++i) wv[u][i] = ok ? wrow[i][k] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if ((j0 + u) < steps) {
#pragma unroll
                for (int b = 0; b < TB; ++b)
#pragma unroll
                    for (int i = 0; i < TE; ++i)
                        acc[b][i] = __builtin_fmaf(xv[u][b], wv[u][i], acc[b][i]);
            }
        }
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
                if (t < n_tok && e < n_experts)
                    logits[static_cast<size_t>(t) * n_experts + e] =
                        acc[b][i] + (bias ? bias[e] : 0.0f);
            }
    }
}

__device__ __forceinline__ bool ranks_before(float la, int a, float lb, int b) {
    // b == INT_MAX marks "no candidate".
    if (b == 0x7fffffff) return a != 0x7fffffff;
    if (a == 0x7fffffff) return false;
    return la > lb || (la == lb && a < b);
}

// One wave per token.  Each lane holds up to 16 logits (experts lane + 64i).
__global__ __launch_bounds__(64) void topk_kernel(const float *__restrict__ logits,
                                                  int n_tok, int n_experts, int k,
                                                  int32_t *__restrict__ idx,
                                                  float *__restrict__ w) {
    const int t = blockIdx.x;
    const int lane = threadIdx.x;
    constexpr int kPer = kMaxExperts / 64;
    float v[kPer];
    uint32_t avail = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        v[i] = 0.0f;
        if (e < n_experts) {
            // + 0.0f maps -0 to +0; the compare below already treats them
            // as equal, this keeps the stored key canonical.
            v[i] = logits[static_cast<size_t>(t) * n_experts + e] + 0.0f;
            avail |= 1u << i;
        }
    }
    int my_idx = 0;
    float my_logit = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane + 64 * i;
            if (((avail >> i) & 1u) && ranks_before(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (ranks_before(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) avail &= ~(1u << (bi >> 6));
        if (lane == j) {
            my_idx = bi;
            my_logit = bv;
        }
    }
    const float sig = 1.0f / (1.0f + expf(-my_logit));
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum = sum + __shfl(sig, j, 64);
    if (lane < k) {
        idx[static_cast<size_t>(t) * k + lane] = my_idx;
        w[static_cast<size_t>(t) * k + lane] = sig / sum;
    }
}

template <int TB, int TE, int UNROLL>
hipError_t launch_logits_t(const void *x, int act_bf16, const float *wt,
                           const float *bias, int n_tok, int hidden,
                           int n_experts, float *logits, hipStream_t s) {
    const int tiles = ((n_tok + TB - 1) / TB) * ((n_experts + TE - 1) / TE);
    if (act_bf16)
        router_logits_kernel<TB, TE, true, UNROLL><<<tiles, 64, 0, s>>>(
            x, wt, bias, n_tok, hidden, n_experts, logits);
    else
        router_logits_kernel<TB, TE, false, UNROLL><<<tiles, 64, 0, s>>>(
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
    if (n_tok <= 32)
        return launch_logits_t<4, 2, 8>(x, act_bf16, wt, bias, n_tok, hidden,
                                        n_experts, logits, s);
    return launch_logits_t<8, 8, 2>(x, act_bf16, wt, bias, n_tok, hidden,
                                    n_experts, logits, s);
}

hipError_t launch_topk(const float *logits, int n_tok, int n_experts, int k,
                       int32_t *idx, float *w, hipStream_t s) {
    if (n_tok <= 0) return hipSuccess;
    topk_kernel<<<n_tok, 64, 0, s>>>(logits, n_tok, n_experts, k, idx, w);
    return hipGetLastError();
}

}  // namespace coli
