// gemv.hip -- decode-shaped expert FFNs on the vector ALUs.
//
// When each union expert serves one or two tokens the expert matmuls are
// matrix-vector products bound by HBM bandwidth: every weight byte is used
// once or twice, so the work is kept on the VALU and shaped for streaming.
// One 256-thread workgroup owns one 16-row panel of one expert; its four
// waves split the reduction axis (chunk c goes to wave c mod 4), each lane
// issues one 16-byte load per 1 KB chunk (fully coalesced), and the int4
// values are expanded with two integer ops per pair and fed to v_dot2:
//   gate/up: bf16 pairs (128 + u) against bf16 activations, then the
//            per-32-group correction s * (d - 136 * sum(x)) = s * sum(q x);
//   down:    exact fp16 q = (1024 + u) - 1032 against the fp16 hidden
//            activation, then the group scale.
// Partial sums are reduced across the four lanes that share a row and then
// across the four waves in a fixed order, so results are deterministic.
//
// The expert FFN is SwiGLU, y = Wd (silu(Wg x) * (Wu x)); the routed output
// row for entry t*k+j is written pre-multiplied by its routing weight, the
// shared expert's row with weight 1, and the combine kernel sums them.
#include "internal.h"

namespace coli {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_f32(uint32_t h16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h16)));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// Pair j of a packed dword: columns 2j and 2j+1 as u = q + 8 in the low and
// high 16-bit halves, OR-ed with an exponent pattern.
__device__ __forceinline__ uint32_t pair(uint32_t w, int j, uint32_t magic) {
    return ((w >> (4 * j)) & 0x000F000Fu) | magic;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float dot2_f16(half2v a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(half2v, b), c, false);
}

// Resolve work unit u: routed union entry (u < n_union) or the shared expert
// (u == n_union).  Returns false for no work.
__device__ __forceinline__ bool resolve(const FwdArgs &a, int u, int &e, int &r0, int &m) {
    const int nu = *a.n_union;
    if (u < nu) {
        e = a.union_ids[u];
        r0 = a.offsets[e];
        m = a.counts[e];
        return true;
    }
    if (u == nu && a.has_shared) {
        e = a.n_experts;
        r0 = a.n_tok * a.k;
        m = a.n_tok;
        return true;
    }
    return false;
}

__device__ __forceinline__ int token_of_row(const FwdArgs &a, int row) {
    const int routed = a.n_tok * a.k;
    return row < routed ? a.gather[row] / a.k : row - routed;
}

template <int MAXM, bool F32X>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(FwdArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int H = a.hidden, I = a.inter;
    const int P = I / kPanel;
    const int u = blockIdx.x / P, p = blockIdx.x % P;
    int e, r0, M;
    if (!resolve(a, u, e, r0, M)) return;
    const uint8_t *blob = a.table[e];
    if (!blob || M <= 0) return;

    const int C = H / kChunkK;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = lane & 15, kq = lane >> 4;
    const uint8_t *gq = blob + a.lay.gate_q + static_cast<size_t>(p) * C * kChunkBytes + lane * 16;
    const uint8_t *uq = blob + a.lay.up_q + static_cast<size_t>(p) * C * kChunkBytes + lane * 16;
    const uint8_t *gs = blob + a.lay.gate_s + static_cast<size_t>(p) * C * kScaleChunkBytes + row * 8;
    const uint8_t *us = blob + a.lay.up_s + static_cast<size_t>(p) * C * kScaleChunkBytes + row * 8;

    // LDS: x [MAXM][H] (bf16 or f32), group sums [MAXM][H/8] (bf16 only),
    // cross-wave partials [4][MAXM][16][2].
    const size_t xbytes = static_cast<size_t>(MAXM) * H * (F32X ? 4 : 2);
    float *s8 = reinterpret_cast<float *>(lds + xbytes);
    float *red = s8 + (F32X ? 0 : MAXM * (H / 8));

    for (int mb = 0; mb < M; mb += MAXM) {
        const int mc = min(MAXM, M - mb);
        __syncthreads();
        for (int i = tid; i < mc * (H / 8); i += 256) {
            const int m = i / (H / 8), q = i % (H / 8);
            const int t = token_of_row(a, r0 + mb + m);
            if (F32X) {
                const float4 *src = reinterpret_cast<const float4 *>(
                    static_cast<const float *>(a.x) + static_cast<size_t>(t) * H + 8 * q);
                float4 *dst = reinterpret_cast<float4 *>(lds) + (static_cast<size_t>(m) * H + 8 * q) / 4;
                dst[0] = src[0];
                dst[1] = src[1];
            } else {
                const uint4 v = *reinterpret_cast<const uint4 *>(
                    static_cast<const uint16_t *>(a.x) + static_cast<size_t>(t) * H + 8 * q);
                *reinterpret_cast<uint4 *>(lds + (static_cast<size_t>(m) * H + 8 * q) * 2) = v;
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    s = s + bf16_bits_to_f32(w4[j] & 0xFFFFu);
                    s = s + bf16_bits_to_f32(w4[j] >> 16);
                }
                s8[m * (H / 8) + q] = s;
            }
        }
        __syncthreads();

        float gacc[MAXM], vacc[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) gacc[m] = vacc[m] = 0.0f;

        for (int c = wave; c < C; c += 4) {
            const uint4 gw = *reinterpret_cast<const uint4 *>(gq + static_cast<size_t>(c) * kChunkBytes);
            const uint4 uw = *reinterpret_cast<const uint4 *>(uq + static_cast<size_t>(c) * kChunkBytes);
            const uint2 gsc = *reinterpret_cast<const uint2 *>(gs + static_cast<size_t>(c) * kScaleChunkBytes);
            const uint2 usc = *reinterpret_cast<const uint2 *>(us + static_cast<size_t>(c) * kScaleChunkBytes);
            const uint32_t gws[4] = {gw.x, gw.y, gw.z, gw.w};
            const uint32_t uws[4] = {uw.x, uw.y, uw.z, uw.w};
            const uint32_t gss[2] = {gsc.x, gsc.y};
            const uint32_t uss[2] = {usc.x, usc.y};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float sg = half_bits_to_f32((gss[s >> 1] >> (16 * (s & 1))) & 0xFFFFu);
                const float su = half_bits_to_f32((uss[s >> 1] >> (16 * (s & 1))) & 0xFFFFu);
                const int k0 = c * kChunkK + 32 * s + 8 * kq;
                if (F32X) {
#pragma unroll
                    for (int m = 0; m < MAXM; ++m) {
                        if (m < mc) {
                            const float *xr = reinterpret_cast<const float *>(lds) + static_cast<size_t>(m) * H + k0;
                            float dg = 0.0f, du = 0.0f;
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                const int slot = (i & 1) ? 4 + (i >> 1) : (i >> 1);
                                const float qg = static_cast<float>((gws[s] >> (4 * slot)) & 15u) - 8.0f;
                                const float qu = static_cast<float>((uws[s] >> (4 * slot)) & 15u) - 8.0f;
                                dg = __builtin_fmaf(qg, xr[i], dg);
                                du = __builtin_fmaf(qu, xr[i], du);
                            }
                            gacc[m] = __builtin_fmaf(sg, dg, gacc[m]);
                            vacc[m] = __builtin_fmaf(su, du, vacc[m]);
                        }
                    }
                } else {
                    uint32_t pg[4], pu[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pg[j] = pair(gws[s], j, 0x43004300u);
                        pu[j] = pair(uws[s], j, 0x43004300u);
                    }
#pragma unroll
                    for (int m = 0; m < MAXM; ++m) {
                        if (m < mc) {
                            const uint4 xv = *reinterpret_cast<const uint4 *>(
                                lds + (static_cast<size_t>(m) * H + k0) * 2);
                            const float sx = s8[m * (H / 8) + (k0 >> 3)];
                            float dg = dot2_bf16(pg[0], xv.x, 0.0f);
                            dg = dot2_bf16(pg[1], xv.y, dg);
                            dg = dot2_bf16(pg[2], xv.z, dg);
                            dg = dot2_bf16(pg[3], xv.w, dg);
                            float du = dot2_bf16(pu[0], xv.x, 0.0f);
                            du = dot2_bf16(pu[1], xv.y, du);
                            du = dot2_bf16(pu[2], xv.z, du);
                            du = dot2_bf16(pu[3], xv.w, du);
                            gacc[m] = __builtin_fmaf(sg, __builtin_fmaf(-136.0f, sx, dg), gacc[m]);
                            vacc[m] = __builtin_fmaf(su, __builtin_fmaf(-136.0f, sx, du), vacc[m]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            gacc[m] = gacc[m] + __shfl_xor(gacc[m], 16, 64);
            gacc[m] = gacc[m] + __shfl_xor(gacc[m], 32, 64);
            vacc[m] = vacc[m] + __shfl_xor(vacc[m], 16, 64);
            vacc[m] = vacc[m] + __shfl_xor(vacc[m], 32, 64);
        }
        if (lane < 16) {
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                red[((wave * MAXM + m) * 16 + row) * 2 + 0] = gacc[m];
                red[((wave * MAXM + m) * 16 + row) * 2 + 1] = vacc[m];
            }
        }
        __syncthreads();
        if (tid < mc * 16) {
            const int m = tid >> 4, r = tid & 15;
            float g = 0.0f, v = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                g = g + red[((w * MAXM + m) * 16 + r) * 2 + 0];
                v = v + red[((w * MAXM + m) * 16 + r) * 2 + 1];
            }
            const float hval = g / (1.0f + expf(-g)) * v;
            a.h[static_cast<size_t>(r0 + mb + m) * I + p * kPanel + r] = static_cast<_Float16>(hval);
        }
    }
}

template <int MAXM>
__global__ __launch_bounds__(256) void gemv_down_kernel(FwdArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int H = a.hidden, I = a.inter;
    const int P = H / kPanel;
    const int u = blockIdx.x / P, p = blockIdx.x % P;
    int e, r0, M;
    if (!resolve(a, u, e, r0, M)) return;
    const uint8_t *blob = a.table[e];
    if (!blob || M <= 0) return;

    const int C = I / kChunkK;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = lane & 15, kq = lane >> 4;
    const uint8_t *dq = blob + a.lay.down_q + static_cast<size_t>(p) * C * kChunkBytes + lane * 16;
    const uint8_t *ds = blob + a.lay.down_s + static_cast<size_t>(p) * C * kScaleChunkBytes + row * 8;
    float *red = reinterpret_cast<float *>(lds + static_cast<size_t>(MAXM) * I * 2);
    const int routed = a.n_tok * a.k;
    const half2v k1032 = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};

    for (int mb = 0; mb < M; mb += MAXM) {
        const int mc = min(MAXM, M - mb);
        __syncthreads();
        for (int i = tid; i < mc * (I / 8); i += 256) {
            const int m = i / (I / 8), q = i % (I / 8);
            *reinterpret_cast<uint4 *>(lds + (static_cast<size_t>(m) * I + 8 * q) * 2) =
                *reinterpret_cast<const uint4 *>(a.h + static_cast<size_t>(r0 + mb + m) * I + 8 * q);
        }
        __syncthreads();
        float acc[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;
        for (int c = wave; c < C; c += 4) {
            const uint4 w = *reinterpret_cast<const uint4 *>(dq + static_cast<size_t>(c) * kChunkBytes);
            const uint2 sc = *reinterpret_cast<const uint2 *>(ds + static_cast<size_t>(c) * kScaleChunkBytes);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
            const uint32_t ss[2] = {sc.x, sc.y};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float sf = half_bits_to_f32((ss[s >> 1] >> (16 * (s & 1))) & 0xFFFFu);
                half2v q[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    q[j] = __builtin_bit_cast(half2v, pair(ws[s], j, 0x64006400u)) - k1032;
                const int k0 = c * kChunkK + 32 * s + 8 * kq;
#pragma unroll
                for (int m = 0; m < MAXM; ++m) {
                    if (m < mc) {
                        const uint4 hv = *reinterpret_cast<const uint4 *>(lds + (static_cast<size_t>(m) * I + k0) * 2);
                        float d = dot2_f16(q[0], hv.x, 0.0f);
                        d = dot2_f16(q[1], hv.y, d);
                        d = dot2_f16(q[2], hv.z, d);
                        d = dot2_f16(q[3], hv.w, d);
                        acc[m] = __builtin_fmaf(sf, d, acc[m]);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            acc[m] = acc[m] + __shfl_xor(acc[m], 16, 64);
            acc[m] = acc[m] + __shfl_xor(acc[m], 32, 64);
        }
        if (lane < 16) {
#pragma unroll
            for (int m = 0; m < MAXM; ++m) red[(wave * MAXM + m) * 16 + row] = acc[m];
        }
        __syncthreads();
        if (tid < mc * 16) {
            const int m = tid >> 4, r = tid & 15;
            float d = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) d = d + red[(w * MAXM + m) * 16 + r];
            const int hrow = r0 + mb + m;
            const int entry = hrow < routed ? a.gather[hrow] : hrow;
            const float wgt = hrow < routed ? a.topk_w[entry] : 1.0f;
            a.ys[static_cast<size_t>(entry) * H + p * kPanel + r] = wgt * d;
        }
    }
}

size_t gateup_lds(int maxm, int hidden, bool f32x) {
    return static_cast<size_t>(maxm) * hidden * (f32x ? 4 : 2) +
           (f32x ? 0 : static_cast<size_t>(maxm) * (hidden / 8) * 4) +
           static_cast<size_t>(4) * maxm * 16 * 2 * 4;
}

size_t down_lds(int maxm, int inter) {
    return static_cast<size_t>(maxm) * inter * 2 + static_cast<size_t>(4) * maxm * 16 * 4;
}

int units(const FwdArgs &a) {
    const int routed = a.n_tok * a.k < a.n_experts ? a.n_tok * a.k : a.n_experts;
    return routed + (a.has_shared ? 1 : 0);
}

}  // namespace

hipError_t launch_gemv_gateup(const FwdArgs &a, size_t max_lds, hipStream_t s) {
    const bool f32x = !a.act_bf16;
    int maxm = a.n_tok >= 4 ? 4 : (a.n_tok >= 2 ? 2 : 1);
    while (maxm > 1 && gateup_lds(maxm, a.hidden, f32x) > max_lds) maxm >>= 1;
    const size_t lds = gateup_lds(maxm, a.hidden, f32x);
    if (lds > max_lds) return hipErrorInvalidValue;
    const int grid = units(a) * (a.inter / kPanel);
    if (f32x) {
        if (maxm == 4) gemv_gateup_kernel<4, true><<<grid, 256, lds, s>>>(a);
        else if (maxm == 2) gemv_gateup_kernel<2, true><<<grid, 256, lds, s>>>(a);
        else gemv_gateup_kernel<1, true><<<grid, 256, lds, s>>>(a);
    } else {
        if (maxm == 4) gemv_gateup_kernel<4, false><<<grid, 256, lds, s>>>(a);
        else if (maxm == 2) gemv_gateup_kernel<2, false><<<grid, 256, lds, s>>>(a);
        else gemv_gateup_kernel<1, false><<<grid, 256, lds, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_down(const FwdArgs &a, size_t max_lds, hipStream_t s) {
    int maxm = a.n_tok >= 4 ? 4 : (a.n_tok >= 2 ? 2 : 1);
    while (maxm > 1 && down_lds(maxm, a.inter) > max_lds) maxm >>= 1;
    const size_t lds = down_lds(maxm, a.inter);
    if (lds > max_lds) return hipErrorInvalidValue;
    const int grid = units(a) * (a.hidden / kPanel);
    if (maxm == 4) gemv_down_kernel<4><<<grid, 256, lds, s>>>(a);
    else if (maxm == 2) gemv_down_kernel<2><<<grid, 256, lds, s>>>(a);
    else gemv_down_kernel<1><<<grid, 256, lds, s>>>(a);
    return hipGetLastError();
}

}  // namespace coli
