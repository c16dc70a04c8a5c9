// dev_gemv.h -- decode-shaped expert FFN work items on the vector ALUs.
//
// When each union expert serves one to four tokens the expert matmuls are
// matrix-vector products bound by HBM bandwidth: every weight byte is used
// once per token, so the work stays on the VALU and is shaped for streaming.
// A 256-thread workgroup owns one 16-row panel (gate/up) or two panels
// (down) of one expert; its waves split the reduction axis, each lane issues
// one 16-byte load per 1 KB chunk (fully coalesced), weight loads are double
// buffered in registers (the next group of chunks is in flight while the
// current one is multiplied), and the activations sit in LDS.
//
// Int4 expansion costs five integer ops per 8 weights.  A packed dword holds
// columns k0..k0+7 as u = q + 8 in nibble slots (j, 4+j) for the column pair
// (2j, 2j+1).  With the fp16 exponent pattern 0x6400 (1024, ulp 1):
//   pair 0: (w & 0x000F000F) | 0x64006400           -> 1024 + u
//   pair 1: (w & 0x00F000F0) | 0x64006400           -> 1024 + 16 u
//   pairs 2, 3: the same on w >> 8.
// The activations of pairs 1 and 3 are staged pre-divided by 16 (exact), so
// every v_dot2 product is (1024 + u) x or (64 + u) x.  The offsets are
// removed by seeding the dot with
//   c = -1032 (x0 + x1 + x4 + x5) - 1152 (x2' + x3' + x6' + x7')
// (x' the staged, divided values), computed once per 8 activations, so the
// dot of one dword is sum (u-8) x = sum q x up to fp32 rounding, and one
// fused multiply-add applies the fp16 group scale.  Activations enter as
// fp16 (bf16/fp32 inputs are rounded once when staged; a value outside the
// fp16 range, or not finite, sets a device error flag, as does an h value
// that rounds to inf).
//
// Int8 weights (WFmt<.., 8>) use the same scheme with one byte per column:
// u = q + 128 sits in the low byte of each fp16 half, the activations are
// staged plainly and the seed is -1152 times their sum.
//
// Partial sums are reduced across the four lanes that share a row and then
// across waves in a fixed order, so results are deterministic.
#pragma once

#include <type_traits>

#include "dev_common.h"

namespace coli {
namespace dev {

// sum over the 8 columns of one packed dword of q * x, given the staged
// activations xv (pairs 1 and 3 pre-divided by 16) and their seed c.
__device__ __forceinline__ float dot8(uint32_t w, uint4 xv, float c, uint32_t M0, uint32_t M1,
                                      uint32_t G) {
    const uint32_t w8 = w >> 8;
    float d = dot2_f16((w & M0) | G, xv.x, c);
    d = dot2_f16((w & M1) | G, xv.y, d);
    d = dot2_f16((w8 & M0) | G, xv.z, d);
    d = dot2_f16((w8 & M1) | G, xv.w, d);
    return d;
}

// Stage 8 activations into LDS as fp16 with the pair-1/3 columns divided by
// 16, and their dot seed.  Returns true if a value lies outside the fp16
// range (or is not finite).
__device__ __forceinline__ bool stage8(const float *v, uint8_t *dst_x, float *dst_c) {
    _Float16 h[8];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bool odd_pair = (i & 2) != 0;          // columns 2,3,6,7
        h[i] = static_cast<_Float16>(odd_pair ? v[i] * 0.0625f : v[i]);
        bad = bad || outside_half(v[i]);
    }
    float ce = 0.0f, co = 0.0f;
    ce = ce + static_cast<float>(h[0]);
    ce = ce + static_cast<float>(h[1]);
    ce = ce + static_cast<float>(h[4]);
    ce = ce + static_cast<float>(h[5]);
    co = co + static_cast<float>(h[2]);
    co = co + static_cast<float>(h[3]);
    co = co + static_cast<float>(h[6]);
    co = co + static_cast<float>(h[7]);
    // (1024+u) x - 1032 x = (u-8) x;  (1024+16u) x' - 1152 x' = (u-8) (16 x').
    *dst_c = -1032.0f * ce - 1152.0f * co;
    *reinterpret_cast<uint4 *>(dst_x) = __builtin_bit_cast(uint4, h);
    return bad;
}

// LDS bytes of one gate/up panel item / one down panel-group item: staged
// activations (fp16), their 8-column seeds, the cross-wave partial sums, and
// for the down items of two or more tokens (the matrix-core form) the
// 32-column seed sums.
__host__ __device__ inline size_t gateup_lds_bytes(int maxm, int hidden) {
    return static_cast<size_t>(maxm) * hidden * 2 + static_cast<size_t>(maxm) * (hidden / 8) * 4 +
           static_cast<size_t>(4) * maxm * 16 * 2 * 4;
}
// LDS floats the fused combine gets: the down item's LDS, and at least one
// token's rows (k routed + shared) of a 32-column panel pair.
__host__ __device__ inline size_t combine_lds_floats(size_t down_bytes, int k, int has_shared) {
    const size_t one_token = static_cast<size_t>(2 * kPanel) * (k + (has_shared ? 1 : 0));
    return down_bytes / sizeof(float) > one_token ? down_bytes / sizeof(float) : one_token;
}

// The down items of two to four tokens multiply on the matrix cores: each
// 32-column slice of a 16-row chunk is one v_mfma_f32_16x16x32_f16 with the
// unpacked weights as the B operand (the chunk layout is that operand's lane
// layout) and the staged h rows of the tokens as A, so the vector ALUs only
// unpack and scale (per token, the v_dot2 form costs four dots per weight
// dword).  One-token items and the gate/up items keep the v_dot2 form, which
// measured faster for them.
template <int MAXM>
constexpr bool down_mfma() { return MAXM >= 2; }

__host__ __device__ inline size_t down_lds_bytes(int maxm, int inter) {
    return static_cast<size_t>(maxm) * inter * 2 + static_cast<size_t>(maxm) * (inter / 8) * 4 +
           static_cast<size_t>(4) * maxm * 16 * 4 + (maxm >= 2 ? static_cast<size_t>(maxm) * (inter / 32) * 4 : 0);
}

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// The matrix-core form needs each 32-column slice's seed, the sum of its four
// 8-column seeds, (c0 + c1) + (c2 + c3).  The staging loops hand 8-column
// group q of a row to thread i = m K/8 + q (plus multiples of the block
// size), so the four groups of a slice are on four adjacent lanes of one
// wave, all active or all idle; the first of them stores the sum.
__device__ __forceinline__ void stage_slice_seed(float c8, float *cs32, int K, int m, int q) {
    float c = c8 + __shfl_xor(c8, 1, 64);
    c = c + __shfl_xor(c, 2, 64);
    if ((q & 3) == 0) cs32[m * (K / 32) + (q >> 2)] = c;
}

// Gate/up chunks per register buffer.  One (with two buffers and four
// workgroups per CU, 64 KB of weights in flight per CU): the HBM streams
// faster with less in flight per CU -- a plain read of 2 GiB peaks at about
// 32 KB per CU and slows beyond -- and two per buffer measured slower
// (decode B=1 gate/up 21.4 against 20.5 us, B=4 74.9 against 69.4 us).
constexpr int kGateUpGroup = 1;
// Down chunks per register buffer: one, as for gate/up (less in flight per CU;
// down 15.1 -> 15.0 us at decode B=1, 55.0 -> 54.2 us at B=4).
constexpr int kPipeGroup = 1;

// sum over the 8 columns k0..k0+7 of two int8 dwords (columns k0..k0+3 in
// w0, k0+4..k0+7 in w1, each stored as u = q + 128 in byte order k, k+2, k+1,
// k+3) of q * x, given the plainly staged activations xv and their seed c:
// (w & 0x00FF00FF) | 0x64006400 is the fp16 pair (1024 + u_k, 1024 + u_k+1),
// the same on w >> 8 gives columns k+2, k+3, and the seed removes
// 1152 x per column.
__device__ __forceinline__ float dot8_i8(uint32_t w0, uint32_t w1, uint4 xv, float c, uint32_t M8,
                                         uint32_t G) {
    float d = dot2_f16((w0 & M8) | G, xv.x, c);
    d = dot2_f16(((w0 >> 8) & M8) | G, xv.y, d);
    d = dot2_f16((w1 & M8) | G, xv.z, d);
    d = dot2_f16(((w1 >> 8) & M8) | G, xv.w, d);
    return d;
}

// Stage 8 activations into LDS as plain fp16 with the int8 dot seed; true
// if a value lies outside the fp16 range.
__device__ __forceinline__ bool stage8_i8(const float *v, uint8_t *dst_x, float *dst_c) {
    _Float16 h[8];
    float sum = 0.0f;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = static_cast<_Float16>(v[i]);
        sum = sum + static_cast<float>(h[i]);
        bad = bad || outside_half(v[i]);
    }
    // (1024 + q + 128) x - 1152 x = q x.
    *dst_c = -1152.0f * sum;
    *reinterpret_cast<uint4 *>(dst_x) = __builtin_bit_cast(uint4, h);
    return bad;
}

// Weight format of the GEMV work items: GS reduction elements per fp16 scale
// (32 or 64) and WB bits per weight (4 or 8).  A 1 KB chunk covers 16 rows x
// kCols columns (128 int4 or 64 int8); the 16 bytes of lane L hold row L & 15
// and, for each 32-column slice j of the chunk, columns 32j + 8(L >> 4) +
// 0..7: one dword (int4 nibbles, dword j) or two (int8 bytes, dwords 2j and
// 2j + 1).  A chunk's scales are [16 rows][kCols / GS] fp16; each lane
// loads its row's record (an int8 group-64 record of 2 bytes is read as the
// dword of its row pair).
template <int GS, int WB>
struct WFmt {
    static_assert((GS == 32 || GS == 64) && (WB == 4 || WB == 8), "group 32 or 64, 4 or 8 bits");
    static constexpr int kGroup = GS;
    static constexpr int kBits = WB;
    static constexpr int kCols = WB == 4 ? 128 : 64;
    static constexpr int kSlices = kCols / 32;
    static constexpr int kGroupsPerChunk = kCols / GS;
    static constexpr int kScaleChunkBytes = kPanel * kGroupsPerChunk * 2;
    using Rec = typename std::conditional<kGroupsPerChunk == 4, uint2, uint32_t>::type;
    static constexpr uint32_t kMask0 = WB == 4 ? 0x000F000Fu : 0x00FF00FFu;
    static constexpr uint32_t kMask1 = WB == 4 ? 0x00F000F0u : 0x00FF00FFu;

    __device__ static uint32_t rec_offset(int row) {
        return kGroupsPerChunk == 1 ? static_cast<uint32_t>(row & ~1) * 2
                                    : static_cast<uint32_t>(row) * kGroupsPerChunk * 2;
    }
    // Scale of slice j for the lane of row `row`.
    __device__ static float scale(Rec r, int j, int row) {
        if constexpr (kGroupsPerChunk == 4) {
            const uint32_t d = (j >> 1) ? r.y : r.x;
            return half_bits_to_f32((d >> (16 * (j & 1))) & 0xFFFFu);
        } else if constexpr (kGroupsPerChunk == 2) {
            return half_bits_to_f32((r >> (16 * (j / (GS / 32)))) & 0xFFFFu);
        } else {
            return half_bits_to_f32((r >> (16 * (row & 1))) & 0xFFFFu);
        }
    }
    // q . x over the lane's 8 columns of slice j.
    __device__ static float dot(const uint32_t (&w)[4], int j, uint4 xv, float c, uint32_t M0, uint32_t M1,
                                uint32_t G) {
        if constexpr (WB == 4) return dot8(w[j], xv, c, M0, M1, G);
        else return dot8_i8(w[2 * j], w[2 * j + 1], xv, c, M0, G);
    }
    __device__ static bool stage(const float *v, uint8_t *dst_x, float *dst_c) {
        if constexpr (WB == 4) return stage8(v, dst_x, dst_c);
        else return stage8_i8(v, dst_x, dst_c);
    }
    // The lane's 8 columns of slice j as fp16 (1024 + u, or 1024 + 16 u for
    // the int4 column pairs whose activations are staged divided by 16), in
    // column order: the B fragment of v_mfma_f32_16x16x32_f16 for this lane.
    __device__ static half8v frag(const uint32_t (&w)[4], int j, uint32_t M0, uint32_t M1, uint32_t G) {
        uint4 r;
        if constexpr (WB == 4) {
            const uint32_t x = w[j], x8 = x >> 8;
            r.x = (x & M0) | G;
            r.y = (x & M1) | G;
            r.z = (x8 & M0) | G;
            r.w = (x8 & M1) | G;
        } else {
            const uint32_t w0 = w[2 * j], w1 = w[2 * j + 1];
            r.x = (w0 & M0) | G;
            r.y = ((w0 >> 8) & M0) | G;
            r.z = (w1 & M0) | G;
            r.w = ((w1 >> 8) & M0) | G;
        }
        return __builtin_bit_cast(half8v, r);
    }
};

// Calls fn(F{}) with the format of a layer.
template <class Fn>
inline void dispatch_format(int group, int bits, Fn &&fn) {
    if (bits == 8) {
        if (group == 64) fn(WFmt<64, 8>{});
        else fn(WFmt<32, 8>{});
    } else {
        if (group == 64) fn(WFmt<64, 4>{});
        else fn(WFmt<32, 4>{});
    }
}

template <int NG, class F>
struct GateUpBuf {
    uint4 gw[NG], uw[NG];
    typename F::Rec gs[NG], us[NG];
};

// Sources of one gate/up panel: the blob descriptor, the lane offsets of a
// weight chunk and of its scales, and the panel's section offsets.
struct GateUpSrc {
    rsrc_t r;
    uint32_t vq, vs;          // per lane
    uint32_t gq, uq, gs, us;  // uniform
};

template <int NG, class F>
__device__ __forceinline__ void gateup_load(GateUpBuf<NG, F> &b, const GateUpSrc &S, int first, int step, int C) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const uint32_t c = static_cast<uint32_t>(min(first + step * g, C - 1));
        b.gw[g] = bload<uint4, kLoadStream>(S.r, S.vq, S.gq + c * kChunkBytes);
        b.uw[g] = bload<uint4, kLoadStream>(S.r, S.vq, S.uq + c * kChunkBytes);
        b.gs[g] = bload<typename F::Rec, kLoadStream>(S.r, S.vs, S.gs + c * F::kScaleChunkBytes);
        b.us[g] = bload<typename F::Rec, kLoadStream>(S.r, S.vs, S.us + c * F::kScaleChunkBytes);
    }
}

template <int MAXM, int NG, class F>
__device__ __forceinline__ void gateup_math(const GateUpBuf<NG, F> &b, const uint8_t *xs, const float *cs, int H,
                                            int first, int step, int count, int row, int kq, int mc,
                                            uint32_t M0, uint32_t M1, uint32_t G, float *gacc,
                                            float *vacc) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        if (g >= count) continue;
        const int c = first + step * g;
        const uint32_t gws[4] = {b.gw[g].x, b.gw[g].y, b.gw[g].z, b.gw[g].w};
        const uint32_t uws[4] = {b.uw[g].x, b.uw[g].y, b.uw[g].z, b.uw[g].w};
        // The lane's activations and seeds of this chunk: one base address
        // each, slice s at a constant offset (64 bytes of x, 4 seeds).
        const int k0 = c * F::kCols + 8 * kq;
#pragma unroll
        for (int s = 0; s < F::kSlices; ++s) {
            const float sg = F::scale(b.gs[g], s, row);
            const float su = F::scale(b.us[g], s, row);
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                if (m < mc) {
                    const uint8_t *xrow = xs + (static_cast<size_t>(m) * H + k0) * 2;
                    const float *crow = cs + m * (H / 8) + (k0 >> 3);
                    const uint4 xv = *reinterpret_cast<const uint4 *>(xrow + 64 * s);
                    const float c8 = crow[4 * s];
                    gacc[m] = __builtin_fmaf(sg, F::dot(gws, s, xv, c8, M0, M1, G), gacc[m]);
                    vacc[m] = __builtin_fmaf(su, F::dot(uws, s, xv, c8, M0, M1, G), vacc[m]);
                }
            }
        }
    }
}

// One gate/up work item: rows 16p..16p+15 of expert blob `blob`, for the M
// tokens of hidden-buffer rows r0..r0+M-1 (rows.token(row) names the token of
// a row).  Writes h rows (fp16), read by a later launch.  All 256 threads
// must call it (it synchronises the workgroup).  NG chunks per register
// buffer (two buffers in flight): more for few workgroups per CU.  F is the
// weight format (WFmt).
template <class F, int MAXM, int NG = kGateUpGroup, class Rows>
__device__ void gateup_panel(const FwdArgs &a, const Rows &rows, const uint8_t *blob, int r0, int M, int p,
                             uint8_t *lds, uint32_t lds_addr) {
    const int H = a.hidden, I = a.inter;
    const int C = H / F::kCols;
    const int tid = opaque_tid(), wave = wave_id(), lane = tid & 63;
    const int row = lane & 15, kq = lane >> 4;
    GateUpSrc P;
    P.r = make_rsrc(blob, static_cast<uint32_t>(a.lay.total));
    P.vq = static_cast<uint32_t>(lane) * 16;
    P.vs = F::rec_offset(row);
    P.gq = static_cast<uint32_t>(a.lay.gate_q + static_cast<size_t>(p) * C * kChunkBytes);
    P.uq = static_cast<uint32_t>(a.lay.up_q + static_cast<size_t>(p) * C * kChunkBytes);
    P.gs = static_cast<uint32_t>(a.lay.gate_s + static_cast<size_t>(p) * C * F::kScaleChunkBytes);
    P.us = static_cast<uint32_t>(a.lay.up_s + static_cast<size_t>(p) * C * F::kScaleChunkBytes);
    // Chunks of this wave: wave, wave + 4, ...
    const int nper = wave < C ? (C - wave + 3) / 4 : 0;
    const uint32_t M0 = vconst(F::kMask0), M1 = vconst(F::kMask1), G = vconst(0x64006400u);

    // LDS: x [MAXM][H] fp16, seeds [MAXM][H/8] fp32, partials [4][MAXM][16][2].
    uint8_t *xs = lds;
    float *cs = reinterpret_cast<float *>(lds + static_cast<size_t>(MAXM) * H * 2);
    float *red = cs + MAXM * (H / 8);

    for (int mb = 0; mb < M; mb += MAXM) {
        const int mc = min(MAXM, M - mb);
        float gacc[MAXM], vacc[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) gacc[m] = vacc[m] = 0.0f;

        GateUpBuf<NG, F> A, B;
        bool b_issued = false;
        if (a.act_bf16 && (H * 2) % 1024 == 0) {
            // bf16 rows are copied straight into the staging area (1 KB per
            // wave instruction) before the weight loads are issued; the wait
            // below then covers only those copies (memory returns are counted
            // in issue order), not the first weight burst.  Each thread then
            // turns its own 16 bytes into the staged fp16 form in place.
            __syncthreads();                    // the previous row block is done with xs
            const int per_row = H / 512;
            int toks[MAXM];                     // token lookups first: none sits between the copies
#pragma unroll
            for (int m = 0; m < MAXM; ++m) toks[m] = m < mc ? rows.token(r0 + mb + m) : 0;
            for (int ci = wave; ci < mc * per_row; ci += 4) {
                const int m = ci / per_row, part = ci % per_row;
                int t = toks[0];
#pragma unroll
                for (int mm = 1; mm < MAXM; ++mm) t = m == mm ? toks[mm] : t;
                copy16_to_lds(static_cast<const uint16_t *>(a.x) + static_cast<size_t>(t) * H + part * 512 + 8 * lane,
                              lds_addr + static_cast<uint32_t>((m * H + part * 512) * 2));
            }
            // Both weight buffers go out before the wait (weights do not
            // depend on x): twice the bytes in flight while x lands.  Lookahead
            // past the last chunk repeats it (never used), so the count of
            // loads behind the copies is always 8 NG.
            gateup_load(A, P, wave, 4, C);
            gateup_load(B, P, wave + 4 * NG, 4, C);
            b_issued = true;
            // Plain barriers here: __syncthreads' fence would also wait for
            // the weight loads just issued.
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8 * NG) : "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            bool bad = false;
            for (int i = tid; i < mc * (H / 8); i += 256) {
                const int m = i / (H / 8), q = i % (H / 8);
                uint8_t *dst = xs + (static_cast<size_t>(m) * H + 8 * q) * 2;
                const uint4 raw = *reinterpret_cast<const uint4 *>(dst);
                const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
                float v[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = bf16_bits_to_f32(w4[j] & 0xFFFFu);
                    v[2 * j + 1] = bf16_bits_to_f32(w4[j] >> 16);
                }
                bad = F::stage(v, dst, cs + m * (H / 8) + q) || bad;
            }
            flag_if(bad, a.err, kErrActRange);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        } else {
        gateup_load(A, P, wave, 4, C);          // weights do not depend on x
        __syncthreads();
        bool bad = false;
        for (int i = tid; i < mc * (H / 8); i += 256) {
            const int m = i / (H / 8), q = i % (H / 8);
            const int t = rows.token(r0 + mb + m);
            float v[8];
            if (a.act_bf16) {
                const uint4 raw = gload<uint4>(static_cast<const uint16_t *>(a.x) + static_cast<size_t>(t) * H + 8 * q);
                const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = bf16_bits_to_f32(w4[j] & 0xFFFFu);
                    v[2 * j + 1] = bf16_bits_to_f32(w4[j] >> 16);
                }
            } else {
                const float *src = static_cast<const float *>(a.x) + static_cast<size_t>(t) * H + 8 * q;
                const float4 lo = gload<float4>(src), hi = gload<float4>(src + 4);
                v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
                v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
            }
            bad = F::stage(v, xs + (static_cast<size_t>(m) * H + 8 * q) * 2, cs + m * (H / 8) + q) || bad;
        }
        flag_if(bad, a.err, kErrActRange);
        __syncthreads();
        }
        // i indexes this wave's chunk list; buffers alternate A, B.
        for (int i = 0; i < nper; i += 2 * NG) {
            if (i + NG < nper && (i > 0 || !b_issued)) gateup_load(B, P, wave + 4 * (i + NG), 4, C);
            gateup_math<MAXM>(A, xs, cs, H, wave + 4 * i, 4, min(NG, nper - i), row, kq, mc, M0, M1, G,
                              gacc, vacc);
            if (i + 2 * NG < nper) gateup_load(A, P, wave + 4 * (i + 2 * NG), 4, C);
            if (i + NG < nper)
                gateup_math<MAXM>(B, xs, cs, H, wave + 4 * (i + NG), 4, min(NG, nper - i - NG), row, kq, mc, M0, M1, G,
                                  gacc, vacc);
        }
        // The four lanes of a row hold the dots of its four 8-column groups.
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
        bool hbad = false;
        if (tid < mc * 16) {
            const int m = tid >> 4, r = tid & 15;
            float g = 0.0f, v = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                g = g + red[((w * MAXM + m) * 16 + r) * 2 + 0];
                v = v + red[((w * MAXM + m) * 16 + r) * 2 + 1];
            }
            const _Float16 hh = static_cast<_Float16>(swiglu(g, v));
            hbad = half_nonfinite(hh);
            a.h[static_cast<size_t>(r0 + mb + m) * I + p * kPanel + r] = hh;
        }
        flag_if(hbad, a.err, kErrHiddenRange);
    }
}

// Rows of a forward call read straight from its routing arrays (kernels that
// run after the routing kernels have finished).
struct PlainRows {
    const FwdArgs &a;
    __device__ int token(int row) const { return token_of_row(a, row); }
    __device__ int entry(int row) const { return row < a.n_tok * a.k ? ld_uniform(a.gather + row) : row; }
    __device__ float weight(int row) const {
        return row < a.n_tok * a.k ? ld_uniform(a.topk_w + ld_uniform(a.gather + row)) : 1.0f;
    }
};

template <class F>
struct DownBuf {
    uint4 w[kPipeGroup];
    typename F::Rec s[kPipeGroup];
};

template <class F>
__device__ __forceinline__ void down_load(DownBuf<F> &b, rsrc_t r, uint32_t vq, uint32_t vs, uint32_t sq, uint32_t ss,
                                          int first, int C) {
#pragma unroll
    for (int g = 0; g < kPipeGroup; ++g) {
        const uint32_t c = static_cast<uint32_t>(min(first + g, C - 1));
        b.w[g] = bload<uint4, kLoadStream>(r, vq, sq + c * kChunkBytes);
        b.s[g] = bload<typename F::Rec, kLoadStream>(r, vs, ss + c * F::kScaleChunkBytes);
    }
}

template <int MAXM, class F>
__device__ __forceinline__ void down_math(const DownBuf<F> &b, const uint8_t *hs, const float *cs, int I,
                                          int first, int count, int row, int kq, int mc, uint32_t M0,
                                          uint32_t M1, uint32_t G, float *acc) {
#pragma unroll
    for (int g = 0; g < kPipeGroup; ++g) {
        if (g >= count) continue;
        const int c = first + g;
        const uint32_t ws[4] = {b.w[g].x, b.w[g].y, b.w[g].z, b.w[g].w};
        const int k0 = c * F::kCols + 8 * kq;
#pragma unroll
        for (int s = 0; s < F::kSlices; ++s) {
            const float sf = F::scale(b.s[g], s, row);
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                if (m < mc) {
                    const uint8_t *hrow = hs + (static_cast<size_t>(m) * I + k0) * 2;
                    const float *crow = cs + m * (I / 8) + (k0 >> 3);
                    const uint4 hv = *reinterpret_cast<const uint4 *>(hrow + 64 * s);
                    const float c8 = crow[4 * s];
                    acc[m] = __builtin_fmaf(sf, F::dot(ws, s, hv, c8, M0, M1, G), acc[m]);
                }
            }
        }
    }
}

// Matrix-core form of down_math: each 32-column slice s of a chunk is one
// v_mfma_f32_16x16x32_f16 whose B operand is the lane's unpacked dword s
// (F::frag: weight row L & 15, columns 32 s + 8 (L >> 4) .. + 7, exactly the
// chunk layout) and whose A operand is the staged h row of token L & 15
// (rows past MAXM read token 0; their results are never used).  Lane L < 16
// then holds token m's dot with weight row L in d[m]; adding the slice's
// seed sum gives the slice's dot product (the quantity the four v_dot2
// groups form, summed in another order), and the group scale is applied per
// slice as in down_math.
template <int MAXM, class F>
__device__ __forceinline__ void down_math_mfma(const DownBuf<F> &b, const uint8_t *hs, const float *cs32, int I,
                                               int first, int count, int row, int kq, int mc, uint32_t M0,
                                               uint32_t M1, uint32_t G, float *acc) {
    const int ma = row < MAXM ? row : 0;
#pragma unroll
    for (int g = 0; g < kPipeGroup; ++g) {
        if (g >= count) continue;
        const int c = first + g;
        const uint32_t ws[4] = {b.w[g].x, b.w[g].y, b.w[g].z, b.w[g].w};
        const uint8_t *hrow = hs + (static_cast<size_t>(ma) * I + c * F::kCols + 8 * kq) * 2;
        const float *crow = cs32 + (c * F::kCols) / 32;
#pragma unroll
        for (int s = 0; s < F::kSlices; ++s) {
            const half8v av = *reinterpret_cast<const half8v *>(hrow + 64 * s);
            const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
            const float4v d = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, F::frag(ws, s, M0, M1, G), zero, 0, 0, 0);
            const float sf = F::scale(b.s[g], s, row);
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
                if (m < mc) acc[m] = __builtin_fmaf(sf, d[m] + crow[m * (I / 32) + s], acc[m]);
        }
    }
}

// One down work item: output panels 2pg and 2pg+1 of expert blob `blob` for
// hidden rows r0..r0+M-1.  Wave w takes panel 2pg + (w & 1) and reduction
// half (w >> 1); the halves are summed through LDS in a fixed order.  Writes
// ys row rows.entry(row) scaled by rows.weight(row) (the routing weight of a
// routed row, 1 for a shared row).  With COHERENT, ys is written
// device-coherently (the fused combine's last arriver, in the same launch,
// reads it).  h comes from an earlier launch.  All 256 threads must call it.
// F is the weight format (WFmt).
template <class F, int MAXM, bool COHERENT = false, class Rows>
__device__ void down_panelgroup(const FwdArgs &a, const Rows &rows, const uint8_t *blob, int r0, int M, int pg,
                                uint8_t *lds, uint32_t lds_addr) {
    const int H = a.hidden, I = a.inter;
    const int C = I / F::kCols;
    const int tid = opaque_tid(), wave = wave_id(), lane = tid & 63;
    const int row = lane & 15, kq = lane >> 4;
    const int p = 2 * pg + (wave & 1), half = wave >> 1;
    const int c_begin = half == 0 ? 0 : (C + 1) / 2;
    const int c_end = half == 0 ? (C + 1) / 2 : C;
    const int nper = c_end - c_begin;
    const rsrc_t rs = make_rsrc(blob, static_cast<uint32_t>(a.lay.total));
    const uint32_t vq = static_cast<uint32_t>(lane) * 16, vs = F::rec_offset(row);
    const uint32_t sq = static_cast<uint32_t>(a.lay.down_q + static_cast<size_t>(p) * C * kChunkBytes);
    const uint32_t ss = static_cast<uint32_t>(a.lay.down_s + static_cast<size_t>(p) * C * F::kScaleChunkBytes);
    uint8_t *hs = lds;
    float *cs = reinterpret_cast<float *>(lds + static_cast<size_t>(MAXM) * I * 2);
    float *red = cs + MAXM * (I / 8);
    float *cs32 = red + 4 * MAXM * 16;
    const uint32_t M0 = vconst(F::kMask0), M1 = vconst(F::kMask1), G = vconst(0x64006400u);

    for (int mb = 0; mb < M; mb += MAXM) {
        const int mc = min(MAXM, M - mb);
        float acc[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;
        // Output entry and routing weight of each row, looked up while the
        // first weights and h are in flight (not as a chain in front of the
        // ys stores, nor in front of the weight loads).
        int ents[MAXM];
        float wgts[MAXM];
        auto lookup_rows = [&]() {
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                const int hrow = r0 + mb + (m < mc ? m : 0);
                ents[m] = rows.entry(hrow);
                wgts[m] = rows.weight(hrow);
            }
        };
        DownBuf<F> A, B;
        bool b_issued = false;
        __syncthreads();                        // the previous row block is done with hs
        if ((I * 2) % 1024 == 0) {
            // h rows (fp16, from an earlier launch) are copied straight into
            // the staging area before the weight loads, and converted in
            // place once the copies alone have landed (as in gateup_panel).
            const int per_row = I / 512;
            for (int ci = wave; ci < mc * per_row; ci += 4) {
                const int m = ci / per_row, part = ci % per_row;
                copy16_to_lds(a.h + static_cast<size_t>(r0 + mb + m) * I + part * 512 + 8 * lane,
                              lds_addr + static_cast<uint32_t>((m * I + part * 512) * 2));
            }
            // Both weight buffers go out before the wait, as in gateup_panel
            // (lookahead past the half's last chunk is clamped and unused).
            down_load(A, rs, vq, vs, sq, ss, c_begin, C);
            down_load(B, rs, vq, vs, sq, ss, c_begin + kPipeGroup, C);
            b_issued = true;
            lookup_rows();
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kPipeGroup) : "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            for (int i = tid; i < mc * (I / 8); i += 256) {
                const int m = i / (I / 8), q = i % (I / 8);
                uint8_t *dst = hs + (static_cast<size_t>(m) * I + 8 * q) * 2;
                const uint4 raw = *reinterpret_cast<const uint4 *>(dst);
                const _Float16 *hv = reinterpret_cast<const _Float16 *>(&raw);
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = static_cast<float>(hv[j]);
                F::stage(v, dst, cs + m * (I / 8) + q);
                if constexpr (down_mfma<MAXM>()) stage_slice_seed(cs[m * (I / 8) + q], cs32, I, m, q);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        } else {
            down_load(A, rs, vq, vs, sq, ss, c_begin, C);
            lookup_rows();
            for (int i = tid; i < mc * (I / 8); i += 256) {
                const int m = i / (I / 8), q = i % (I / 8);
                const _Float16 *src = a.h + static_cast<size_t>(r0 + mb + m) * I + 8 * q;
                const uint4 raw = gload<uint4>(src);     // h comes from an earlier launch
                const _Float16 *hv = reinterpret_cast<const _Float16 *>(&raw);
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = static_cast<float>(hv[j]);
                F::stage(v, hs + (static_cast<size_t>(m) * I + 8 * q) * 2, cs + m * (I / 8) + q);
                if constexpr (down_mfma<MAXM>()) stage_slice_seed(cs[m * (I / 8) + q], cs32, I, m, q);
            }
            __syncthreads();
        }
        auto math = [&](const DownBuf<F> &buf, int first, int count) {
            if constexpr (down_mfma<MAXM>())
                down_math_mfma<MAXM>(buf, hs, cs32, I, first, count, row, kq, mc, M0, M1, G, acc);
            else
                down_math<MAXM>(buf, hs, cs, I, first, count, row, kq, mc, M0, M1, G, acc);
        };
        for (int i = 0; i < nper; i += 2 * kPipeGroup) {
            if (i + kPipeGroup < nper && (i > 0 || !b_issued))
                down_load(B, rs, vq, vs, sq, ss, c_begin + i + kPipeGroup, C);
            math(A, c_begin + i, min(kPipeGroup, nper - i));
            if (i + 2 * kPipeGroup < nper) down_load(A, rs, vq, vs, sq, ss, c_begin + i + 2 * kPipeGroup, C);
            if (i + kPipeGroup < nper) math(B, c_begin + i + kPipeGroup, min(kPipeGroup, nper - i - kPipeGroup));
        }
        if constexpr (!down_mfma<MAXM>()) {
            // The four lanes of a row hold the dots of its four 8-column groups.
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                acc[m] = acc[m] + __shfl_xor(acc[m], 16, 64);
                acc[m] = acc[m] + __shfl_xor(acc[m], 32, 64);
            }
        }
        if (lane < 16) {
#pragma unroll
            for (int m = 0; m < MAXM; ++m) red[(wave * MAXM + m) * 16 + row] = acc[m];
        }
        __syncthreads();
        if (tid < 2 * mc * 16) {
            const int side = tid / (mc * 16), rest = tid % (mc * 16);
            const int m = rest >> 4, r = rest & 15;
            // waves `side` (first half) and `side + 2` (second half)
            const float d = red[(side * MAXM + m) * 16 + r] + red[((side + 2) * MAXM + m) * 16 + r];
            int entry = ents[0];
            float wgt = wgts[0];
#pragma unroll
            for (int mm = 1; mm < MAXM; ++mm) {
                entry = m == mm ? ents[mm] : entry;
                wgt = m == mm ? wgts[mm] : wgt;
            }
            float *dst = a.ys + static_cast<size_t>(entry) * H + (2 * pg + side) * kPanel + r;
            if (COHERENT) store_coherent(dst, wgt * d);
            else *dst = wgt * d;
        }
    }
}

// y rows for output panels 2pg, 2pg+1: per token, its k routed rows in slot
// order, then the shared row.  Same order as the standalone combine kernel.
// The rows were written by other workgroups with store_coherent.  All rows
// of as many tokens as fit in `cap` floats of LDS are loaded at once (two
// loads in flight per thread), so the tail costs about one memory round trip
// per pass instead of one per row.  All threads of the workgroup must call it.
__device__ __forceinline__ void combine_panelgroup(const FwdArgs &a, int pg, float *lds, int cap) {
    const int H = a.hidden, k = a.k;
    const int nrows = k + (a.has_shared ? 1 : 0);
    const int per_tok = 2 * kPanel * nrows;
    const int tpp = cap / per_tok > 0 ? cap / per_tok : 1;
    const int col0 = 2 * kPanel * pg;
    const int tid = threadIdx.x;
    auto src = [&](int t0, int i) {
        // item i of a pass: token t0 + i / per_tok, row j, column c
        const int tt = i / per_tok, rem = i % per_tok;
        const int j = rem / (2 * kPanel), c = rem % (2 * kPanel);
        const int t = t0 + tt;
        const int row = j < k ? t * k + j : a.n_tok * k + t;
        return a.ys + static_cast<size_t>(row) * H + col0 + c;
    };
    for (int t0 = 0; t0 < a.n_tok; t0 += tpp) {
        const int nt = min(tpp, a.n_tok - t0);
        const int n = nt * per_tok;
        for (int i = tid; i < n; i += 2 * blockDim.x) {
            const int i2 = i + static_cast<int>(blockDim.x);
            const float v0 = load_coherent(src(t0, i));
            const float v1 = i2 < n ? load_coherent(src(t0, i2)) : 0.0f;
            lds[i] = v0;
            if (i2 < n) lds[i2] = v1;
        }
        __syncthreads();
        for (int i = tid; i < nt * 2 * kPanel; i += blockDim.x) {
            const int tt = i / (2 * kPanel), c = i % (2 * kPanel);
            const float *r = lds + tt * per_tok + c;
            float acc = r[0];
            for (int j = 1; j < nrows; ++j) acc = acc + r[j * 2 * kPanel];
            a.y[static_cast<size_t>(t0 + tt) * H + col0 + c] = acc;
        }
        __syncthreads();
    }
}

}  // namespace dev
}  // namespace coli
