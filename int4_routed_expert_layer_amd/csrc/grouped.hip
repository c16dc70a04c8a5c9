// grouped.hip -- batched expert FFNs as grouped GEMMs on MFMA, and the
// routing-weighted combine.
//
// When the union gives experts many tokens (large decode batches, prefill)
// the expert matmuls become dense contractions, [M_u x K] x [K x N] per
// union expert.  Work is a list of chunks (one expert, <= 128 rows) crossed
// with N-blocks; a persistent grid walks that list (consecutive items, which
// share the same activation rows, land on the same XCD and its L2).
//
// Per item a 256-thread workgroup stages the chunk's activation rows for 128
// reduction columns at a time into LDS as fp16 (XOR-swizzled 16-byte units,
// conflict-free for the fragment reads), while each wave streams its own
// int4 weight panels straight from HBM: one 16-byte load per lane per 1 KB
// chunk, already in B-fragment order of v_mfma_f32_16x16x32_f16.  Each
// dword is turned into eight fp16 weights in registers: q = (1024 + u) -
// 1032 (exact) times the group's fp16 scale (one rounding), so a fragment
// covers exactly one 32-wide scale group and the MFMA accumulates in fp32.
//   gate/up: A = gathered token rows (bf16 or fp32 -> fp16); each wave owns
//            32 intermediate rows of both gate and up, so SwiGLU is applied
//            in registers and h is stored as fp16.
//   down:    A = h rows of the chunk; each wave owns 64 output columns; the
//            epilogue multiplies by the entry's routing weight (1 for the
//            shared expert) and writes the entry's fp32 output row.
// The combine then sums, per token, its k routed rows in slot order and the
// shared row.  All sums have a fixed order: results are deterministic.
#include "internal.h"

namespace coli {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRowBytes = kChunkK * 2;     // one staged row: 128 fp16

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// Eight fp16 weights (columns k0..k0+7) of one packed dword times scale.
__device__ __forceinline__ half8 dequant8(uint32_t w, half2v scale) {
    const half2v k1032 = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    half2v p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t bits = ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        p[j] = (__builtin_bit_cast(half2v, bits) - k1032) * scale;
    }
    half8 r;
    r[0] = p[0][0]; r[1] = p[0][1]; r[2] = p[1][0]; r[3] = p[1][1];
    r[4] = p[2][0]; r[5] = p[2][1]; r[6] = p[3][0]; r[7] = p[3][1];
    return r;
}

__device__ __forceinline__ half2v scale_pair(uint2 sc, int s) {
    const uint32_t word = (s < 2) ? sc.x : sc.y;
    const uint16_t h = static_cast<uint16_t>(word >> (16 * (s & 1)));
    const _Float16 f = __builtin_bit_cast(_Float16, h);
    return half2v{f, f};
}

__device__ __forceinline__ int lds_unit(int m, int q) {
    return m * kRowBytes + ((q ^ (m & 15)) << 4);
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void grouped_kernel(FwdArgs a) {
    __shared__ __align__(16) uint8_t s_a[kChunkRows * kRowBytes];
    __shared__ int s_tok[kChunkRows];
    const int H = a.hidden, I = a.inter;
    const int K = GATEUP ? H : I;
    const int C = K / kChunkK;
    const int NB = GATEUP ? I / 128 : (H + 255) / 256;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l15 = lane & 15, l4 = lane >> 4;
    const int n_items = *a.n_chunks * NB;
    const int routed = a.n_tok * a.k;

    // Consecutive virtual block ids on the same XCD (blocks go round-robin
    // over 8 XCDs).
    int vb = blockIdx.x;
    if ((gridDim.x & 7) == 0) vb = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);

    for (int item = vb; item < n_items; item += gridDim.x) {
        const int chunk = item / NB, nb = item % NB;
        const ChunkDesc d = a.chunks[chunk];
        const uint8_t *blob = a.table[d.expert];
        if (!blob) continue;
        const int rows = d.rows;
        const int nf = (rows + 15) >> 4;

        // Weight panels of this wave (4 B fragments of 16 rows each), as
        // wave-uniform byte offsets into the blob.
        const uint8_t *qbase = blob + lane * 16;
        const uint8_t *sbase = blob + l15 * 8;
        uint32_t qoff[4], soff[4];
        bool bvalid[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            int panel;
            size_t qs, ss;
            if (GATEUP) {
                panel = nb * 8 + wave * 2 + (b & 1);
                qs = (b < 2) ? a.lay.gate_q : a.lay.up_q;
                ss = (b < 2) ? a.lay.gate_s : a.lay.up_s;
                bvalid[b] = true;
            } else {
                panel = nb * 16 + wave * 4 + b;
                qs = a.lay.down_q;
                ss = a.lay.down_s;
                bvalid[b] = panel < H / kPanel;
                if (!bvalid[b]) panel = 0;
            }
            qoff[b] = static_cast<uint32_t>(qs + static_cast<size_t>(panel) * C * kChunkBytes);
            soff[b] = static_cast<uint32_t>(ss + static_cast<size_t>(panel) * C * kScaleChunkBytes);
        }

        __syncthreads();
        if (GATEUP) {
            for (int m = tid; m < nf * 16; m += 256) {
                const int r = d.row0 + m;
                s_tok[m] = m < rows ? (r < routed ? a.gather[r] / a.k : r - routed) : -1;
            }
        }

        floatx4 acc[kMaxFrags][4];
#pragma unroll
        for (int f = 0; f < kMaxFrags; ++f)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[f][b] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

        for (int c = 0; c < C; ++c) {
            __syncthreads();
            // Stage rows x 128 columns of A as fp16.
            for (int i = tid; i < nf * 16 * 16; i += 256) {
                const int m = i >> 4, q = i & 15;
                half8 v = {0, 0, 0, 0, 0, 0, 0, 0};
                if (m < rows) {
                    const size_t col = static_cast<size_t>(c) * kChunkK + 8 * q;
                    if (GATEUP) {
                        const size_t off = static_cast<size_t>(s_tok[m]) * H + col;
                        if (a.act_bf16) {
                            const uint4 raw = *reinterpret_cast<const uint4 *>(
                                static_cast<const uint16_t *>(a.x) + off);
                            const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                v[2 * j] = static_cast<_Float16>(bf16_bits_to_f32(w4[j] & 0xFFFFu));
                                v[2 * j + 1] = static_cast<_Float16>(bf16_bits_to_f32(w4[j] >> 16));
                            }
                        } else {
                            const float4 *src = reinterpret_cast<const float4 *>(
                                static_cast<const float *>(a.x) + off);
                            const float4 lo = src[0], hi = src[1];
                            v[0] = static_cast<_Float16>(lo.x); v[1] = static_cast<_Float16>(lo.y);
                            v[2] = static_cast<_Float16>(lo.z); v[3] = static_cast<_Float16>(lo.w);
                            v[4] = static_cast<_Float16>(hi.x); v[5] = static_cast<_Float16>(hi.y);
                            v[6] = static_cast<_Float16>(hi.z); v[7] = static_cast<_Float16>(hi.w);
                        }
                    } else {
                        v = *reinterpret_cast<const half8 *>(a.h + static_cast<size_t>(d.row0 + m) * I + col);
                    }
                }
                *reinterpret_cast<half8 *>(s_a + lds_unit(m, q)) = v;
            }
            uint4 wq[4];
            uint2 ws[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if (bvalid[b]) {
                    wq[b] = *reinterpret_cast<const uint4 *>(qbase + qoff[b] + c * kChunkBytes);
                    ws[b] = *reinterpret_cast<const uint2 *>(sbase + soff[b] + c * kScaleChunkBytes);
                } else {
                    wq[b] = uint4{0, 0, 0, 0};
                    ws[b] = uint2{0, 0};
                }
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                half8 bf[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t w = (s == 0) ? wq[b].x : (s == 1) ? wq[b].y : (s == 2) ? wq[b].z : wq[b].w;
                    bf[b] = dequant8(w, scale_pair(ws[b], s));
                }
#pragma unroll
                for (int f = 0; f < kMaxFrags; ++f) {
                    if (f < nf) {
                        const half8 av = *reinterpret_cast<const half8 *>(
                            s_a + lds_unit(16 * f + l15, 4 * s + l4));
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            acc[f][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bf[b], acc[f][b], 0, 0, 0);
                    }
                }
            }
        }

        // Epilogue.  Lane holds D[m = 4*l4 + j][n = l15] of each 16x16 tile.
#pragma unroll
        for (int f = 0; f < kMaxFrags; ++f) {
            if (f < nf) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int m = 16 * f + 4 * l4 + j;
                    if (m < rows) {
                        if (GATEUP) {
#pragma unroll
                            for (int pb = 0; pb < 2; ++pb) {
                                const float g = acc[f][pb][j], v = acc[f][2 + pb][j];
                                const float hval = g / (1.0f + expf(-g)) * v;
                                const int col = nb * 128 + wave * 32 + pb * 16 + l15;
                                a.h[static_cast<size_t>(d.row0 + m) * I + col] = static_cast<_Float16>(hval);
                            }
                        } else {
                            const int hrow = d.row0 + m;
                            const int entry = hrow < routed ? a.gather[hrow] : hrow;
                            const float wgt = hrow < routed ? a.topk_w[entry] : 1.0f;
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                if (bvalid[b]) {
                                    const int col = (nb * 16 + wave * 4 + b) * kPanel + l15;
                                    a.ys[static_cast<size_t>(entry) * H + col] = wgt * acc[f][b][j];
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void combine_kernel(FwdArgs a) {
    const int H4 = a.hidden / 4;
    const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<size_t>(a.n_tok) * H4) return;
    const int t = static_cast<int>(idx / H4), n4 = static_cast<int>(idx % H4);
    const float4 *ys = reinterpret_cast<const float4 *>(a.ys);
    float4 acc = ys[static_cast<size_t>(t * a.k) * H4 + n4];
    for (int j = 1; j < a.k; ++j) {
        const float4 v = ys[static_cast<size_t>(t * a.k + j) * H4 + n4];
        acc.x = acc.x + v.x; acc.y = acc.y + v.y; acc.z = acc.z + v.z; acc.w = acc.w + v.w;
    }
    if (a.has_shared) {
        const float4 v = ys[static_cast<size_t>(a.n_tok * a.k + t) * H4 + n4];
        acc.x = acc.x + v.x; acc.y = acc.y + v.y; acc.z = acc.z + v.z; acc.w = acc.w + v.w;
    }
    reinterpret_cast<float4 *>(a.y)[idx] = acc;
}

int grid_for(int items, int n_cu) {
    int g = 2 * n_cu;
    if (items < g) g = items;
    if (g >= 8) g &= ~7;
    return g < 1 ? 1 : g;
}

}  // namespace

hipError_t launch_grouped_gateup(const FwdArgs &a, int max_chunks, int n_cu, hipStream_t s) {
    const int grid = grid_for(max_chunks * (a.inter / 128), n_cu);
    grouped_kernel<true><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_grouped_down(const FwdArgs &a, int max_chunks, int n_cu, hipStream_t s) {
    const int grid = grid_for(max_chunks * ((a.hidden + 255) / 256), n_cu);
    grouped_kernel<false><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_combine(const FwdArgs &a, hipStream_t s) {
    const size_t n = static_cast<size_t>(a.n_tok) * (a.hidden / 4);
    if (n == 0) return hipSuccess;
    combine_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace coli
