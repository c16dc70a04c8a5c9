// grouped.hip -- batched expert FFNs as grouped GEMMs on MFMA, and the
// routing-weighted combine.
//
// When the union gives experts many tokens (large decode batches, prefill)
// the expert matmuls become dense contractions, [M_u x K] x [K x N] per
// union expert.  Work is a list of chunks (one expert, <= 128 rows) crossed
// with N-blocks; a persistent grid walks that list (consecutive items, which
// share the same activation rows, land on the same XCD and its L2).
//
// Per item a 256-thread workgroup copies the chunk's fp16 activation rows for
// 128 reduction columns at a time straight from global memory into LDS
// (global_load_lds, double-buffered: the next 128 columns are in flight while
// the current ones are multiplied; XOR-swizzled 16-byte units, conflict-free
// for the fragment reads), while each wave streams its own int4 weight
// panels from HBM (prefetched one step ahead): one 16-byte load per lane per
// 1 KB chunk, already in B-fragment order of v_mfma_f32_16x16x32_f16.  Each
// dword is turned into eight fp16 weights in registers: q = (1024 + u) -
// 1032 (exact) times the group's fp16 scale (one rounding), so a fragment
// covers exactly one 32-wide scale group and the MFMA accumulates in fp32.
//   gate/up: A = gathered token rows (fp16 copy of x); each wave owns
//            32 intermediate rows of both gate and up, so SwiGLU is applied
//            in registers and h is stored as fp16.
//   down:    A = h rows of the chunk; each wave owns 64 output columns; the
//            epilogue multiplies by the entry's routing weight (1 for the
//            shared expert) and writes the entry's fp32 output row.
// The combine then sums, per token, its k routed rows in slot order and the
// shared row.  All sums have a fixed order: results are deterministic.
#include "dev_common.h"

namespace coli {
namespace {

using dev::gload;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRowBytes = kChunkK * 2;     // one staged row: 128 fp16

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// Keeps a constant in a VGPR so the compiler can use three-operand
// v_and_or_b32 (VOP3 cannot encode literals on this ISA).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
    asm volatile("" : "+v"(c));
    return c;
}

// Eight fp16 weights (columns k0..k0+7) of one packed dword times scale.
// Column pairs (0,1) and (4,5) come out as 1024 + u, pairs (2,3) and (6,7)
// as 1024 + 16 u (no shift needed); both are turned into the exact integer
// q = u - 8 and then multiplied by the fp16 group scale (one rounding).
__device__ __forceinline__ half8 dequant8(uint32_t w, half2v scale, uint32_t M0, uint32_t M1, uint32_t G) {
    const half2v k1032 = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    const half2v k16th = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
    const half2v km72 = {static_cast<_Float16>(-72.0f), static_cast<_Float16>(-72.0f)};
    const uint32_t w8 = w >> 8;
    const half2v p0 = __builtin_bit_cast(half2v, (w & M0) | G) - k1032;
    const half2v p1 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, (w & M1) | G), k16th, km72);
    const half2v p2 = __builtin_bit_cast(half2v, (w8 & M0) | G) - k1032;
    const half2v p3 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, (w8 & M1) | G), k16th, km72);
    const half2v q0 = p0 * scale, q1 = p1 * scale, q2 = p2 * scale, q3 = p3 * scale;
    half8 r;
    r[0] = q0[0]; r[1] = q0[1]; r[2] = q1[0]; r[3] = q1[1];
    r[4] = q2[0]; r[5] = q2[1]; r[6] = q3[0]; r[7] = q3[1];
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

// Direct global -> LDS copy of 16 bytes per lane: lane L's bytes land at
// lds_base + 16 L (lds_base must be wave-uniform).
__device__ __forceinline__ void copy16_to_lds(const void *src, uint8_t *lds_base) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(src),
                                     (void __attribute__((address_space(3))) *)(lds_base), 16, 0, 0);
}

struct BFrag {
    uint4 q[4];
    uint2 s[4];
};

// State of one work item (chunk x N-block) shared by its K loop and
// epilogue.
struct ItemState {
    const _Float16 *asrc;
    uint32_t src_off[2][4];      // A rows staged by this wave (fp16 elements, column 0)
    int my_groups;
    dev::rsrc_t brs;             // weight blob
    uint32_t qlane, slane;
    uint32_t qoff[4], soff[4];   // this wave's 4 B panels
    bool bvalid[4];
    int row0, rows, nb, C;
};

// K loop and epilogue of one item with NF 16-row fragments (rows of the
// chunk past `rows` are padding, computed and discarded).  A fixed fragment
// count keeps the MFMA stream free of per-fragment branches.
template <bool GATEUP, int NF>
__device__ __forceinline__ void run_item(const FwdArgs &a, const ItemState &st, uint8_t (*s_a)[kChunkRows * kRowBytes]) {
    const int H = a.hidden, I = a.inter;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l15 = lane & 15, l4 = lane >> 4;
    const int routed = a.n_tok * a.k;
    auto stage = [&](int c, int buf) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            if (g < st.my_groups) {
                const int grp = wave + 4 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    copy16_to_lds(st.asrc + st.src_off[g][i] + c * kChunkK, &s_a[buf][(grp * 16 + i * 4) * kRowBytes]);
            }
        }
    };
    auto load_b = [&](int c, BFrag &f) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f.q[b] = dev::bload<uint4>(st.brs, st.qlane, st.qoff[b] + static_cast<uint32_t>(c) * kChunkBytes);
            f.s[b] = dev::bload<uint2>(st.brs, st.slane, st.soff[b] + static_cast<uint32_t>(c) * kScaleChunkBytes);
        }
    };

    floatx4 acc[NF][4];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[f][b] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // LDS byte offset of this lane's A fragment for k-step s (frag f adds
    // f * 16 rows).
    uint32_t a_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a_off[s] = lds_unit(l15, 4 * s + l4);
    const uint32_t M0 = vconst(0x000F000Fu), M1 = vconst(0x00F000F0u), G = vconst(0x64006400u);

    BFrag bn, bc;
    stage(0, 0);
    load_b(0, bn);
    for (int c = 0; c < st.C; ++c) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        bc = bn;
        if (c + 1 < st.C) {
            stage(c + 1, (c + 1) & 1);
            load_b(c + 1, bn);
        }
        const uint8_t *tile = s_a[c & 1];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8 bf[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t w = (s == 0) ? bc.q[b].x : (s == 1) ? bc.q[b].y : (s == 2) ? bc.q[b].z : bc.q[b].w;
                bf[b] = dequant8(w, scale_pair(bc.s[b], s), M0, M1, G);
            }
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const half8 av = *reinterpret_cast<const half8 *>(tile + a_off[s] + f * 16 * kRowBytes);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[f][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bf[b], acc[f][b], 0, 0, 0);
            }
        }
    }

    // Epilogue.  Lane holds D[m = 4*l4 + j][n = l15] of each 16x16 tile.
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 16 * f + 4 * l4 + j;
            if (m < st.rows) {
                if (GATEUP) {
#pragma unroll
                    for (int pb = 0; pb < 2; ++pb) {
                        const float g = acc[f][pb][j], v = acc[f][2 + pb][j];
                        const float hval = g / (1.0f + expf(-g)) * v;
                        const int col = st.nb * 128 + wave * 32 + pb * 16 + l15;
                        a.h[static_cast<size_t>(st.row0 + m) * I + col] = static_cast<_Float16>(hval);
                    }
                } else {
                    const int hrow = st.row0 + m;
                    const int entry = hrow < routed ? a.gather[hrow] : hrow;
                    const float wgt = hrow < routed ? a.topk_w[entry] : 1.0f;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        if (st.bvalid[b]) {
                            const int col = (st.nb * 16 + wave * 4 + b) * kPanel + l15;
                            a.ys[static_cast<size_t>(entry) * H + col] = wgt * acc[f][b][j];
                        }
                    }
                }
            }
        }
    }
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void grouped_kernel(FwdArgs a) {
    // Two A tiles (double buffer): kChunkRows rows x 128 fp16 each.
    __shared__ __align__(16) uint8_t s_a[2][kChunkRows * kRowBytes];
    __shared__ int s_tok[kChunkRows];
    const int H = a.hidden, I = a.inter;
    const int K = GATEUP ? H : I;
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
        ItemState st;
        st.asrc = GATEUP ? a.xh : a.h;
        st.row0 = d.row0;
        st.rows = d.rows;
        st.nb = nb;
        st.C = K / kChunkK;
        const int nf = (d.rows + 15) >> 4;
        // Fragment count: 2 for small chunks, else 8 (padding rows are
        // computed and discarded).
        const int nfc = nf > 2 ? 8 : 2;

        // Weight panels of this wave (4 B fragments of 16 rows each), as
        // wave-uniform byte offsets into the blob, read with buffer loads.
        st.brs = dev::make_rsrc(blob, static_cast<uint32_t>(a.lay.total));
        st.qlane = static_cast<uint32_t>(lane) * 16;
        st.slane = static_cast<uint32_t>(l15) * 8;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            int panel;
            size_t qs, ss;
            if (GATEUP) {
                panel = nb * 8 + wave * 2 + (b & 1);
                qs = (b < 2) ? a.lay.gate_q : a.lay.up_q;
                ss = (b < 2) ? a.lay.gate_s : a.lay.up_s;
                st.bvalid[b] = true;
            } else {
                panel = nb * 16 + wave * 4 + b;
                qs = a.lay.down_q;
                ss = a.lay.down_s;
                st.bvalid[b] = panel < H / kPanel;
                if (!st.bvalid[b]) panel = 0;
            }
            st.qoff[b] = static_cast<uint32_t>(qs + static_cast<size_t>(panel) * st.C * kChunkBytes);
            st.soff[b] = static_cast<uint32_t>(ss + static_cast<size_t>(panel) * st.C * kScaleChunkBytes);
        }

        __syncthreads();   // previous item is done with s_tok and the A tiles
        for (int m = tid; m < kChunkRows; m += 256) {
            // Rows past `rows` repeat row 0: their results are discarded.
            const int mm = m < d.rows ? m : 0;
            const int r = d.row0 + mm;
            s_tok[m] = GATEUP ? (r < routed ? a.gather[r] / a.k : r - routed) : r;
        }
        __syncthreads();
        // This wave stages 16-row groups wave, wave+4 of the first nfc*16
        // rows: one copy16 per 4 rows, swizzled on the source side so that
        // lane L fills slot (L & 15) of row (L >> 4).
        const size_t arow = GATEUP ? static_cast<size_t>(H) : static_cast<size_t>(I);
        st.my_groups = nfc > wave ? (nfc - wave + 3) / 4 : 0;
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = (wave + 4 * g) * 16 + i * 4 + l4;
                const int q = l15 ^ (m & 15);
                st.src_off[g][i] = static_cast<uint32_t>(s_tok[m]) * static_cast<uint32_t>(arow) + 8 * q;
            }
        if (nfc == 8) run_item<GATEUP, 8>(a, st, s_a);
        else run_item<GATEUP, 2>(a, st, s_a);
    }
}

// fp16 copy of the activations (the A operand of the gate/up GEMM).
__global__ __launch_bounds__(256) void to_half_kernel(const void *x, int act_bf16, size_t n8, _Float16 *xh) {
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n8) return;
    float v[8];
    if (act_bf16) {
        const uint4 raw = reinterpret_cast<const uint4 *>(x)[i];
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_bits_to_f32(w4[j] & 0xFFFFu);
            v[2 * j + 1] = bf16_bits_to_f32(w4[j] >> 16);
        }
    } else {
        const float4 lo = reinterpret_cast<const float4 *>(x)[2 * i];
        const float4 hi = reinterpret_cast<const float4 *>(x)[2 * i + 1];
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    }
    half8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = static_cast<_Float16>(v[j]);
    reinterpret_cast<half8 *>(xh)[i] = h;
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

hipError_t launch_to_half(const FwdArgs &a, hipStream_t s) {
    const size_t n8 = static_cast<size_t>(a.n_tok) * a.hidden / 8;
    if (n8 == 0) return hipSuccess;
    launch(to_half_kernel, static_cast<unsigned>((n8 + 255) / 256), 256, 0, s, a.x, a.act_bf16, n8, a.xh);
    return hipGetLastError();
}

hipError_t launch_grouped_gateup(const FwdArgs &a, int max_chunks, int n_cu, hipStream_t s) {
    const int grid = grid_for(max_chunks * (a.inter / 128), n_cu);
    launch(grouped_kernel<true>, grid, 256, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_grouped_down(const FwdArgs &a, int max_chunks, int n_cu, hipStream_t s) {
    const int grid = grid_for(max_chunks * ((a.hidden + 255) / 256), n_cu);
    launch(grouped_kernel<false>, grid, 256, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const FwdArgs &a, hipStream_t s) {
    const size_t n = static_cast<size_t>(a.n_tok) * (a.hidden / 4);
    if (n == 0) return hipSuccess;
    launch(combine_kernel, static_cast<unsigned>((n + 255) / 256), 256, 0, s, a);
    return hipGetLastError();
}

}  // namespace coli
