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
typedef float floatx16 __attribute__((ext_vector_type(16)));

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
    uint32_t qv_even, qv_odd, sv; // per-lane byte offsets of the B slots and scales
    uint32_t qoff[2], soff[2];   // this wave's two 32-row B tiles (uniform)
    bool bvalid[2];
    int row0, rows, nb, C;
};

// K loop and epilogue of one item on v_mfma_f32_32x32x16_f16 with MT 32-row
// tiles of the chunk (rows past `rows` are padding, computed and discarded).
//
// B tile nt covers 32 weight rows = two 16-row panels.  For the 16-wide K
// slice t of a 128-wide chunk, lane L needs rows n = L % 32, columns
// 16t + 8(L / 32) + 0..7: in the device layout those are dword t / 2 of the
// 16-byte slot (n % 16) + 16 (L / 32) (t even) or (n % 16) + 16 (2 + L / 32)
// (t odd) of panel n / 16, so each lane loads two 16-byte slots per tile and
// step and every byte is used once.  The A fragment of slice t is the 16-byte
// unit 2t + L / 32 of row L % 32 in the staged tile.
template <bool GATEUP, int MT>
__device__ __forceinline__ void run_item(const FwdArgs &a, const ItemState &st, uint8_t (*s_a)[kChunkRows * kRowBytes],
                                         const int *s_ent, const float *s_w) {
    const int H = a.hidden, I = a.inter;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l31 = lane & 31, lh = lane >> 5;
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
    struct B32 {
        uint4 qe[2], qo[2];
        uint2 sc[2];
    };
    auto load_b = [&](int c, B32 &f) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const uint32_t cq = st.qoff[nt] + static_cast<uint32_t>(c) * kChunkBytes;
            f.qe[nt] = dev::bload<uint4>(st.brs, st.qv_even, cq);
            f.qo[nt] = dev::bload<uint4>(st.brs, st.qv_odd, cq);
            f.sc[nt] = dev::bload<uint2>(st.brs, st.sv, st.soff[nt] + static_cast<uint32_t>(c) * kScaleChunkBytes);
        }
    };

    floatx16 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;

    const uint32_t M0 = vconst(0x000F000Fu), M1 = vconst(0x00F000F0u), G = vconst(0x64006400u);

    B32 bn, bc;
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
        // A fragments are read one slice ahead so LDS latency overlaps the
        // MFMAs of the current slice.
        half8 av[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            av[mt] = *reinterpret_cast<const half8 *>(tile + lds_unit(mt * 32 + l31, lh));
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            half8 an[MT];
            if (t + 1 < 8) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    an[mt] = *reinterpret_cast<const half8 *>(tile + lds_unit(mt * 32 + l31, 2 * (t + 1) + lh));
            }
            half8 bf[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const uint4 &q = (t & 1) ? bc.qo[nt] : bc.qe[nt];
                const int s2 = t >> 1;
                const uint32_t w = s2 == 0 ? q.x : s2 == 1 ? q.y : s2 == 2 ? q.z : q.w;
                bf[nt] = dequant8(w, scale_pair(bc.sc[nt], s2), M0, M1, G);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[mt], bf[nt], acc[mt][nt], 0, 0, 0);
            if (t + 1 < 8) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) av[mt] = an[mt];
            }
        }
    }

    // Epilogue.  Lane holds D[m = 8(i / 4) + 4(L / 32) + i % 4][n = L % 32]
    // of each 32x32 tile.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = mt * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
            if (m < st.rows) {
                if (GATEUP) {
                    const float g = acc[mt][0][i], v = acc[mt][1][i];
                    const float hval = g / (1.0f + expf(-g)) * v;
                    const int col = st.nb * 128 + wave * 32 + l31;
                    a.h[static_cast<size_t>(st.row0 + m) * I + col] = static_cast<_Float16>(hval);
                } else {
                    const int entry = s_ent[m];
                    const float wgt = s_w[m];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        if (st.bvalid[nt]) {
                            const int col = st.nb * 256 + wave * 64 + nt * 32 + l31;
                            a.ys[static_cast<size_t>(entry) * H + col] = wgt * acc[mt][nt][i];
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
    __shared__ int s_ent[GATEUP ? 1 : kChunkRows];     // down: output entry and routing weight per row
    __shared__ float s_w[GATEUP ? 1 : kChunkRows];
    const int H = a.hidden, I = a.inter;
    const int K = GATEUP ? H : I;
    const int NB = GATEUP ? I / 128 : (H + 255) / 256;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l15 = lane & 15, l4 = lane >> 4;
    const int l31 = lane & 31, lh = lane >> 5;
    const int routed = a.n_tok * a.k;

    // Work items (chunk, N-block) are dealt to kGroupedQueues queues by
    // chunk (chunk c to queue c mod 8) and taken dynamically: workgroup b
    // draws from queue b mod 8, which on an 8-XCD part is the queue of its
    // XCD, so the N-blocks of a chunk (same activation rows) share an L2.
    // Items differ in cost (chunks of 1 to 128 rows); dynamic claiming keeps
    // every workgroup busy until its queue is empty.
    const int nq = gridDim.x >= kGroupedQueues ? kGroupedQueues : 1;
    const int q = blockIdx.x % nq;
    const int n_chunks = *a.n_chunks;
    const int q_items = (n_chunks > q ? (n_chunks - q + nq - 1) / nq : 0) * NB;
    int32_t *ticket = a.queues + q * kQueueStride;
    __shared__ int s_item;

    for (;;) {
        __syncthreads();       // every thread has read the previous s_item
        if (tid == 0) s_item = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int j = s_item;
        if (j >= q_items) break;
        const int item = (q + nq * (j / NB)) * NB + j % NB;
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
        // 32-row tiles: 1, 2 or 4 (padding rows are computed and discarded).
        const int mt = d.rows > 64 ? 4 : (d.rows > 32 ? 2 : 1);

        // This wave's two 32-row B tiles (two 16-row panels each), as
        // uniform offsets, and the per-lane slot offsets inside them.
        st.brs = dev::make_rsrc(blob, static_cast<uint32_t>(a.lay.total));
        const uint32_t pstep = static_cast<uint32_t>(st.C) * kChunkBytes;   // bytes per panel
        const uint32_t r16 = static_cast<uint32_t>(l31 & 15), hi = static_cast<uint32_t>(l31 >> 4);
        st.qv_even = hi * pstep + 16 * (r16 + 16 * static_cast<uint32_t>(lh));
        st.qv_odd = hi * pstep + 16 * (r16 + 16 * (2 + static_cast<uint32_t>(lh)));
        st.sv = hi * static_cast<uint32_t>(st.C) * kScaleChunkBytes + r16 * 8;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            int panel;
            size_t qs, ss;
            if (GATEUP) {
                panel = nb * 8 + wave * 2;          // gate (nt 0) or up (nt 1) rows of the same columns
                qs = nt == 0 ? a.lay.gate_q : a.lay.up_q;
                ss = nt == 0 ? a.lay.gate_s : a.lay.up_s;
                st.bvalid[nt] = true;
            } else {
                panel = nb * 16 + wave * 4 + nt * 2;
                qs = a.lay.down_q;
                ss = a.lay.down_s;
                st.bvalid[nt] = panel + 1 < H / kPanel;
                if (!st.bvalid[nt]) panel = 0;
            }
            st.qoff[nt] = static_cast<uint32_t>(qs + static_cast<size_t>(panel) * st.C * kChunkBytes);
            st.soff[nt] = static_cast<uint32_t>(ss + static_cast<size_t>(panel) * st.C * kScaleChunkBytes);
        }

        __syncthreads();   // previous item is done with s_tok and the A tiles
        for (int m = tid; m < kChunkRows; m += 256) {
            // Rows past `rows` repeat row 0: their results are discarded.
            const int mm = m < d.rows ? m : 0;
            const int r = d.row0 + mm;
            s_tok[m] = GATEUP ? (r < routed ? a.gather[r] / a.k : r - routed) : r;
            if (!GATEUP) {
                const int entry = r < routed ? a.gather[r] : r;
                s_ent[m] = entry;
                s_w[m] = r < routed ? a.topk_w[entry] : 1.0f;
            }
        }
        __syncthreads();
        // This wave stages 16-row groups wave, wave+4 of the first mt*32
        // rows: one copy16 per 4 rows, swizzled on the source side so that
        // lane L fills slot (L & 15) of row (L >> 4).
        const size_t arow = GATEUP ? static_cast<size_t>(H) : static_cast<size_t>(I);
        const int ng = 2 * mt;
        st.my_groups = ng > wave ? (ng - wave + 3) / 4 : 0;
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = (wave + 4 * g) * 16 + i * 4 + l4;
                const int q = l15 ^ (m & 15);
                st.src_off[g][i] = static_cast<uint32_t>(s_tok[m]) * static_cast<uint32_t>(arow) + 8 * q;
            }
        if (mt == 4) run_item<GATEUP, 4>(a, st, s_a, s_ent, s_w);
        else if (mt == 2) run_item<GATEUP, 2>(a, st, s_a, s_ent, s_w);
        else run_item<GATEUP, 1>(a, st, s_a, s_ent, s_w);
    }
    // The last workgroup out clears the queue counters for the next launch.
    if (dev::arrive_last(a.queues + kGroupedQueues * kQueueStride, gridDim.x) && tid < kGroupedQueues)
        dev::store_coherent(a.queues + tid * kQueueStride, 0);
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

int grid_for(int items, int slots) {
    int g = slots;
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
    launch(grouped_kernel<true>, grid_for(max_chunks * (a.inter / 128), 2 * n_cu), 256, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_grouped_down(const FwdArgs &a, int max_chunks, int n_cu, hipStream_t s) {
    launch(grouped_kernel<false>, grid_for(max_chunks * ((a.hidden + 255) / 256), 2 * n_cu), 256, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const FwdArgs &a, hipStream_t s) {
    const size_t n = static_cast<size_t>(a.n_tok) * (a.hidden / 4);
    if (n == 0) return hipSuccess;
    launch(combine_kernel, static_cast<unsigned>((n + 255) / 256), 256, 0, s, a);
    return hipGetLastError();
}

}  // namespace coli
