// grouped.hip -- batched expert FFNs as grouped GEMMs on MFMA, and the
// routing-weighted combine.
//
// When the union gives experts many tokens (large decode batches, prefill)
// the expert matmuls become dense contractions, [M_u x K] x [K x N] per
// union expert.  Work is a list of chunks (one expert, <= 160 rows; <= 32
// rows for calls of at most 64 tokens, where experts get a few rows each)
// crossed with N-blocks; a persistent grid walks that list (the N-blocks of a
// chunk, which share its activation rows, are queued on one XCD and its L2).
//
// Per item a 256-thread workgroup (two per CU) walks the reduction axis in
// 64-column steps through a ring of three LDS stages: the chunk's fp16
// activation rows of step c + 2 are copied straight from global memory into
// LDS (global_load_lds; XOR-swizzled 16-byte units, conflict-free for the
// fragment reads) and each wave's int4 weight fragments of step c + 2 are
// loaded into registers (buffer loads, already in B-fragment order of
// v_mfma_f32_32x32x16_f16) while step c is multiplied.  With 32-row chunks
// (four workgroups per CU) a step is a whole 128-column chunk and the ring
// has two stages: the weight slots are then read whole, by one load each
// (the 64-column step reads each slot in two halves a step apart; measured at
// 64 tokens, 128-column steps take both GEMMs 7-9% faster).  Inside a step the LDS
// reads and the dequantisation of the next 16-column slice are interleaved
// between the MFMAs of the current one.  Each weight dword becomes eight fp16
// weights: q = (1024 + u) - 1032 (exact) times the group's fp16 scale (one
// rounding), so a fragment lies inside one scale group (32 or 64 wide) and
// the MFMA accumulates in fp32.  A chunk that would end in a 32-row tile of
// 16 rows or fewer ends in a 16-row tile on v_mfma_f32_16x16x32_f16 instead,
// fed by the same fragments regrouped across lanes; rows past a chunk's end
// read a zeroed row.
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

// The K loop of 160-row chunks (two workgroups per CU) advances 64 reduction
// columns per step through a ring of three LDS stages: the activation copy
// and the weight loads of step c + 2 are issued while step c is multiplied.
constexpr int kStepK = 64;
constexpr int kStageRowBytes = kStepK * 2;                  // one staged row: 64 fp16
constexpr int kStages = 3;
constexpr int kAhead = 2;                                   // steps issued ahead
template <int CR>
constexpr int stage_bytes() { return CR * kStageRowBytes; }  // 20 KB
// The 32-row instance steps a whole 128-column chunk at a time (each 16-byte
// weight slot is then read by one load), through a ring of two stages.
constexpr int kSmallRowBytes = kChunkK * 2;                  // one staged row: 128 fp16
constexpr int kSmallStages = 2;
constexpr int kSmallAhead = kSmallStages - 1;
constexpr int kSmallStageBytes = kSmallChunkRows * kSmallRowBytes;   // 8 KB
template <int CR>
constexpr int ring_bytes() { return CR == kSmallChunkRows ? kSmallStages * kSmallStageBytes : kStages * stage_bytes<CR>(); }
template <int CR>
constexpr int blocks_per_cu() { return CR == kSmallChunkRows ? 4 : 2; }

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

// Byte offset of logical 16-byte unit q (0..7) of staged row m.  A fragment
// read has 16 consecutive lanes read 16 bytes each from rows m..m+15 at the
// same logical unit; with 64 four-byte banks a 128-byte row spans half of
// them, so the physical unit is q ^ ((m >> 1) & 7): the 16 rows then cover
// all 64 banks once.
__device__ __forceinline__ int lds_swz(int m) { return (m >> 1) & 7; }
__device__ __forceinline__ int lds_unit(int m, int q) {
    return m * kStageRowBytes + ((q ^ lds_swz(m)) << 4);
}
// The same for the 256-byte rows of the 32-row instance: a row spans all 64
// banks, and physical unit q ^ (m & 15) spreads 16 rows over them.
__device__ __forceinline__ int lds_unit256(int m, int q) { return m * kSmallRowBytes + ((q ^ (m & 15)) << 4); }

// Scheduling groups for one slice: N times (one MFMA, on odd turns one LDS
// read, V VALU instructions), so the reads and dequantisation of the next
// slice issue between the MFMAs of this one.
template <int I, int N, int V>
__device__ __forceinline__ void interleave() {
    if constexpr (I < N) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (I & 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
        interleave<I + 1, N, V>();
    }
}

// State of one work item (chunk x N-block) shared by its K loop and
// epilogue.
struct ItemState {
    const _Float16 *asrc;
    uint32_t src_off[5];         // this wave's copy j (< MT): lane's source (fp16 elements, column 0)
    dev::rsrc_t brs;             // weight blob
    uint32_t qv_even, qv_odd, sv; // per-lane byte offsets of the B slots and scales
    uint32_t qoff[2], soff[2];   // this wave's two 32-row B tiles (uniform)
    bool bvalid[2];
    int row0, rows, nb, C2;      // C2 = K steps (64 or 128 columns each)
};

// Stores 32-row tile mt of an item: lane L holds D[m = 8(i / 4) + 4(L / 32)
// + i % 4][n = L % 32] of the tile's two 32-column B tiles.  gate/up: SwiGLU
// of the gate (B tile 0) and up (1) values into h as fp16; down: times the
// row's routing weight into its entry's output row.  Padding rows
// (m >= rows) store into the discard row, so no store is predicated.
template <bool GATEUP>
__device__ __forceinline__ void store_tile(const FwdArgs &a, const ItemState &st, const floatx16 (&acc)[2], int mt,
                                           const int *s_ent, const float *s_w, bool &hbad) {
    const int H = a.hidden, I = a.inter;
    const int wave = dev::wave_id(), lane = threadIdx.x & 63;
    const int l31 = lane & 31, lh = lane >> 5;
    if (GATEUP) {
        const int col = st.nb * 128 + wave * 32 + l31;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = mt * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
            const int r = m < st.rows ? st.row0 + m : a.discard_row;
            const _Float16 hh = static_cast<_Float16>(dev::swiglu(acc[0][i], acc[1][i]));
            hbad = hbad || dev::half_nonfinite(hh);
            a.h[static_cast<size_t>(r) * I + col] = hh;
        }
    } else {
        // The tile's output entries (the discard row for padding) and
        // routing weights, read from LDS in one batch ahead of the stores.
        const int col = st.nb * 256 + wave * 64 + l31;
#pragma unroll
        for (int i0 = 0; i0 < 16; i0 += 8) {
            int ent[8];
            float wgt[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int m = mt * 32 + 8 * ((i0 + i) >> 2) + 4 * lh + (i & 3);
                ent[i] = s_ent[m];
                wgt[i] = s_w[m];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float *yrow = a.ys + static_cast<size_t>(ent[i]) * H + col;
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    if (st.bvalid[nt]) yrow[nt * 32] = wgt[i] * acc[nt][i0 + i];
            }
        }
    }
}

// K loop and epilogue of one item on v_mfma_f32_32x32x16_f16 with MT 32-row
// tiles of the chunk, and with TAIL a 16-row tile after them (rows 32 MT ..
// 32 MT + 15) on v_mfma_f32_16x16x32_f16 (rows past `rows` are padding,
// computed and discarded).
//
// B tile nt covers 32 weight rows = two 16-row panels.  For the 16-wide K
// slice T of a 128-wide chunk, lane L needs rows n = L % 32, columns
// 16T + 8(L / 32) + 0..7: in the device layout those are dword T / 2 of the
// 16-byte slot (n % 16) + 16 (L / 32) (T even) or (n % 16) + 16 (2 + L / 32)
// (T odd) of panel n / 16, so a 64-column step (half h of a chunk) takes the
// 8 bytes at 8h of each of the two slots, plus the dword of its two scales.
// The A fragment of slice t of a step is the 16-byte unit 2t + L / 32 of row
// L % 32 of the staged tile.
//
// Step c waits for its own copies with an explicit count: after them this
// wave has issued exactly the B loads of step c (6) and the copies (MT, plus
// one for the tail tile's rows) and B loads (6) of steps c + 1 .. c + kAhead
// - 1 (other memory operations only make that wait stricter).  Lookahead past the last step repeats the last
// step's addresses (never used), so that count holds at every step; the loop
// ends with a full wait before the stages are reused.
template <bool GATEUP, int MT, int GS, int CR, bool TAIL>
__device__ __forceinline__ void run_item(const FwdArgs &a, const ItemState &st, const uint8_t *s_a,
                                         uint32_t sa_lds, const int *s_ent, const float *s_w) {
    const int H = a.hidden, I = a.inter;
    const int wave = dev::wave_id(), lane = threadIdx.x & 63;
    const int l31 = lane & 31, lh = lane >> 5;
    constexpr int kCopies = MT + (TAIL ? 1 : 0);   // 8-row copies per wave and step
    struct B64 {
        uint2 qe[2], qo[2];
        uint32_t sc[2];
    };
    auto issue = [&](int c, B64 &f) {
        const int cc = min(c, st.C2 - 1);
        const uint32_t dst = sa_lds + static_cast<uint32_t>(c % kStages) * stage_bytes<CR>();
#pragma unroll
        for (int j = 0; j < kCopies; ++j)
            dev::copy16_to_lds(st.asrc + st.src_off[j] + cc * kStepK,
                          dst + static_cast<uint32_t>(8 * (wave + 4 * j) * kStageRowBytes));
        asm volatile("" ::: "memory");
        const uint32_t ch = static_cast<uint32_t>(cc >> 1), h = static_cast<uint32_t>(cc & 1);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const uint32_t cq = st.qoff[nt] + ch * kChunkBytes + 8 * h;
            f.qe[nt] = dev::bload<uint2>(st.brs, st.qv_even, cq);
            f.qo[nt] = dev::bload<uint2>(st.brs, st.qv_odd, cq);
            // Group size 32: the step's two scales (groups 2h, 2h+1 of the
            // chunk); 64: the chunk's two, of which group h is the step's.
            f.sc[nt] = dev::bload<uint32_t>(st.brs, st.sv,
                                            st.soff[nt] + ch * scale_chunk_bytes<GS>() + (GS == 32 ? 4 * h : 0));
        }
        asm volatile("" ::: "memory");
    };

    floatx16 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;
    // The 16-row tail tile (rows 32 MT .. 32 MT + 15): per B tile nt, its two
    // 16-column halves hi as 16x16 accumulators.
    floatx4 acct[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) acct[nt][hi] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    const uint32_t M0 = vconst(0x000F000Fu), M1 = vconst(0x00F000F0u), G = vconst(0x64006400u);

    // B fragment of slice t (0..3) of step c: dword t / 2 of the even or odd
    // slot half, times the scale of its group (t / 2 of the step's pair for
    // group size 32; half c & 1 of the chunk's pair for 64).
    auto bfrag = [&](const B64 &f, int t, int nt, int c) {
        const uint2 &q = (t & 1) ? f.qo[nt] : f.qe[nt];
        const uint32_t w = (t >> 1) ? q.y : q.x;
        const int sel = GS == 32 ? (t >> 1) : (c & 1);
        const _Float16 sh = __builtin_bit_cast(_Float16, static_cast<uint16_t>(f.sc[nt] >> (16 * sel)));
        return dequant8(w, half2v{sh, sh}, M0, M1, G);
    };
    // Software pipeline over the four slices of a step: the A fragments and
    // dequantised B fragments of slice t + 1 are produced before the MFMAs of
    // slice t are issued (the scheduling barriers keep that order), so LDS
    // latency and dequantisation overlap the matrix pipe.
    auto compute = [&](int c, const B64 &f) {
        if (c >= st.C2) return;
        const uint8_t *tile = s_a + (c % kStages) * stage_bytes<CR>();
        half8 av[MT], bc[2], bprev[2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            av[mt] = *reinterpret_cast<const half8 *>(tile + lds_unit(mt * 32 + l31, lh));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) bc[nt] = bfrag(f, 0, nt, c);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            half8 an[MT], bn[2];
            if (t + 1 < 4) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    an[mt] = *reinterpret_cast<const half8 *>(tile + lds_unit(mt * 32 + l31, 2 * (t + 1) + lh));
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) bn[nt] = bfrag(f, t + 1, nt, c);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[mt], bc[nt], acc[mt][nt], 0, 0, 0);
            // Interleave: after each MFMA of slice t, a share of the LDS reads
            // and dequantisation of slice t + 1, which then execute while the
            // MFMA occupies the matrix pipe.
            interleave<0, 2 * MT, 26 / (2 * MT) + 1>();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (TAIL) {
                if (t & 1) {
                    // 32-column slice t / 2 on v_mfma_f32_16x16x32_f16.  Its B
                    // fragments are the 32x32x16 fragments of slices t - 1 and
                    // t with their 16-lane rows regrouped: (row r of slice
                    // t - 1, ...) -> [X0 X2 Y0 Y2] for columns 0-15 and
                    // [X1 X3 Y1 Y3] for 16-31, two lane swaps per dword.
                    const half8 at = *reinterpret_cast<const half8 *>(
                        tile + lds_unit(MT * 32 + (lane & 15), 4 * (t >> 1) + (lane >> 4)));
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const uint4 x = __builtin_bit_cast(uint4, bprev[nt]);
                        const uint4 y = __builtin_bit_cast(uint4, bc[nt]);
                        const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
                        uint32_t f0[4], f1[4];
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const auto p32 = __builtin_amdgcn_permlane32_swap(xs[d], ys[d], false, false);
                            const auto p16 = __builtin_amdgcn_permlane16_swap(p32[0], p32[1], false, false);
                            f0[d] = p16[0];
                            f1[d] = p16[1];
                        }
                        const half8 h0 = __builtin_bit_cast(half8, uint4{f0[0], f0[1], f0[2], f0[3]});
                        const half8 h1 = __builtin_bit_cast(half8, uint4{f1[0], f1[1], f1[2], f1[3]});
                        acct[nt][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(at, h0, acct[nt][0], 0, 0, 0);
                        acct[nt][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(at, h1, acct[nt][1], 0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) bprev[nt] = bc[nt];
                }
            }
            if (t + 1 < 4) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) av[mt] = an[mt];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) bc[nt] = bn[nt];
            }
        }
    };
    auto step = [&](int c, const B64 &cur, B64 &ahead) {
        // A plain barrier, not __syncthreads: its release fence would wait
        // for every load in flight, which is the lookahead itself.  LDS reads
        // of the previous step are complete (lgkmcnt) before any wave passes.
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(6 + (kAhead - 1) * (kCopies + 6)) : "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(c + kAhead, ahead);
        compute(c, cur);
    };

    B64 b[kStages];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) issue(i, b[i]);
    for (int c = 0; c < st.C2; c += kStages) {
#pragma unroll
        for (int i = 0; i < kStages; ++i) step(c + i, b[i], b[(i + kAhead) % kStages]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Epilogue (see store_tile); padding rows store into the discard row.
    bool hbad = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) store_tile<GATEUP>(a, st, acc[mt], mt, s_ent, s_w, hbad);
    if constexpr (TAIL) {
        // The 16x16 tiles: lane L holds D[m = 32 MT + 4 (L / 16) + i][n = L % 16]
        // of column half hi of B tile nt.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = MT * 32 + 4 * (lane >> 4) + i;
            if (GATEUP) {
                const int r = m < st.rows ? st.row0 + m : a.discard_row;
#pragma unroll
                for (int hi = 0; hi < 2; ++hi) {
                    const int col = st.nb * 128 + wave * 32 + 16 * hi + (lane & 15);
                    const _Float16 hh = static_cast<_Float16>(dev::swiglu(acct[0][hi][i], acct[1][hi][i]));
                    hbad = hbad || dev::half_nonfinite(hh);
                    a.h[static_cast<size_t>(r) * I + col] = hh;
                }
            } else {
                float *yrow = a.ys + static_cast<size_t>(s_ent[m]) * H + st.nb * 256 + wave * 64 + (lane & 15);
                const float wgt = s_w[m];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int hi = 0; hi < 2; ++hi)
                        if (st.bvalid[nt]) yrow[nt * 32 + 16 * hi] = wgt * acct[nt][hi][i];
            }
        }
    }
    if (GATEUP) dev::flag_if(hbad, a.err, kErrHiddenRange);
}

// K loop and epilogue of an item of the 32-row instance: one 32-row tile,
// 128-column steps (eight 16-column slices each).  Slice T of chunk c takes
// dword T / 2 of the even (T even) or odd slot of its lane (the mapping of
// run_item) and the scale of group T / 2 (size 32) or T / 4 (size 64); a step
// loads each lane's two 16-byte slots whole, and its scales (four or two per
// row).  Each weight and scale byte is then read once, by the load that
// fetches it, so those loads are non-temporal (as the GEMV streams): the
// weight stream does not evict the data other kernels of the call reuse.
// Step c waits for its copies with an explicit count: after them this wave
// has issued the B loads of step c (6) and the copies (2) and B loads (6) of
// steps c + 1 .. c + kSmallAhead - 1.
template <bool GATEUP, int GS>
__device__ __forceinline__ void run_item_small(const FwdArgs &a, const ItemState &st, const uint8_t *s_a,
                                               uint32_t sa_lds, const int *s_ent, const float *s_w) {
    const int wave = dev::wave_id(), lane = threadIdx.x & 63;
    const int l31 = lane & 31, lh = lane >> 5;
    struct B128 {
        uint4 qe[2], qo[2];
        uint32_t sc[2][GS == 32 ? 2 : 1];
    };
    auto issue = [&](int c, B128 &f) {
        const int cc = min(c, st.C2 - 1);
        const uint32_t dst = sa_lds + static_cast<uint32_t>(c % kSmallStages) * kSmallStageBytes;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dev::copy16_to_lds(st.asrc + st.src_off[j] + cc * kChunkK,
                               dst + static_cast<uint32_t>(4 * (wave + 4 * j) * kSmallRowBytes));
        asm volatile("" ::: "memory");
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const uint32_t cq = st.qoff[nt] + static_cast<uint32_t>(cc) * kChunkBytes;
            f.qe[nt] = dev::bload<uint4, dev::kLoadStream>(st.brs, st.qv_even, cq);
            f.qo[nt] = dev::bload<uint4, dev::kLoadStream>(st.brs, st.qv_odd, cq);
            const uint32_t cs = st.soff[nt] + static_cast<uint32_t>(cc) * scale_chunk_bytes<GS>();
            if constexpr (GS == 32) {
                const uint2 v = dev::bload<uint2, dev::kLoadStream>(st.brs, st.sv, cs);
                f.sc[nt][0] = v.x;
                f.sc[nt][1] = v.y;
            } else {
                f.sc[nt][0] = dev::bload<uint32_t, dev::kLoadStream>(st.brs, st.sv, cs);
            }
        }
        asm volatile("" ::: "memory");
    };

    floatx16 acc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nt][i] = 0.0f;
    const uint32_t M0 = vconst(0x000F000Fu), M1 = vconst(0x00F000F0u), G = vconst(0x64006400u);
    auto bfrag = [&](const B128 &f, int T, int nt) {
        const uint4 &q = (T & 1) ? f.qo[nt] : f.qe[nt];
        const int d = T >> 1;
        const uint32_t w = d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w;
        const uint32_t sw = GS == 32 ? f.sc[nt][(T >> 2) & (GS == 32 ? 1 : 0)] : f.sc[nt][0];
        const int sel = GS == 32 ? ((T >> 1) & 1) : (T >> 2);
        const _Float16 sh = __builtin_bit_cast(_Float16, static_cast<uint16_t>(sw >> (16 * sel)));
        return dequant8(w, half2v{sh, sh}, M0, M1, G);
    };
    // The software pipeline of run_item over eight slices.
    auto compute = [&](int c, const B128 &f) {
        if (c >= st.C2) return;
        const uint8_t *tile = s_a + (c % kSmallStages) * kSmallStageBytes;
        half8 av = *reinterpret_cast<const half8 *>(tile + lds_unit256(l31, lh)), bc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) bc[nt] = bfrag(f, 0, nt);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            half8 an, bn[2];
            if (t + 1 < 8) {
                an = *reinterpret_cast<const half8 *>(tile + lds_unit256(l31, 2 * (t + 1) + lh));
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) bn[nt] = bfrag(f, t + 1, nt);
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bc[nt], acc[nt], 0, 0, 0);
            interleave<0, 2, 14>();
            __builtin_amdgcn_sched_barrier(0);
            if (t + 1 < 8) {
                av = an;
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) bc[nt] = bn[nt];
            }
        }
    };
    auto step = [&](int c, const B128 &cur, B128 &ahead) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(6 + (kSmallAhead - 1) * 8) : "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(c + kSmallAhead, ahead);
        compute(c, cur);
    };
    B128 b[kSmallStages];
#pragma unroll
    for (int i = 0; i < kSmallAhead; ++i) issue(i, b[i]);
    for (int c = 0; c < st.C2; c += kSmallStages) {
#pragma unroll
        for (int i = 0; i < kSmallStages; ++i) step(c + i, b[i], b[(i + kSmallAhead) % kSmallStages]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    bool hbad = false;
    store_tile<GATEUP>(a, st, acc, 0, s_ent, s_w, hbad);
    if (GATEUP) dev::flag_if(hbad, a.err, kErrHiddenRange);
}

template <bool GATEUP, int GS, int CR>
__global__ __launch_bounds__(256, blocks_per_cu<CR>()) void grouped_kernel(FwdArgs a) {
    // Ring of A stages, CR rows x kStepK fp16 each.
    __shared__ __align__(16) uint8_t s_a[ring_bytes<CR>()];
    // LDS byte address of s_a (for the copies' M0).
    const uint32_t sa_lds = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t *)(&s_a[0])));
    __shared__ int s_tok[CR];
    __shared__ int s_ent[GATEUP ? 1 : CR];     // down: output entry and routing weight per row
    __shared__ float s_w[GATEUP ? 1 : CR];
    const int H = a.hidden, I = a.inter;
    const int K = GATEUP ? H : I;
    const int NB = GATEUP ? I / 128 : (H + 255) / 256;
    const int tid = threadIdx.x, wave = dev::wave_id(), lane = tid & 63;
    const int l31 = lane & 31, lh = lane >> 5;
    const int routed = a.n_tok * a.k;

    // Work items (chunk, N-block) are dealt to kGroupedQueues queues by
    // chunk (chunk c to queue c mod 8) and taken dynamically: workgroup b
    // draws from queue b mod 8, which on an 8-XCD part is the queue of its
    // XCD, so the N-blocks of a chunk (same activation rows) share an L2.
    // Items differ in cost (chunks of 1 to 160 rows) and the queues in total
    // work; dynamic claiming keeps every workgroup busy until its queue is
    // empty, and then it takes items from the other queues in turn.
    const int nq = gridDim.x >= kGroupedQueues ? kGroupedQueues : 1;
    const int n_chunks = *a.n_chunks;
    int qq = static_cast<int>(blockIdx.x) % nq, tried = 0;
    __shared__ int s_item;

    for (;;) {
        __syncthreads();       // every thread has read the previous s_item
        if (tid == 0)
            s_item = __hip_atomic_fetch_add(a.queues + qq * kQueueStride, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        // Uniform across the workgroup: everything derived from it (chunk,
        // blob, descriptor, offsets) then lives in scalar registers.
        const int j = __builtin_amdgcn_readfirstlane(s_item);
        const int q_items = (n_chunks > qq ? (n_chunks - qq + nq - 1) / nq : 0) * NB;
        if (j >= q_items) {
            if (++tried >= nq) break;
            qq = qq + 1 < nq ? qq + 1 : 0;   // this queue is empty: the next one
            continue;
        }
        const int item = (qq + nq * (j / NB)) * NB + j % NB;
        const int chunk = item / NB, nb = item % NB;
        // The chunk descriptor and the blob pointer are read by every lane
        // from one address; readfirstlane makes them scalar, so the weight
        // descriptor built from them is known to be uniform (a per-lane
        // descriptor would turn every buffer load into a loop over lanes).
        ChunkDesc d = a.chunks[chunk];
        d.expert = __builtin_amdgcn_readfirstlane(d.expert);
        d.row0 = __builtin_amdgcn_readfirstlane(d.row0);
        d.rows = __builtin_amdgcn_readfirstlane(d.rows);
        const uint64_t braw = reinterpret_cast<uint64_t>(a.table[d.expert]);
        const uint64_t bl = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(braw)));
        const uint64_t bh = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(braw >> 32)));
        const uint8_t *blob = reinterpret_cast<const uint8_t *>(bl | (bh << 32));
        if (!blob) continue;
        ItemState st;
        st.asrc = GATEUP ? a.xh : a.h;
        st.row0 = d.row0;
        st.rows = d.rows;
        st.nb = nb;
        st.C2 = CR == kSmallChunkRows ? K / kChunkK : K / kStepK;
        const int C = K / kChunkK;
        // 32-row tiles: 1 to CR / 32 (padding rows are computed and discarded).
        const int mt = (d.rows + 31) / 32;

        // This wave's two 32-row B tiles (two 16-row panels each), as
        // uniform offsets, and the per-lane slot offsets inside them.
        st.brs = dev::make_rsrc(blob, static_cast<uint32_t>(a.lay.total));
        const uint32_t pstep = static_cast<uint32_t>(C) * kChunkBytes;   // bytes per panel
        const uint32_t r16 = static_cast<uint32_t>(l31 & 15), hi = static_cast<uint32_t>(l31 >> 4);
        st.qv_even = hi * pstep + 16 * (r16 + 16 * static_cast<uint32_t>(lh));
        st.qv_odd = hi * pstep + 16 * (r16 + 16 * (2 + static_cast<uint32_t>(lh)));
        st.sv = hi * static_cast<uint32_t>(C) * scale_chunk_bytes<GS>() + r16 * scale_row_bytes<GS>();
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
            st.qoff[nt] = static_cast<uint32_t>(qs + static_cast<size_t>(panel) * C * kChunkBytes);
            st.soff[nt] = static_cast<uint32_t>(ss + static_cast<size_t>(panel) * C * scale_chunk_bytes<GS>());
        }

        __syncthreads();   // previous item is done with s_tok and the A tiles
        for (int m = tid; m < CR; m += 256) {
            // Rows past `rows` read a row of zeros (their results are
            // discarded): zero operands draw less power in the matrix cores,
            // which run at a power limit (measured: B = 64 GEMMs 5-7% faster
            // than with a repeated real row).
            const int mm = m < d.rows ? m : 0;
            const int r = d.row0 + mm;
            s_tok[m] = m >= d.rows ? (GATEUP ? a.zero_row_x : a.zero_row_h)
                                   : (GATEUP ? (r < routed ? a.gather[r] / a.k : r - routed) : r);
            if (!GATEUP) {
                const int entry = r < routed ? a.gather[r] : r;
                s_ent[m] = m < d.rows ? entry : a.discard_row;
                s_w[m] = r < routed ? a.topk_w[entry] : 1.0f;
            }
        }
        __syncthreads();
        // Copy j of this wave stages rows 8 (wave + 4j) .. +7 (MT copies per
        // wave cover the first mt*32 rows): lane L fills LDS unit L & 7 of row
        // m = 8 (wave + 4j) + L / 8 with logical unit (L & 7) ^ lds_swz(m).
        const size_t arow = GATEUP ? static_cast<size_t>(H) : static_cast<size_t>(I);
        if constexpr (CR == kSmallChunkRows) {
            // 256-byte rows: copy j of this wave stages rows 4 (wave + 4j) ..
            // +3; lane L fills unit L & 15 of row 4 (wave + 4j) + L / 16 with
            // logical unit (L & 15) ^ (m & 15).
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int m = 4 * (wave + 4 * j) + (lane >> 4);
                const int q = (lane & 15) ^ (m & 15);
                st.src_off[j] = static_cast<uint32_t>(s_tok[m]) * static_cast<uint32_t>(arow) + 8 * q;
            }
            run_item_small<GATEUP, GS>(a, st, s_a, sa_lds, s_ent, s_w);
        } else {
#pragma unroll
            for (int j = 0; j < CR / 32; ++j) {
                const int m = 8 * (wave + 4 * j) + (lane >> 3);
                const int q = (lane & 7) ^ lds_swz(m);
                st.src_off[j] = static_cast<uint32_t>(s_tok[m]) * static_cast<uint32_t>(arow) + 8 * q;
            }
            if (mt >= 2 && d.rows - 32 * (mt - 1) <= 16) {
                // The last tile would hold 16 rows or fewer: a 16-row tile on
                // v_mfma_f32_16x16x32_f16 instead of a 32-row one (half the MFMA
                // work of that tile).
                switch (mt) {
                    case 5: run_item<GATEUP, 4, GS, CR, true>(a, st, s_a, sa_lds, s_ent, s_w); break;
                    case 4: run_item<GATEUP, 3, GS, CR, true>(a, st, s_a, sa_lds, s_ent, s_w); break;
                    case 3: run_item<GATEUP, 2, GS, CR, true>(a, st, s_a, sa_lds, s_ent, s_w); break;
                    default: run_item<GATEUP, 1, GS, CR, true>(a, st, s_a, sa_lds, s_ent, s_w); break;
                }
            } else {
                switch (mt) {
                    case 5: run_item<GATEUP, 5, GS, CR, false>(a, st, s_a, sa_lds, s_ent, s_w); break;
                    case 4: run_item<GATEUP, 4, GS, CR, false>(a, st, s_a, sa_lds, s_ent, s_w); break;
                    case 3: run_item<GATEUP, 3, GS, CR, false>(a, st, s_a, sa_lds, s_ent, s_w); break;
                    case 2: run_item<GATEUP, 2, GS, CR, false>(a, st, s_a, sa_lds, s_ent, s_w); break;
                    default: run_item<GATEUP, 1, GS, CR, false>(a, st, s_a, sa_lds, s_ent, s_w); break;
                }
            }
        }
    }
    // The last workgroup out clears the queue counters for the next launch.
    if (dev::arrive_last(a.queues + kGroupedQueues * kQueueStride, gridDim.x) && tid < kGroupedQueues)
        dev::store_coherent(a.queues + tid * kQueueStride, 0);
}

// fp16 copy of the activations (the A operand of the gate/up GEMM); values
// outside the fp16 range set a device error flag.
__global__ __launch_bounds__(256) void to_half_kernel(const void *x, int act_bf16, size_t n8, _Float16 *xh,
                                                      int32_t *err) {
    dev::to_half8(x, act_bf16, static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x, n8, xh, err);
}

// The per-entry rows are read exactly once, each by the instruction that
// fetches it: non-temporal loads (combine at 4096 tokens 188 -> 154 us).
__global__ __launch_bounds__(256) void combine_kernel(FwdArgs a) {
    const int H4 = a.hidden / 4;
    const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<size_t>(a.n_tok) * H4) return;
    const int t = static_cast<int>(idx / H4), n4 = static_cast<int>(idx % H4);
    const floatx4 *ys = reinterpret_cast<const floatx4 *>(a.ys);
    floatx4 acc = __builtin_nontemporal_load(ys + static_cast<size_t>(t * a.k) * H4 + n4);
    for (int j = 1; j < a.k; ++j) acc = acc + __builtin_nontemporal_load(ys + static_cast<size_t>(t * a.k + j) * H4 + n4);
    if (a.has_shared) acc = acc + __builtin_nontemporal_load(ys + static_cast<size_t>(a.n_tok * a.k + t) * H4 + n4);
    reinterpret_cast<floatx4 *>(a.y)[idx] = acc;
}

int grid_for(int items, int slots) {
    int g = slots;
    if (items < g) g = items;
    if (g >= 8) g &= ~7;
    return g < 1 ? 1 : g;
}

template <bool GATEUP, int CR>
void launch_grouped_as(const FwdArgs &a, int items, int n_cu, hipStream_t s) {
    const unsigned grid = grid_for(items, blocks_per_cu<CR>() * n_cu);
    if (a.lay.group == 64) launch(grouped_kernel<GATEUP, 64, CR>, grid, 256, 0, s, a);
    else launch(grouped_kernel<GATEUP, 32, CR>, grid, 256, 0, s, a);
}

template <bool GATEUP>
hipError_t launch_grouped(const FwdArgs &a, int max_chunks, int n_cu, hipStream_t s) {
    if (a.lay.bits != 4) return hipErrorInvalidValue;      // the MFMA fragments are int4 only
    const int items = max_chunks * (GATEUP ? a.inter / 128 : (a.hidden + 255) / 256);
    if (a.chunk_rows == kSmallChunkRows) launch_grouped_as<GATEUP, kSmallChunkRows>(a, items, n_cu, s);
    else if (a.chunk_rows == kChunkRows) launch_grouped_as<GATEUP, kChunkRows>(a, items, n_cu, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_to_half(const FwdArgs &a, hipStream_t s) {
    const size_t n8 = static_cast<size_t>(a.n_tok) * a.hidden / 8;
    if (n8 == 0) return hipSuccess;
    launch(to_half_kernel, static_cast<unsigned>((n8 + 255) / 256), 256, 0, s, a.x, a.act_bf16, n8, a.xh, a.err);
    return hipGetLastError();
}

hipError_t launch_grouped_gateup(const FwdArgs &a, int max_chunks, int n_cu, hipStream_t s) {
    return launch_grouped<true>(a, max_chunks, n_cu, s);
}

hipError_t launch_grouped_down(const FwdArgs &a, int max_chunks, int n_cu, hipStream_t s) {
    return launch_grouped<false>(a, max_chunks, n_cu, s);
}

hipError_t launch_combine(const FwdArgs &a, hipStream_t s) {
    const size_t n = static_cast<size_t>(a.n_tok) * (a.hidden / 4);
    if (n == 0) return hipSuccess;
    launch(combine_kernel, static_cast<unsigned>((n + 255) / 256), 256, 0, s, a);
    return hipGetLastError();
}

}  // namespace coli
