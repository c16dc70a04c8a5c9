// internal.h -- shared declarations of the HIP library (not part of the ABI).
//
// Device layout of one expert (written once by coli_expert_place):
//   The blob keeps the section offsets of the ABI blob (gate_q, up_q, down_q,
//   gate_s, up_s, down_s), but each [R x K] int4 matrix is re-tiled so that
//   one 16-byte load per lane of a 64-lane wave fetches a 16-row x 128-column
//   block (1 KB, a "chunk"):
//     chunk (p, c) of rows 16p..16p+15, columns 128c..128c+127 sits at byte
//     (p * K/128 + c) * 1024; lane L owns bytes L*16 .. L*16+15; dword s
//     (0..3) of that lane holds row 16p + (L & 15), columns
//     k0 = 128c + 32s + 8(L >> 4) .. k0+7.
//   That is exactly the B-operand fragment of v_mfma_f32_16x16x32_f16 for
//   k-step (c, s), and each dword is one 32-element scale group's 8-wide slice.
//   Inside a dword, column k0+i is stored as u = q + 8 (0..15) in nibble slot
//   i/2 (i even) or 4 + i/2 (i odd), so ((w >> 4j) & 0x000F000F) puts columns
//   k0+2j and k0+2j+1 in the low and high 16-bit halves: OR-ing an fp16
//   (0x6400 -> 1024 + u) or bf16 (0x4300 -> 128 + u) exponent turns each
//   half into an exact small integer.
//   Scales: chunk (p, c) has 16 * 128/G fp16 at (p * K/128 + c) times that
//   size in the scale section, [16 rows][128/G groups]: for group size
//   G = 32, 128 bytes holding groups 4c .. 4c+3 of each row; for G = 64,
//   64 bytes holding groups 2c, 2c+1.  Dword s of a lane's weight slot
//   (columns 32s + ...) takes group s (G = 32) or s / 2 (G = 64) of the
//   chunk.
//   Int8 experts (8 bits per weight): the same 1 KB chunks hold 16 rows x 64
//   columns, chunk (p, c) at (p * K/64 + c) * 1024; dword s of lane L holds
//   row 16p + (L & 15), columns k0 = 64c + 32(s >> 1) + 8(L >> 4) + 4(s & 1)
//   .. k0+3, stored as u = q + 128 in the byte order k0, k0+2, k0+1, k0+3, so
//   (w & 0x00FF00FF) | 0x64006400 makes the fp16 pair (1024 + u) of columns
//   k0, k0+1 and the same on w >> 8 that of k0+2, k0+3.  Scales: [16 rows]
//   [64/G] fp16 per chunk.  Int8 experts run on the GEMV kernels only.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

namespace coli {

constexpr int kChunkK = 128;        // reduction elements per 1 KB chunk
constexpr int kPanel = 16;          // matrix rows per chunk
constexpr int kChunkBytes = 1024;

// Reduction elements per fp16 scale: 32, or 64 (the container of the README's
// "Scarica il modello" section); bits per weight: 4, or 8 (the int8 the same
// section requires for the MTP head).
constexpr bool group_supported(int g) { return g == 32 || g == 64; }
constexpr bool bits_supported(int b) { return b == 4 || b == 8; }
// Bytes of one chunk's scales, and of one row's share of them.
template <int G>
constexpr int scale_chunk_bytes() { return kPanel * (kChunkK / G) * 2; }
template <int G>
constexpr int scale_row_bytes() { return (kChunkK / G) * 2; }
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kChunkRows = 160;     // rows per grouped work chunk: five 32-row MFMA tiles
// Calls of at most kSmallChunkMaxTok tokens cut chunks at one tile (most
// experts then have a few rows each): the grouped kernel instance for them
// needs a fifth of the LDS and registers, so twice as many workgroups fit.
constexpr int kSmallChunkRows = 32;
constexpr int kSmallChunkMaxTok = 64;
inline int chunk_rows_for(int n_tok) { return n_tok <= kSmallChunkMaxTok ? kSmallChunkRows : kChunkRows; }

struct BlobLayout {
    size_t gate_q, up_q, down_q, gate_s, up_s, down_s, total;
    int group;   // reduction elements per fp16 scale: 32 or 64
    int bits;    // bits per weight: 4 or 8
};
BlobLayout blob_layout(int hidden, int inter, int group, int bits);

// One grouped-GEMM work chunk: up to kChunkRows rows of one expert.
// expert == n_experts means the shared expert.  row0 indexes the rows of the
// hidden-activation buffer (routed rows in gather order, then shared rows at
// n_tok*k + t).
struct ChunkDesc {
    int32_t expert;
    int32_t row0;
    int32_t rows;
    int32_t pad;
};

// One work unit of a fused small-batch call, resolved by the decode front's
// selection so that the expert launches after it read it in one scalar
// round: the expert's blob, its first hidden-buffer row and row count, and
// its id (E for the shared expert); m < 0 marks a unit past the last one.
struct alignas(32) UnitDesc {
    const uint8_t *blob;
    int32_t r0, m, e, pad;
    int64_t pad2;
};

struct FwdArgs {
    const void *x;                  // [n_tok x H] fp32 or bf16
    int act_bf16;
    const uint8_t *const *table;    // [E + 1] device blob pointers (NULL = skip)
    const int32_t *n_union;
    const int32_t *union_ids;
    const int32_t *counts;
    const int32_t *offsets;
    const int32_t *gather;
    const float *topk_w;
    int n_tok, k, hidden, inter, n_experts, has_shared;
    BlobLayout lay;
    _Float16 *h;                    // [(n_tok*k + n_tok) x I], plus the discard row and a zero row
    _Float16 *xh;                   // [n_tok x H] fp16 copy of x (grouped path), plus a zero row
    float *ys;                      // [(n_tok*k + n_tok) x H], plus the discard row
    int discard_row;                // row of h and ys that takes the padding rows' stores
    int zero_row_x, zero_row_h;     // rows of xh and h holding zeros: the padding rows' A operand
    float *y;                       // [n_tok x H]
    const ChunkDesc *chunks;        // grouped path work list
    int chunk_rows;                 // grouped path: kChunkRows or kSmallChunkRows (chunk_rows_for)
    const int32_t *n_chunks;
    int32_t *queues;                // grouped path: kQueueInts counters, zero at rest
    int skip_shared;                // gate/up: the shared unit was already done
    const UnitDesc *units;          // resolved units (fused small-batch call), or NULL
    int32_t *err;                   // device error flags (kErr* bits), sticky until read
};

// Device error flags (coli_layer_device_errors).
constexpr int32_t kErrExpertId = 1;     // an out-of-range expert id reached the union
constexpr int32_t kErrActRange = 2;     // an activation was non-finite or outside the fp16 range
constexpr int32_t kErrHiddenRange = 4;  // a SwiGLU value h was non-finite or outside the fp16 range

// Kernel launch used by every launcher.  When the calling thread has armed
// a pair of events (timing mode), the next launch records the kernel's own
// start and end timestamps into them (hipExtLaunchKernel); otherwise it is a
// plain launch.  The slot is thread-local and disarmed by that launch.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchTiming &launch_timing();

template <typename... P, typename... A>
void launch(void (*kern)(P...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s, A... args) {
    LaunchTiming &t = launch_timing();
    if (t.start) {
        hipEvent_t a = t.start, b = t.stop;
        t.start = t.stop = nullptr;
        hipExtLaunchKernelGGL(kern, grid, block, lds, s, a, b, 0u, static_cast<P>(args)...);
    } else {
        kern<<<grid, block, lds, s>>>(static_cast<P>(args)...);
    }
}

// route.hip
hipError_t launch_router_logits(const void *x, int act_bf16, const float *wt,
                                const float *bias, int n_tok, int hidden,
                                int n_experts, float *logits, hipStream_t s);
hipError_t launch_topk(const float *logits, int n_tok, int n_experts, int k,
                       int32_t *idx, float *w, hipStream_t s);
// union.hip
// The union runs in two launches (rank, then scatter) over slabs of entries;
// UnionScratch is the layer's workspace for them: blk [kUnionMaxBlocks x E]
// per-slab counts, counter (zero at rest) and rank [max_tokens * k].
constexpr int kUnionMaxBlocks = 64;
struct UnionScratch {
    int32_t *blk;
    int32_t *counter;
    int32_t *rank;
};
struct UnionSplit {
    int nb;    // workgroups (slabs)
    int slab;  // entries per slab, a multiple of 256
};
UnionSplit union_split(int n_tok, int k);
hipError_t launch_union_rank(const int32_t *idx, int n_tok, int k, int n_experts, UnionScratch ws,
                             int32_t *n_union, int32_t *union_ids, int32_t *counts, int32_t *offsets,
                             int32_t *err, hipStream_t s);
hipError_t launch_union_scatter(const int32_t *idx, int n_tok, int k, int n_experts, UnionScratch ws,
                                const int32_t *offsets, int32_t *gather, hipStream_t s);
hipError_t launch_plan(const FwdArgs &a, ChunkDesc *chunks, int32_t *n_chunks,
                       hipStream_t s);
// Up to kUnionSmallEntries entries (n_tok * k): the union in one launch of
// one workgroup, the same outputs as rank + scatter.  With chunks non-NULL
// the launch also writes the grouped work list (as launch_plan) and the fp16
// copy of a.x (as launch_to_half); a carries a.err, and for the work list and
// the copy n_tok, k, n_experts, has_shared, chunk_rows, x, act_bf16, hidden
// and xh.
constexpr int kUnionSmallEntries = 2048;
hipError_t launch_union_small(const int32_t *idx, int n_tok, int k, int n_experts, int32_t *n_union,
                              int32_t *union_ids, int32_t *counts, int32_t *offsets, int32_t *gather,
                              const FwdArgs &a, ChunkDesc *chunks, int32_t *n_chunks, hipStream_t s);
// gemv.hip.  gate/up covers units [u_begin, u_begin + u_count) (u_count < 0:
// to the end).  down with non-NULL combine_counters ([H/32] ints, zero at
// rest) also writes y and needs every unit to be computed in this launch;
// idle_counter (may be NULL), a counter of an earlier launch of the same
// call, is cleared by it (see FrontArgs::next_counters).
hipError_t launch_gemv_gateup(const FwdArgs &a, size_t max_lds, hipStream_t s, int u_begin = 0,
                              int u_count = -1);
hipError_t launch_gemv_down(const FwdArgs &a, size_t max_lds, hipStream_t s,
                            int32_t *combine_counters = nullptr, int32_t *idle_counter = nullptr);
// decode.hip: route + top-k + union of up to kFrontMaxTok tokens and, in the
// same launch, the shared expert's gate/up.  Needs n_experts <= 256.
constexpr int kFrontMaxTok = 4;
struct FrontArgs {
    const float *wt;          // router weight [E x H]
    const float *bias;        // [E]
    float *logits;            // [n_tok x E] scratch
    int32_t *topk_idx;        // [n_tok x k]
    float *topk_w;            // [n_tok x k]
    int32_t *n_union, *union_ids, *counts, *offsets, *gather;
    int32_t *counter;         // one int, zero at rest
    // The arrival counters of the fused down launch that follows (n_next
    // ints): idle while this launch runs, so the first router block clears
    // them, and a call that follows calls which overlapped (and raced) on
    // the counters starts from zero again.
    int32_t *next_counters;
    int n_next;
    // Resolved units for the expert launches that follow (n_units of them:
    // the routed slots min(n_tok k, E) plus the shared unit), or NULL.
    UnitDesc *units;
    int n_units;
};
hipError_t launch_decode_front(const FwdArgs &a, const FrontArgs &f, size_t max_lds, hipStream_t s);
// grouped.hip
hipError_t launch_grouped_gateup(const FwdArgs &a, int max_chunks, int n_cu,
                                 hipStream_t s);
hipError_t launch_grouped_down(const FwdArgs &a, int max_chunks, int n_cu,
                               hipStream_t s);
hipError_t launch_combine(const FwdArgs &a, hipStream_t s);
hipError_t launch_to_half(const FwdArgs &a, hipStream_t s);

// Grouped-path work queues: one counter per XCD (8), each on its own
// 256-byte line, plus the exit count.
constexpr int kGroupedQueues = 8;
constexpr int kQueueStride = 64;
constexpr int kQueueInts = (kGroupedQueues + 1) * kQueueStride;

// Upper bound on grouped work chunks for n_tok tokens cut at chunk_rows.
int max_work_chunks(int n_tok, int k, int n_experts, int has_shared, int chunk_rows);
// Work-list capacity a layer of max_tokens needs (either chunk size).
int work_list_capacity(int max_tokens, int k, int n_experts, int has_shared);

}  // namespace coli
