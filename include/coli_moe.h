/*
 * coli_moe.h -- C ABI of the int4 routed-expert MoE layer for AMD MI355X
 * (gfx950).  ABI version 5 (COLI_ABI_VERSION).
 *
 * One call sequence runs one Mixture-of-Experts layer over a batch of tokens,
 * following the per-token path of the Colibri pages (getting-started page,
 * "動作原理 / トークンごとの処理経路"; README "Come funziona / Il percorso di
 * ogni token"):
 *
 *   coli_moe_route    Route: router logits, top-k experts per token and their
 *                     weights.
 *   coli_moe_union    Union: deduplicate the selected experts across the
 *                     batch ("batch-union", README "Mai aspettare il disco due
 *                     volte"), so each unique expert is read once.
 *   coli_moe_forward  the int4 (or int8) SwiGLU expert FFNs over the union, plus the
 *                     always-on shared expert, and the routing-weighted
 *                     combine.
 *   coli_expert_place Place: keep an expert in VRAM or in pinned host memory
 *                     (streamed over PCIe on a side stream when used).  The
 *                     README states that placement changes speed only, never
 *                     router decisions or weight precision: results are
 *                     bit-identical across placements.
 *
 * The pages give no formula for any step.  The definitions implemented here:
 *
 *   logit[t][e]  = fp32 dot(x_t, W_r[:, e]) + b[e], summed in one fixed order:
 *                  64 interleaved fmaf chains (chain l takes reduction indices
 *                  l, l+64, l+128, ... ascending) folded by the tree
 *                  s = 32,16,8,4,2,1 (p[i] = p[i] + p[i+s]), then + b[e].
 *   top-k        = the k largest logits under (logit desc, expert id asc);
 *                  slot order is rank order.
 *   weight       = sigmoid(logit_j) / sum over the k selected of sigmoid.
 *   expert e     = y = Wd (silu(Wg x) * (Wu x)), silu(z) = z sigmoid(z).
 *   output y_t   = sum_j weight_j * expert_{e_j}(x_t) + shared(x_t).
 *
 * Expert weights are int4 (two's complement, element 2j in the low nibble of
 * byte j, 2j+1 in the high nibble) or int8 (one two's-complement byte per
 * element) with one fp16 scale per `group` consecutive reduction elements
 * (w = q * s), group 32 or 64.  The int4 container and its group scales
 * follow the README "Scarica il modello" (group-scaled int4, 64 elements per
 * scale in the shipped files); the same section and the getting-started page
 * require int8 for the MTP head, whose layout the pages do not give: int8
 * blobs keep the int4 blob's sections and scales with one byte per weight.
 * Int8 layers run on the GEMV path for every batch size.
 *
 * Accepted values: activations x must be finite with |x| < 65520 (they are
 * rounded to fp16 on the device), and each SwiGLU value h must round to a
 * finite fp16.  A value outside that range is not an error return (the
 * device cannot report it before the call returns): it sets a bit in the
 * layer's device error flags (coli_layer_device_errors) and the affected
 * outputs are inf or NaN.
 *
 * Conventions for every entry point:
 *  - Return codes only; nothing aborts or throws across the ABI.  On error
 *    the layer stays usable and coli_last_error() holds a message.
 *  - Arguments are validated on the host before any device work; a call that
 *    fails validation has no effect.
 *  - "device pointer" arguments are HIP device memory owned by the caller
 *    (e.g. torch tensors); "host pointer" arguments are ordinary host memory.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Device work is
 *    enqueued on it asynchronously, except where a call says it synchronises.
 *  - One host thread at a time per layer handle.  Distinct handles are
 *    independent.
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COLI_ABI_VERSION 5

typedef enum {
    COLI_OK = 0,
    COLI_E_INVALID = 1,      /* bad argument; nothing was done */
    COLI_E_NOMEM = 2,        /* device or pinned-host allocation failed */
    COLI_E_DEVICE = 3,       /* a HIP call failed (text in coli_last_error) */
    COLI_E_STATE = 4,        /* layer not ready: router or an expert unplaced */
    COLI_E_UNSUPPORTED = 5   /* shape outside what the kernels support */
} coli_status;

typedef enum { COLI_ACT_F32 = 0, COLI_ACT_BF16 = 1 } coli_act;
typedef enum { COLI_TIER_VRAM = 0, COLI_TIER_HOST = 1 } coli_tier;

/* Forward strategy.  AUTO picks the VALU GEMV path for n_tok <= 4 and the
 * grouped MFMA path otherwise.  Both give results within tolerance of the
 * definition; for a given strategy results are deterministic. */
typedef enum {
    COLI_PATH_AUTO = 0,
    COLI_PATH_GEMV = 1,      /* int4 or int8 GEMV on the vector ALUs */
    COLI_PATH_GROUPED = 2    /* grouped int4->fp16 GEMM on MFMA (int4 only) */
} coli_path;

/* Expert id of the shared expert in coli_expert_place. */
#define COLI_SHARED (-1)

typedef struct {
    int32_t hidden;      /* H: multiple of 128 */
    int32_t inter;       /* I: multiple of 128 */
    int32_t n_experts;   /* E: 1..1024 routed experts */
    int32_t top_k;       /* k: 1..min(E, 32) */
    int32_t has_shared;  /* 0 or 1: one always-on shared expert */
    int32_t max_tokens;  /* largest n_tok any call will pass (>= 1) */
    int32_t act;         /* coli_act: dtype of x */
    int32_t group;       /* reduction elements per fp16 weight scale: 32 or 64 */
    int32_t weight_bits; /* 4 (int4) or 8 (int8) */
} coli_moe_dims;

typedef struct coli_layer coli_layer;   /* opaque, library-owned */

/* Bytes of one expert blob for H, I, scale group G and weight width b:
 * gate_q, up_q ([I x H*b/8] bytes each), down_q ([H x I*b/8]), gate_s, up_s
 * (fp16 [I x H/G]), down_s (fp16 [H x I/G]), in that order, each section
 * starting on a 256-byte boundary.  The README stores an expert's three
 * matrices contiguously so one read fetches all of them; this blob is that
 * unit.  Returns 0 for invalid sizes, a group other than 32 and 64, or a
 * width other than 4 and 8. */
size_t coli_expert_blob_bytes(int32_t hidden, int32_t inter, int32_t group, int32_t weight_bits);

/* Repack a blob (host pointer, layout above) into the library's device
 * layout (host pointer `out`, same size): the bytes coli_expert_place keeps
 * per expert.  Each int4 matrix is cut into 1 KB tiles of 16 rows x 128
 * columns ordered so that lane L of a 64-lane wave loads bytes L*16..L*16+15
 * of a tile: row L mod 16, columns 32s + 8(L div 16) + 0..7 in dword s, each
 * stored as q + 8 with columns 2j and 2j+1 in nibbles j and 4+j; each tile's
 * 16 x 128/group fp16 scales are stored row-major at the same tile index in
 * the scale section.  Int8 tiles are 16 rows x 64 columns: dword s of lane
 * L holds row L mod 16, columns 32(s div 2) + 8(L div 16) + 4(s mod 2) +
 * 0..3 as q + 128 in byte order 0, 2, 1, 3; their 16 x 64/group scales
 * likewise.  Host-only, no device needed.  COLI_E_INVALID for NULL pointers,
 * sizes that are not multiples of 128, a group other than 32 and 64, or a
 * width other than 4 and 8. */
coli_status coli_expert_repack(const void *blob_host, void *out_host,
                               int32_t hidden, int32_t inter, int32_t group, int32_t weight_bits);

/* Create a layer on HIP device `device`.  Allocates the router copy, the
 * expert pointer table and scratch sized from dims->max_tokens.
 * COLI_E_INVALID for bad dims, COLI_E_UNSUPPORTED for sizes the kernels do
 * not handle, COLI_E_DEVICE if the device cannot be used, COLI_E_NOMEM on
 * allocation failure.  *out is set only on success. */
coli_status coli_layer_create(const coli_moe_dims *dims, int device,
                              coli_layer **out);

/* Free everything the layer owns (device memory, pinned host copies,
 * streams).  NULL is accepted.  Synchronises the device. */
coli_status coli_layer_destroy(coli_layer *layer);

/* Copy the router weight W_r (host pointer, fp32 [H x E], reduction index
 * outer: w_host[k*E + e]) and optional bias (host pointer, fp32 [E], or NULL
 * for zero) into the layer.  Synchronous: it first waits for all work on the
 * layer's device (every stream), so calls already queued keep the router
 * they were issued with. */
coli_status coli_router_set(coli_layer *layer, const float *w_host,
                            const float *bias_host);

/* Place expert `expert` (0..E-1, or COLI_SHARED) from a host blob in the
 * layout of coli_expert_blob_bytes for the layer's group and weight_bits
 * (blob_bytes must equal that size, else COLI_E_INVALID).  The library repacks it once into its
 * device layout and keeps it in VRAM (COLI_TIER_VRAM) or in pinned host
 * memory (COLI_TIER_HOST, copied to a device staging slot when a forward
 * call needs it).  Re-placing an expert replaces its data and tier.  The
 * shared expert must be VRAM-resident.  blob_host may be freed on return.
 * Synchronous: it first waits for all work on the layer's device (every
 * stream, including copies started by coli_layer_prefetch_union), so calls
 * already queued read the expert they were issued with; the new data is
 * seen by calls made after it returns. */
coli_status coli_expert_place(coli_layer *layer, int32_t expert,
                              const void *blob_host, size_t blob_bytes,
                              coli_tier tier);

/* Route: for n_tok tokens x (device pointer, [n_tok x H], fp32 or bf16 per
 * dims.act), write topk_idx (device, int32 [n_tok x k], rank order) and
 * topk_w (device, fp32 [n_tok x k]).  0 <= n_tok <= max_tokens; n_tok == 0
 * does nothing.  COLI_E_STATE if the router was never set.  3 to 128 tokens
 * run as one launch (the same bits as the two); calls that overlap on one
 * layer race on its arrival counters. */
coli_status coli_moe_route(coli_layer *layer, const void *x, int32_t n_tok,
                           int32_t *topk_idx, float *topk_w, void *stream);

/* Router logits only (device, fp32 [n_tok x E]), in the fixed summation
 * order above; coli_moe_route selects from exactly these values. */
coli_status coli_moe_router_logits(coli_layer *layer, const void *x,
                                   int32_t n_tok, float *logits, void *stream);

/* Union over the batch of topk_idx (device, int32 [n_tok x k], ids in
 * 0..E-1, distinct within a token, as coli_moe_route writes them).  Writes
 * (all device): n_union [1]; union_ids [E] (ascending, first n_union valid);
 * counts [E] (tokens per expert); offsets [E+1] (exclusive prefix sum of
 * counts); gather [n_tok*k] (entries t*k+j ordered by expert id, then token).
 * Out-of-range ids are skipped and raise the layer's device error flag
 * (coli_layer_device_errors).  Two launches that use the layer's scratch:
 * calls on one layer must not overlap. */
coli_status coli_moe_union(coli_layer *layer, const int32_t *topk_idx,
                           int32_t n_tok, int32_t *n_union, int32_t *union_ids,
                           int32_t *counts, int32_t *offsets, int32_t *gather,
                           void *stream);

/* Forward: y (device, fp32 [n_tok x H]) = routing-weighted sum of the expert
 * FFNs over the union, plus the shared expert, for the tokens x (device),
 * given the outputs of coli_moe_route and coli_moe_union for the same batch.
 * Requires the router to have been set and the shared expert (if any) to be
 * VRAM-resident.  If every routed expert is VRAM-resident the call is fully
 * asynchronous.  Otherwise it reads back the union (synchronising `stream`),
 * returns COLI_E_STATE if a routed expert in the union was never placed, and
 * streams pinned-host experts into staging slots on a side stream while the
 * resident ones compute; it returns after the stream has drained.  Results
 * are bit-identical whichever tier an expert sits in. */
coli_status coli_moe_forward(coli_layer *layer, const void *x, int32_t n_tok,
                             const int32_t *topk_idx, const float *topk_w,
                             const int32_t *n_union, const int32_t *union_ids,
                             const int32_t *counts, const int32_t *offsets,
                             const int32_t *gather, float *y, void *stream);

/* The whole layer in one call: route, union and forward of n_tok tokens,
 * writing the same outputs as coli_moe_route, coli_moe_union and
 * coli_moe_forward called in sequence (same pointer conventions).  For small
 * batches (n_tok <= 4, n_experts <= 256, every expert in VRAM, GEMV
 * strategy) it runs as three launches: router + top-k + union together with
 * the shared expert's gate/up, then the routed gate/up, then the down
 * projection which also combines; the results are bit-identical to the
 * three separate calls.  Otherwise it issues the three calls.  Calls on one
 * layer must not overlap in time (they share the layer's arrival counters). */
coli_status coli_moe_layer(coli_layer *layer, const void *x, int32_t n_tok,
                           int32_t *topk_idx, float *topk_w, int32_t *n_union,
                           int32_t *union_ids, int32_t *counts,
                           int32_t *offsets, int32_t *gather, float *y,
                           void *stream);

/* coli_moe_layer for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, outputs and bits as coli_moe_layer's fused small-batch
 * path, but its scratch (logits, h and per-entry output rows, arrival
 * counters, unit descriptors) lives in one static device array of 8 MiB per
 * GPU, set up by the first coli_layer_create on that GPU and held until the
 * process ends; the call allocates nothing and creates no HIP objects
 * (kernel timing is not recorded).  Limits: the fused path only (1..4
 * tokens, n_experts <= 256, every expert in VRAM, router set, GEMV
 * strategy), else COLI_E_UNSUPPORTED; a call needing more than 8 MiB of
 * scratch, about n_tok*(k+1)*(4*H + 2*I) + 32*(n_experts+1) bytes, is
 * refused with COLI_E_UNSUPPORTED before any device work.  Every layer on a GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (any layers, any streams) race and give
 * undefined results; issue them in one stream order. */
coli_status coli_moe_layer_static(coli_layer *layer, const void *x, int32_t n_tok,
                                  int32_t *topk_idx, float *topk_w, int32_t *n_union,
                                  int32_t *union_ids, int32_t *counts,
                                  int32_t *offsets, int32_t *gather, float *y,
                                  void *stream);

/* Choose the forward strategy (coli_path).  Default COLI_PATH_AUTO.
 * COLI_E_UNSUPPORTED for COLI_PATH_GROUPED on an int8 layer (int8 layers
 * always take the GEMV path). */
coli_status coli_layer_set_path(coli_layer *layer, int32_t path);

/* Statistics of the last tiered forward call (host pointers, may be NULL):
 * experts streamed over PCIe and bytes copied. */
coli_status coli_layer_stream_stats(const coli_layer *layer,
                                    int32_t *n_streamed, int64_t *bytes);

/* Keep up to n_slots pinned-host experts in VRAM between tiered forward
 * calls (the pages' placement step: a copy that a later call finds in VRAM
 * needs no PCIe transfer).  Each slot is one expert blob of device memory,
 * allocated at the next tiered call; the least recently used slot is
 * replaced on a miss.  0 (the default) copies every host-tier expert on
 * every call.  Results are bit-identical with or without the cache.
 * Re-placing an expert drops its cached copy; changing n_slots drops all.
 * COLI_E_INVALID unless n_slots is 0 or between 4 and n_experts. */
coli_status coli_layer_set_stream_cache(coli_layer *layer, int32_t n_slots);

/* Host-tier experts of the last tiered forward call that were found in the
 * stream cache (host pointer). */
coli_status coli_layer_stream_hits(const coli_layer *layer, int32_t *hits);

/* Lookahead prefetch into the stream cache: the README ("Mai aspettare il
 * disco due volte") runs the next layer's router ahead of time and fetches
 * the experts it predicts while the current layer computes; the
 * getting-started page's Overlap step overlaps such transfers with compute.
 * Given a union (device pointers n_union [1] and union_ids [E], as
 * coli_moe_union writes them, e.g. for this layer's next batch computed
 * early), this call reads it back (synchronising `stream`), then starts one
 * host-to-device copy per host-tier expert of the union that is not cached
 * yet into a stream-cache slot, on the layer's side stream, and returns
 * without waiting for them.  Slots are taken empty first, then least
 * recently used; a slot filled by this call or whose earlier prefetch copy
 * is still in flight is never taken, so when the slots run out the rest of
 * the union is skipped.  A later forward call that finds a prefetched expert
 * waits for that copy on its own stream (not on the host).  Results are
 * bit-identical with or without prefetch.  *n_started (host pointer, may be
 * NULL) = copies started.  COLI_E_STATE without a stream cache
 * (coli_layer_set_stream_cache), COLI_E_INVALID for NULL pointers or a
 * union id out of range, COLI_E_NOMEM if the slots cannot be allocated. */
coli_status coli_layer_prefetch_union(coli_layer *layer, const int32_t *n_union,
                                      const int32_t *union_ids, void *stream,
                                      int32_t *n_started);

/* Read and clear the device error flags (synchronises the device), set by
 * the kernels of every call since the last read:
 *   bit 0 (1) = an out-of-range expert id reached coli_moe_union;
 *   bit 1 (2) = an activation was not finite or had |x| >= 65520 (outside
 *               the fp16 range the expert kernels compute in);
 *   bit 2 (4) = a SwiGLU value h rounded to an infinite or NaN fp16. */
coli_status coli_layer_device_errors(coli_layer *layer, int32_t *flags);

/* Kernel timing, for tracing and benchmarks.  While enabled, every kernel
 * the layer launches carries two HIP events that receive that kernel's own
 * start and end timestamps (hipExtLaunchKernel), and its duration is added to
 * the total of its kind; launch gaps between kernels are not counted.  coli_layer_kernel_times
 * synchronises the device, writes per-kind totals (host arrays of
 * COLI_KERNEL_KINDS entries, either may be NULL) and resets them. */
typedef enum {
    COLI_K_ROUTER = 0,   /* router logits */
    COLI_K_TOPK = 1,     /* top-k and weights (3 to 128 tokens: in the router's launch) */
    COLI_K_UNION = 2,    /* batch union (2 launches: slab ranks, scatter) */
    COLI_K_PLAN = 3,     /* grouped work list; fp16 activations (2 launches) */
    COLI_K_GATEUP = 4,   /* gate/up + SwiGLU (GEMV or grouped) */
    COLI_K_DOWN = 5,     /* down projection x routing weight */
    COLI_K_COMBINE = 6,  /* per-token sum of expert rows */
    COLI_KERNEL_KINDS = 7
} coli_kernel_kind;
coli_status coli_layer_set_timing(coli_layer *layer, int32_t enable);
coli_status coli_layer_kernel_times(coli_layer *layer, double *ms_total,
                                    int64_t *launches);

const char *coli_status_str(coli_status status);
const char *coli_last_error(const coli_layer *layer);
int32_t coli_abi_version(void);

/* Allocation cap, for tests and capacity planning: the library holds at
 * most `bytes` of device and pinned host memory in total, over all layers
 * of the process (-1, the default, removes the cap).  An allocation that
 * would pass it fails with COLI_E_NOMEM exactly as a real allocation
 * failure does (coli_layer_create checks its whole need before touching the
 * device); the call that failed has no other effect and the layer stays
 * usable.  The cap applies to allocations made after it is set; memory
 * already held is not released.  COLI_E_INVALID for bytes < -1. */
coli_status coli_set_alloc_limit(int64_t bytes);

/* Bytes of device and pinned host memory the library currently holds. */
int64_t coli_alloc_bytes(void);

/* Measurement reference, for benchmarks: streams `bytes` of device memory
 * at `buf` once on `stream` (the current device) with the plainest fast read
 * -- 16-byte non-temporal loads, eight in flight per thread, one 256-thread
 * workgroup per CU striding over the buffer -- and XORs every 32-bit word
 * read into *sink (device memory, one uint32_t, which the caller clears
 * first to read the XOR).  Timed by the caller over a buffer far larger
 * than the 256 MB memory-side cache, its rate is the HBM read bandwidth the
 * part reaches in practice, the ceiling beside the 8 TB/s peak that the
 * expert kernels' algorithmic rates are compared with.  buf and sink stay
 * caller-owned.  COLI_E_INVALID for NULL pointers, a size that is not a
 * multiple of 16 or a buf that is not 16-byte aligned; COLI_E_DEVICE without
 * a device or if the launch fails.  bytes == 0 launches nothing. */
coli_status coli_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* COLI_MOE_H */
