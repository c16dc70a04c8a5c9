// abi.hip -- host side of the C ABI declared in include/coli_moe.h:
// argument validation, layer lifetime, placement (repack into the device
// layout, VRAM or pinned-host tier), and the orchestration of the route,
// union and forward kernels, including the tiered forward that streams
// pinned-host experts over PCIe on a side stream while resident experts
// compute (the README's Place and Overlap steps).
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <optional>
#include <string>
#include <thread>
#include <unordered_map>
#include <vector>

#include "coli_moe.h"
#include "internal.h"

namespace coli {
// probe.hip: the streaming-read reference kernel behind coli_probe_read.
hipError_t launch_probe_read(const void *buf, size_t bytes, uint32_t *sink, int n_cu, hipStream_t s);
// route.hip: router and top-k in one launch for 3 to 128 tokens
// (hipErrorNotSupported outside), with route_topk_counters() arrival
// counters, zero at rest.
int route_topk_counters();
hipError_t launch_router_topk(const void *x, int act_bf16, const float *wt, const float *bias, int n_tok, int hidden,
                              int n_experts, int k, float *logits, int32_t *counters, int32_t *idx, float *w,
                              hipStream_t s);
}  // namespace coli

namespace coli {

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

BlobLayout blob_layout(int hidden, int inter, int group, int bits) {
    const size_t h = static_cast<size_t>(hidden), i = static_cast<size_t>(inter), g = static_cast<size_t>(group);
    const size_t b = static_cast<size_t>(bits);
    const size_t sz[6] = {i * h * b / 8, i * h * b / 8, h * i * b / 8,
                          i * (h / g) * 2, i * (h / g) * 2, h * (i / g) * 2};
    size_t off[7];
    size_t o = 0;
    for (int k = 0; k < 6; ++k) {
        off[k] = o;
        o = align256(o + sz[k]);
    }
    off[6] = o;
    return BlobLayout{off[0], off[1], off[2], off[3], off[4], off[5], off[6], group, bits};
}

namespace {

// Nibble permutation of one packed dword (columns k0..k0+7, column i in bits
// 4i..4i+3, two's complement) into the device order: u = q + 8 in slot
// i/2 (even i) or 4 + i/2 (odd i).  Two 64K-entry tables, one per half.
struct RepackTables {
    uint32_t lo[65536];
    uint32_t hi[65536];
    RepackTables() {
        for (uint32_t v = 0; v < 65536; ++v) {
            uint32_t a = 0, b = 0;
            for (int i = 0; i < 4; ++i) {
                const uint32_t ua = ((v >> (4 * i)) & 15u) ^ 8u;      // column i
                const uint32_t ub = ua;                               // column 4+i
                const int ia = i, ib = 4 + i;
                const int sa = (ia & 1) ? 4 + (ia >> 1) : (ia >> 1);
                const int sb = (ib & 1) ? 4 + (ib >> 1) : (ib >> 1);
                a |= ua << (4 * sa);
                b |= ub << (4 * sb);
            }
            lo[v] = a;
            hi[v] = b;
        }
    }
};

const RepackTables &repack_tables() {
    static const RepackTables *t = new RepackTables();
    return *t;
}

// Repack rows [p_begin, p_end) panels of one [R x K] matrix with one scale
// per `group` columns (the chunk's 128/group scales of each row, row-major).
void repack_panels(const uint8_t *q_src, const uint16_t *s_src, int K, int group, int p_begin,
                   int p_end, uint8_t *q_dst, uint16_t *s_dst) {
    const RepackTables &T = repack_tables();
    const int C = K / kChunkK;
    const size_t row_bytes = static_cast<size_t>(K) / 2;
    const int groups = K / group, per_chunk = kChunkK / group;
    for (int p = p_begin; p < p_end; ++p) {
        for (int c = 0; c < C; ++c) {
            uint8_t *qc = q_dst + (static_cast<size_t>(p) * C + c) * kChunkBytes;
            uint16_t *sc = s_dst + (static_cast<size_t>(p) * C + c) * (kPanel * per_chunk);
            for (int lane = 0; lane < 64; ++lane) {
                const int r = p * kPanel + (lane & 15);
                for (int s = 0; s < 4; ++s) {
                    const int k0 = c * kChunkK + 32 * s + 8 * (lane >> 4);
                    uint32_t in;
                    std::memcpy(&in, q_src + static_cast<size_t>(r) * row_bytes + k0 / 2, 4);
                    const uint32_t out = T.lo[in & 0xFFFFu] | T.hi[in >> 16];
                    std::memcpy(qc + lane * 16 + s * 4, &out, 4);
                }
            }
            for (int r = 0; r < kPanel; ++r)
                for (int s = 0; s < per_chunk; ++s)
                    sc[r * per_chunk + s] = s_src[static_cast<size_t>(p * kPanel + r) * groups + per_chunk * c + s];
        }
    }
}

// Int8 variant: chunks of 16 rows x 64 columns; dword s of lane L holds
// columns k0 = 64c + 32(s >> 1) + 8(L >> 4) + 4(s & 1) .. k0+3 of row
// L & 15 as u = q + 128 in byte order k0, k0+2, k0+1, k0+3; the chunk's
// 16 x 64/group scales follow row-major at its index in the scale section.
void repack_panels_i8(const uint8_t *q_src, const uint16_t *s_src, int K, int group, int p_begin,
                      int p_end, uint8_t *q_dst, uint16_t *s_dst) {
    constexpr int kCols = 64;
    const int C = K / kCols;
    const int groups = K / group, per_chunk = kCols / group;
    for (int p = p_begin; p < p_end; ++p) {
        for (int c = 0; c < C; ++c) {
            uint8_t *qc = q_dst + (static_cast<size_t>(p) * C + c) * kChunkBytes;
            uint16_t *sc = s_dst + (static_cast<size_t>(p) * C + c) * (kPanel * per_chunk);
            for (int lane = 0; lane < 64; ++lane) {
                const uint8_t *row = q_src + static_cast<size_t>(p * kPanel + (lane & 15)) * K;
                for (int s = 0; s < 4; ++s) {
                    const int k0 = c * kCols + 32 * (s >> 1) + 8 * (lane >> 4) + 4 * (s & 1);
                    uint8_t *out = qc + lane * 16 + s * 4;
                    out[0] = row[k0] ^ 0x80u;
                    out[1] = row[k0 + 2] ^ 0x80u;
                    out[2] = row[k0 + 1] ^ 0x80u;
                    out[3] = row[k0 + 3] ^ 0x80u;
                }
            }
            for (int r = 0; r < kPanel; ++r)
                for (int t = 0; t < per_chunk; ++t)
                    sc[r * per_chunk + t] = s_src[static_cast<size_t>(p * kPanel + r) * groups + per_chunk * c + t];
        }
    }
}

void repack_blob(const uint8_t *src, uint8_t *dst, int hidden, int inter, int group, int bits) {
    const BlobLayout L = blob_layout(hidden, inter, group, bits);
    std::memset(dst, 0, L.total);
    struct Mat { size_t q, s; int rows, K; } mats[3] = {
        {L.gate_q, L.gate_s, inter, hidden},
        {L.up_q, L.up_s, inter, hidden},
        {L.down_q, L.down_s, hidden, inter}};
    const unsigned hw = std::max(1u, std::min(8u, std::thread::hardware_concurrency()));
    const size_t work = L.total;
    const int nthreads = work >= (4u << 20) ? static_cast<int>(hw) : 1;
    for (const Mat &m : mats) {
        const int P = m.rows / kPanel;
        auto run = [&](int b, int e) {
            if (bits == 8)
                repack_panels_i8(src + m.q, reinterpret_cast<const uint16_t *>(src + m.s), m.K, group, b, e,
                                 dst + m.q, reinterpret_cast<uint16_t *>(dst + m.s));
            else
                repack_panels(src + m.q, reinterpret_cast<const uint16_t *>(src + m.s), m.K, group, b, e,
                              dst + m.q, reinterpret_cast<uint16_t *>(dst + m.s));
        };
        if (nthreads <= 1 || P < 2 * nthreads) {
            run(0, P);
        } else {
            std::vector<std::thread> th;
            const int per = (P + nthreads - 1) / nthreads;
            for (int t = 0; t < nthreads; ++t) {
                const int b = t * per, e = std::min(P, b + per);
                if (b < e) th.emplace_back(run, b, e);
            }
            for (auto &x : th) x.join();
        }
    }
}

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

thread_local std::string g_create_error;

// Every device and pinned-host allocation the library makes goes through
// these helpers, which keep the bytes held (all layers of the process) and
// apply the optional cap set by coli_set_alloc_limit: an allocation that
// would pass the cap fails as hipErrorOutOfMemory before HIP is called.
struct MemBook {
    std::mutex mu;
    std::unordered_map<void *, size_t> live;
    int64_t used = 0;
    int64_t limit = -1;   // -1: no cap
};
MemBook &mem_book() {
    static MemBook *b = new MemBook();
    return *b;
}
bool mem_fits(size_t n) {
    MemBook &b = mem_book();
    std::lock_guard<std::mutex> g(b.mu);
    return b.limit < 0 || b.used + static_cast<int64_t>(n) <= b.limit;
}
void mem_note(void *p, size_t n) {
    MemBook &b = mem_book();
    std::lock_guard<std::mutex> g(b.mu);
    b.live[p] = n;
    b.used += static_cast<int64_t>(n);
}
void mem_forget(void *p) {
    MemBook &b = mem_book();
    std::lock_guard<std::mutex> g(b.mu);
    auto it = b.live.find(p);
    if (it == b.live.end()) return;
    b.used -= static_cast<int64_t>(it->second);
    b.live.erase(it);
}
template <typename T>
hipError_t dev_alloc(T **p, size_t n) {
    if (!mem_fits(n)) return hipErrorOutOfMemory;
    void *q = nullptr;
    const hipError_t e = hipMalloc(&q, n);
    if (e != hipSuccess) return e;
    mem_note(q, n);
    *p = static_cast<T *>(q);
    return hipSuccess;
}
template <typename T>
hipError_t host_alloc(T **p, size_t n) {
    if (!mem_fits(n)) return hipErrorOutOfMemory;
    void *q = nullptr;
    const hipError_t e = hipHostMalloc(&q, n, hipHostMallocDefault);
    if (e != hipSuccess) return e;
    mem_note(q, n);
    *p = static_cast<T *>(q);
    return hipSuccess;
}
void dev_free(const void *p) {
    if (!p) return;
    mem_forget(const_cast<void *>(p));
    (void)hipFree(const_cast<void *>(p));
}
void host_free(const void *p) {
    if (!p) return;
    mem_forget(const_cast<void *>(p));
    (void)hipHostFree(const_cast<void *>(p));
}

}  // namespace
}  // namespace coli

// Scratch of coli_moe_layer_static, the entry point that allocates
// nothing: one array per GPU, in the code object's device memory, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: host code uses only the per-device address that
// hipGetSymbolAddress returns (static_scratch_ptr).
namespace coli {
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
constexpr int kStaticMaxDevices = 64;
}  // namespace coli
static __device__ __align__(256) uint8_t scratch[coli::kStaticScratchBytes];

namespace coli {
namespace {
std::mutex g_static_mu;
void *g_static_ptr[kStaticMaxDevices] = {};

// Looks up the device address of `scratch` on `device` (current) and zeroes
// it, once per device; later calls return the stored address.
hipError_t static_scratch_setup(int device, void **out) {
    *out = nullptr;
    if (device < 0 || device >= kStaticMaxDevices) return hipSuccess;   // no static scratch there
    std::lock_guard<std::mutex> g(g_static_mu);
    if (!g_static_ptr[device]) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if ((e = hipMemset(p, 0, kStaticScratchBytes)) != hipSuccess) return e;
        if ((e = hipDeviceSynchronize()) != hipSuccess) return e;
        g_static_ptr[device] = p;
    }
    *out = g_static_ptr[device];
    return hipSuccess;
}

void *static_scratch_ptr(int device) {
    if (device < 0 || device >= kStaticMaxDevices) return nullptr;
    std::lock_guard<std::mutex> g(g_static_mu);
    return g_static_ptr[device];
}
}  // namespace
}  // namespace coli

using namespace coli;

struct ExpertSlot {
    uint8_t *dev = nullptr;     // VRAM copy (device layout)
    uint8_t *host = nullptr;    // pinned host copy (device layout)
    int tier = -1;              // -1 unplaced, else coli_tier
};

struct coli_layer {
    coli_moe_dims d{};
    int device = 0;
    int n_cu = 0;
    size_t max_lds = 0;
    BlobLayout lay{};
    int path = COLI_PATH_AUTO;

    float *wt = nullptr;        // router weight, transposed [E x H]
    float *bias = nullptr;      // [E]
    bool router_set = false;

    std::vector<ExpertSlot> experts;          // E + 1 (index E = shared)
    std::vector<const uint8_t *> table_host;  // mirrors table_dev
    const uint8_t **table_dev = nullptr;      // [E + 1]; NULL for non-VRAM experts

    float *logits = nullptr;    // [max_tokens x E]
    _Float16 *h = nullptr;      // [(max_tokens*k + max_tokens + 1) x I]; the last row takes discarded stores
    _Float16 *xh = nullptr;     // [max_tokens x H]
    float *ys = nullptr;        // [(max_tokens*k + max_tokens + 1) x H]; the last row takes discarded stores
    ChunkDesc *chunks = nullptr;
    int32_t *n_chunks = nullptr;
    int max_chunks = 0;
    int32_t *err = nullptr;
    int32_t *sync_counters = nullptr;  // [1 + H/32 + route_topk_counters()] arrival counters, zero at rest
    int32_t *queues = nullptr;         // [kQueueInts] grouped work-queue counters, zero at rest
    int32_t *union_blk = nullptr;      // [kUnionMaxBlocks x E + 64]; counter at [kUnionMaxBlocks x E]
    int32_t *union_rank = nullptr;     // [max_tokens x k]
    UnitDesc *units = nullptr;         // [E + 1] resolved units of the fused small-batch call
    uint8_t *pin_stage = nullptr;    // pinned staging for placement

    // tiered forward
    hipStream_t side = nullptr;
    std::vector<uint8_t *> slots;
    std::vector<hipEvent_t> slot_free;
    std::vector<hipEvent_t> batch_ready;
    std::vector<const uint8_t **> pin_tables;
    std::vector<const uint8_t **> dev_tables;
    int32_t *pin_union = nullptr;    // [1 + E]
    int32_t last_streamed = 0;
    int64_t last_bytes = 0;
    int32_t last_hits = 0;
    // Stream cache: slots keep host-tier experts between calls (LRU).
    int cache_slots = 0;
    std::vector<int> slot_expert;    // expert held by each slot, -1 none
    std::vector<int64_t> slot_stamp; // last call that used the slot
    std::vector<int> expert_slot;    // [E] slot holding the expert, -1 none
    // Prefetch (coli_layer_prefetch_union): a slot filled by a prefetch copy
    // on the side stream is pending until a forward call waits on its
    // slot_ready event.
    std::vector<hipEvent_t> slot_ready;
    std::vector<char> slot_pending;
    int64_t call_no = 0;

    // kernel timing
    bool timing = false;
    struct Mark { int kind; hipEvent_t a, b; };
    std::vector<Mark> marks;          // recorded since the last read
    std::vector<hipEvent_t> ev_pool;  // idle events

    std::string msg;
};

namespace {

constexpr int kSlotCount = 16;
constexpr int kBatchExperts = 4;

coli_status fail(coli_layer *L, coli_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (L) L->msg = buf;
    else g_create_error = buf;
    return st;
}

coli_status hip_fail(coli_layer *L, hipError_t e, const char *what) {
    return fail(L, e == hipErrorOutOfMemory ? COLI_E_NOMEM : COLI_E_DEVICE, "%s: %s", what,
                hipGetErrorString(e));
}

#define HIP_TRY(L, call, what)                          \
    do {                                                \
        hipError_t e_ = (call);                         \
        if (e_ != hipSuccess) return hip_fail(L, e_, what); \
    } while (0)

}  // namespace

LaunchTiming &coli::launch_timing() {
    static thread_local LaunchTiming t;
    return t;
}

namespace {

hipEvent_t take_event(coli_layer *L) {
    if (!L->ev_pool.empty()) {
        hipEvent_t e = L->ev_pool.back();
        L->ev_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Times the one kernel launched while it is alive: when timing is enabled it
// arms the thread's launch slot with two events, which the launch fills with
// the kernel's own start and end timestamps.
struct KernelMark {
    coli_layer *L;
    int kind;
    hipEvent_t a = nullptr, b = nullptr;
    KernelMark(coli_layer *L_, int kind_, hipStream_t) : L(L_), kind(kind_) {
        if (!L->timing) return;
        a = take_event(L);
        b = a ? take_event(L) : nullptr;
        if (!b) {
            if (a) L->ev_pool.push_back(a);
            a = nullptr;
            return;
        }
        launch_timing() = {a, b};
    }
    ~KernelMark() {
        if (!a) return;
        LaunchTiming &t = launch_timing();
        if (t.start == nullptr) {
            L->marks.push_back({kind, a, b});  // the launch used the events
        } else {
            t = {};
            L->ev_pool.push_back(a);
            L->ev_pool.push_back(b);
        }
    }
};

bool dims_valid(const coli_moe_dims *d, std::string &why) {
    char buf[256];
    if (!d) { why = "dims is NULL"; return false; }
    if (d->hidden <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->max_tokens <= 0) {
        why = "dims must be positive";
        return false;
    }
    if (d->has_shared != 0 && d->has_shared != 1) { why = "has_shared must be 0 or 1"; return false; }
    if (d->act != COLI_ACT_F32 && d->act != COLI_ACT_BF16) { why = "act must be COLI_ACT_F32 or COLI_ACT_BF16"; return false; }
    if (!group_supported(d->group)) { why = "group must be 32 or 64"; return false; }
    if (!bits_supported(d->weight_bits)) { why = "weight_bits must be 4 or 8"; return false; }
    if (d->top_k > d->n_experts || d->top_k > kMaxTopK) {
        std::snprintf(buf, sizeof buf, "top_k %d must be <= min(n_experts, %d)", d->top_k, kMaxTopK);
        why = buf;
        return false;
    }
    return true;
}

bool dims_supported(const coli_moe_dims *d, std::string &why) {
    char buf[256];
    if (d->hidden % kChunkK || d->inter % kChunkK) {
        std::snprintf(buf, sizeof buf, "hidden (%d) and inter (%d) must be multiples of %d",
                      d->hidden, d->inter, kChunkK);
        why = buf;
        return false;
    }
    if (d->n_experts + d->has_shared > kMaxExperts) {
        std::snprintf(buf, sizeof buf, "n_experts + has_shared must be <= %d", kMaxExperts);
        why = buf;
        return false;
    }
    if (static_cast<int64_t>(d->max_tokens) * d->top_k > (1 << 26)) {
        why = "max_tokens * top_k too large";
        return false;
    }
    // The grouped kernels address activation and h rows with 32-bit element
    // offsets (row * width + column) over the rows of one call plus the
    // discard and zero rows; buffer descriptors cover one expert blob with a
    // 32-bit byte count.
    const int64_t rows = static_cast<int64_t>(d->max_tokens) * (d->top_k + 1) + 2;
    if (rows * std::max(d->hidden, d->inter) >= (int64_t(1) << 32)) {
        std::snprintf(buf, sizeof buf, "(max_tokens * (top_k + 1) + 2) * max(hidden, inter) = %lld must be < 2^32",
                      static_cast<long long>(rows * std::max(d->hidden, d->inter)));
        why = buf;
        return false;
    }
    if (group_supported(d->group) && bits_supported(d->weight_bits) &&
        blob_layout(d->hidden, d->inter, d->group, d->weight_bits).total >= (size_t(1) << 32)) {
        why = "one expert blob must be smaller than 4 GiB";
        return false;
    }
    return true;
}

// Bytes coli_layer_create allocates (device scratch and tables, the router,
// pinned staging), for the allocation cap's check before any device call.
size_t create_bytes(const coli_moe_dims *d) {
    const size_t E = static_cast<size_t>(d->n_experts), H = static_cast<size_t>(d->hidden),
                 I = static_cast<size_t>(d->inter), T = static_cast<size_t>(d->max_tokens),
                 k = static_cast<size_t>(d->top_k);
    const size_t rows = T * k + T;
    const size_t chunks = static_cast<size_t>(work_list_capacity(d->max_tokens, d->top_k, d->n_experts, d->has_shared));
    return sizeof(float) * E * H + sizeof(float) * E + sizeof(void *) * (E + 1) + sizeof(float) * T * E +
           sizeof(_Float16) * (rows + 2) * I + sizeof(_Float16) * (T + 1) * H + sizeof(float) * (rows + 1) * H +
           sizeof(ChunkDesc) * chunks + 2 * sizeof(int32_t) + sizeof(int32_t) * (1 + H / 32 + route_topk_counters()) +
           sizeof(int32_t) * kQueueInts + sizeof(int32_t) * (kUnionMaxBlocks * E + 64) + sizeof(int32_t) * T * k +
           blob_layout(d->hidden, d->inter, d->group, d->weight_bits).total + sizeof(int32_t) * (E + 1) +
           sizeof(UnitDesc) * (E + 1);
}

bool all_routed_resident(const coli_layer *L) {
    for (int e = 0; e < L->d.n_experts; ++e)
        if (L->experts[e].tier != COLI_TIER_VRAM) return false;
    return true;
}

int choose_path(const coli_layer *L, int n_tok) {
    if (L->d.weight_bits == 8) return COLI_PATH_GEMV;        // int8 runs on the GEMV kernels only
    if (L->path != COLI_PATH_AUTO) return L->path;
    return n_tok <= 4 ? COLI_PATH_GEMV : COLI_PATH_GROUPED;   // B=4: 183 us GEMV, 203 us grouped
}

FwdArgs make_args(coli_layer *L, const void *x, int n_tok, const float *topk_w, const int32_t *n_union,
                  const int32_t *union_ids, const int32_t *counts, const int32_t *offsets,
                  const int32_t *gather, float *y) {
    FwdArgs a{};
    a.x = x;
    a.act_bf16 = L->d.act == COLI_ACT_BF16;
    a.table = L->table_dev;
    a.n_union = n_union;
    a.union_ids = union_ids;
    a.counts = counts;
    a.offsets = offsets;
    a.gather = gather;
    a.topk_w = topk_w;
    a.n_tok = n_tok;
    a.k = L->d.top_k;
    a.hidden = L->d.hidden;
    a.inter = L->d.inter;
    a.n_experts = L->d.n_experts;
    a.has_shared = L->d.has_shared;
    a.lay = L->lay;
    a.h = L->h;
    a.xh = L->xh;
    a.ys = L->ys;
    a.discard_row = static_cast<int>(L->d.max_tokens) * (L->d.top_k + 1);
    a.zero_row_h = a.discard_row + 1;
    a.zero_row_x = static_cast<int>(L->d.max_tokens);
    a.y = y;
    a.chunks = L->chunks;
    a.chunk_rows = chunk_rows_for(n_tok);
    a.n_chunks = L->n_chunks;
    a.queues = L->queues;
    a.skip_shared = 0;
    a.err = L->err;
    return a;
}

coli_status launch_experts(coli_layer *L, const FwdArgs &a, int path, hipStream_t s) {
    hipError_t e;
    if (path == COLI_PATH_GEMV) {
        {
            KernelMark m(L, COLI_K_GATEUP, s);
            if ((e = launch_gemv_gateup(a, L->max_lds, s)) != hipSuccess) return hip_fail(L, e, "gemv gate/up launch");
        }
        KernelMark m(L, COLI_K_DOWN, s);
        if ((e = launch_gemv_down(a, L->max_lds, s)) != hipSuccess) return hip_fail(L, e, "gemv down launch");
    } else {
        const int mc = max_work_chunks(a.n_tok, a.k, a.n_experts, a.has_shared, a.chunk_rows);
        {
            KernelMark m(L, COLI_K_GATEUP, s);
            if ((e = launch_grouped_gateup(a, mc, L->n_cu, s)) != hipSuccess) return hip_fail(L, e, "grouped gate/up launch");
        }
        KernelMark m(L, COLI_K_DOWN, s);
        if ((e = launch_grouped_down(a, mc, L->n_cu, s)) != hipSuccess) return hip_fail(L, e, "grouped down launch");
    }
    return COLI_OK;
}

void free_layer(coli_layer *L) {
    if (!L) return;
    (void)hipDeviceSynchronize();
    for (auto &x : L->experts) {
        dev_free(x.dev);
        host_free(x.host);
    }
    for (auto p : L->slots) dev_free(p);
    for (auto ev : L->slot_free) (void)hipEventDestroy(ev);
    for (auto ev : L->slot_ready) (void)hipEventDestroy(ev);
    for (auto ev : L->batch_ready) (void)hipEventDestroy(ev);
    for (auto &mk : L->marks) {
        (void)hipEventDestroy(mk.a);
        (void)hipEventDestroy(mk.b);
    }
    for (auto ev : L->ev_pool) (void)hipEventDestroy(ev);
    for (auto p : L->pin_tables) host_free(p);
    for (auto p : L->dev_tables) dev_free(p);
    if (L->side) (void)hipStreamDestroy(L->side);
    void *ptrs[] = {L->wt, L->bias, L->table_dev, L->logits, L->h, L->xh, L->ys, L->chunks, L->n_chunks, L->err,
                    L->sync_counters, L->queues, L->union_blk, L->union_rank, L->units};
    for (void *p : ptrs) dev_free(p);
    host_free(L->pin_stage);
    host_free(L->pin_union);
    delete L;
}

coli_status ensure_stream_resources(coli_layer *L, int n_batches) {
    const size_t bytes = L->lay.total;
    if (!L->side) HIP_TRY(L, hipStreamCreateWithFlags(&L->side, hipStreamNonBlocking), "side stream");
    const int n_slots = std::max(kSlotCount, L->cache_slots);
    while (static_cast<int>(L->slots.size()) < n_slots) {
        uint8_t *p = nullptr;
        HIP_TRY(L, dev_alloc(&p, bytes), "staging slot");
        hipEvent_t ev = nullptr, rd = nullptr;
        if (hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming); e != hipSuccess) {
            dev_free(p);
            return hip_fail(L, e, "slot event");
        }
        if (hipError_t e = hipEventCreateWithFlags(&rd, hipEventDisableTiming); e != hipSuccess) {
            (void)hipEventDestroy(ev);
            dev_free(p);
            return hip_fail(L, e, "slot event");
        }
        L->slots.push_back(p);
        L->slot_expert.push_back(-1);
        L->slot_stamp.push_back(0);
        L->slot_free.push_back(ev);
        L->slot_ready.push_back(rd);
        L->slot_pending.push_back(0);
    }
    const size_t tbytes = sizeof(uint8_t *) * (L->d.n_experts + 1);
    while (static_cast<int>(L->dev_tables.size()) < n_batches) {
        void *hp = nullptr, *dp = nullptr;
        HIP_TRY(L, host_alloc(&hp, tbytes), "pinned table");
        if (hipError_t e = dev_alloc(&dp, tbytes); e != hipSuccess) {
            host_free(hp);
            return hip_fail(L, e, "device table");
        }
        L->pin_tables.push_back(static_cast<const uint8_t **>(hp));
        L->dev_tables.push_back(static_cast<const uint8_t **>(dp));
        hipEvent_t ev;
        HIP_TRY(L, hipEventCreateWithFlags(&ev, hipEventDisableTiming), "batch event");
        L->batch_ready.push_back(ev);
    }
    return COLI_OK;
}

// Scratch of one fused small-batch call: logits [n_tok x E], h and ys rows
// (n_tok * k routed + n_tok shared + the discard row), the arrival counters
// [1 + H/32] (zero at rest) and the unit descriptors [E + 1].
struct FusedScratch {
    float *logits;
    _Float16 *h;
    float *ys;
    int32_t *counters;
    int discard_row;
    UnitDesc *units;
};

// True when coli_moe_layer takes the fused small-batch path for n_tok.
bool fused_path(const coli_layer *L, int n_tok) {
    return n_tok <= kFrontMaxTok && L->d.n_experts <= 256 && all_routed_resident(L) &&
           choose_path(L, n_tok) == COLI_PATH_GEMV && L->router_set &&
           (!L->d.has_shared || L->experts[L->d.n_experts].tier == COLI_TIER_VRAM);
}

// The fused small-batch layer call in three launches: router + top-k + union
// with the shared expert's gate/up, the routed gate/up, and the down
// projection that also combines.  `timed` lets the launches carry kernel
// timestamps (coli_layer_set_timing); without it nothing is created.
coli_status run_fused(coli_layer *L, const FusedScratch &w, bool timed, const void *x, int n_tok,
                      int32_t *topk_idx, float *topk_w, int32_t *n_union, int32_t *union_ids, int32_t *counts,
                      int32_t *offsets, int32_t *gather, float *y, hipStream_t s) {
    FwdArgs a = make_args(L, x, n_tok, topk_w, n_union, union_ids, counts, offsets, gather, y);
    a.h = w.h;
    a.ys = w.ys;
    a.xh = nullptr;                      // the fp16 copy of x is a grouped-path buffer
    a.discard_row = w.discard_row;
    a.zero_row_x = a.zero_row_h = -1;    // (grouped path only)
    FrontArgs f{};
    f.wt = L->wt;
    f.bias = L->bias;
    f.logits = w.logits;
    f.topk_idx = topk_idx;
    f.topk_w = topk_w;
    f.n_union = n_union;
    f.union_ids = union_ids;
    f.counts = counts;
    f.offsets = offsets;
    f.gather = gather;
    f.counter = w.counters;
    f.next_counters = w.counters + 1;
    f.n_next = L->d.hidden / 32;
    f.units = w.units;
    f.n_units = std::min(n_tok * L->d.top_k, L->d.n_experts) + (L->d.has_shared ? 1 : 0);
    a.units = w.units;   // the expert launches read their units resolved
    coli_layer *Lt = timed ? L : nullptr;
    hipError_t e;
    {
        std::optional<KernelMark> m;
        if (Lt) m.emplace(Lt, COLI_K_ROUTER, s);
        if ((e = launch_decode_front(a, f, L->max_lds, s)) != hipSuccess) return hip_fail(L, e, "decode front launch");
    }
    {
        std::optional<KernelMark> m;
        if (Lt) m.emplace(Lt, COLI_K_GATEUP, s);
        FwdArgs ar = a;
        ar.skip_shared = 1;
        const int routed = std::min(n_tok * L->d.top_k, L->d.n_experts);
        if ((e = launch_gemv_gateup(ar, L->max_lds, s, 0, routed)) != hipSuccess)
            return hip_fail(L, e, "gemv gate/up launch");
    }
    std::optional<KernelMark> m;
    if (Lt) m.emplace(Lt, COLI_K_DOWN, s);
    if ((e = launch_gemv_down(a, L->max_lds, s, w.counters + 1, w.counters)) != hipSuccess)
        return hip_fail(L, e, "gemv down launch");
    return COLI_OK;
}

}  // namespace


extern "C" {

int32_t coli_abi_version(void) { return COLI_ABI_VERSION; }

coli_status coli_set_alloc_limit(int64_t bytes) {
    if (bytes < -1) return fail(nullptr, COLI_E_INVALID, "limit %lld: -1 or >= 0", static_cast<long long>(bytes));
    MemBook &b = mem_book();
    std::lock_guard<std::mutex> g(b.mu);
    b.limit = bytes;
    return COLI_OK;
}

int64_t coli_alloc_bytes(void) {
    MemBook &b = mem_book();
    std::lock_guard<std::mutex> g(b.mu);
    return b.used;
}

coli_status coli_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink) return fail(nullptr, COLI_E_INVALID, "NULL device pointer");
    if (bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
        return fail(nullptr, COLI_E_INVALID, "bytes (%zu) must be a multiple of 16 and buf 16-byte aligned", bytes);
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(nullptr, COLI_E_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
    if ((e = launch_probe_read(buf, bytes, sink, n_cu, static_cast<hipStream_t>(stream))) != hipSuccess)
        return fail(nullptr, COLI_E_DEVICE, "probe launch: %s", hipGetErrorString(e));
    return COLI_OK;
}

const char *coli_status_str(coli_status s) {
    switch (s) {
        case COLI_OK: return "COLI_OK";
        case COLI_E_INVALID: return "COLI_E_INVALID";
        case COLI_E_NOMEM: return "COLI_E_NOMEM";
        case COLI_E_DEVICE: return "COLI_E_DEVICE";
        case COLI_E_STATE: return "COLI_E_STATE";
        case COLI_E_UNSUPPORTED: return "COLI_E_UNSUPPORTED";
    }
    return "unknown coli_status";
}

const char *coli_last_error(const coli_layer *L) {
    return L ? L->msg.c_str() : g_create_error.c_str();
}

size_t coli_expert_blob_bytes(int32_t hidden, int32_t inter, int32_t group, int32_t weight_bits) {
    if (!group_supported(group) || !bits_supported(weight_bits) || hidden <= 0 || inter <= 0 ||
        hidden % group || inter % group)
        return 0;
    return blob_layout(hidden, inter, group, weight_bits).total;
}

coli_status coli_expert_repack(const void *blob_host, void *out_host, int32_t hidden, int32_t inter,
                               int32_t group, int32_t weight_bits) {
    if (!blob_host || !out_host) return fail(nullptr, COLI_E_INVALID, "NULL host pointer");
    if (hidden <= 0 || inter <= 0 || hidden % kChunkK || inter % kChunkK)
        return fail(nullptr, COLI_E_INVALID, "hidden and inter must be positive multiples of %d", kChunkK);
    if (!group_supported(group)) return fail(nullptr, COLI_E_INVALID, "group %d must be 32 or 64", group);
    if (!bits_supported(weight_bits)) return fail(nullptr, COLI_E_INVALID, "weight_bits %d must be 4 or 8", weight_bits);
    repack_blob(static_cast<const uint8_t *>(blob_host), static_cast<uint8_t *>(out_host), hidden, inter, group,
                weight_bits);
    return COLI_OK;
}

coli_status coli_layer_create(const coli_moe_dims *dims, int device, coli_layer **out) {
    std::string why;
    if (!out) return fail(nullptr, COLI_E_INVALID, "out is NULL");
    if (!dims_valid(dims, why)) return fail(nullptr, COLI_E_INVALID, "%s", why.c_str());
    if (!dims_supported(dims, why)) return fail(nullptr, COLI_E_UNSUPPORTED, "%s", why.c_str());
    if (!mem_fits(create_bytes(dims)))
        return fail(nullptr, COLI_E_NOMEM, "allocation cap: the layer needs %zu bytes", create_bytes(dims));
    int ndev = 0;
    hipError_t he = hipGetDeviceCount(&ndev);
    if (he != hipSuccess || ndev <= 0)
        return fail(nullptr, COLI_E_DEVICE, "no HIP device available (%s)", hipGetErrorString(he));
    if (device < 0 || device >= ndev) return fail(nullptr, COLI_E_INVALID, "device %d out of range", device);
    DeviceGuard guard(device);
    if (!guard.ok) return fail(nullptr, COLI_E_DEVICE, "cannot select device %d", device);
    hipDeviceProp_t prop;
    if ((he = hipGetDeviceProperties(&prop, device)) != hipSuccess)
        return fail(nullptr, COLI_E_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(he));

    coli_layer *L = new coli_layer();
    L->d = *dims;
    L->device = device;
    L->n_cu = prop.multiProcessorCount;
    L->max_lds = prop.sharedMemPerBlock;
    L->lay = blob_layout(dims->hidden, dims->inter, dims->group, dims->weight_bits);
    const int E = dims->n_experts, H = dims->hidden, I = dims->inter;
    const size_t T = static_cast<size_t>(dims->max_tokens);
    const size_t rows = T * dims->top_k + T;
    L->max_chunks = work_list_capacity(dims->max_tokens, dims->top_k, E, dims->has_shared);
    L->experts.resize(E + 1);
    L->expert_slot.assign(E, -1);
    L->table_host.assign(E + 1, nullptr);

    struct A { void **p; size_t n; const char *what; } allocs[] = {
        {reinterpret_cast<void **>(&L->wt), sizeof(float) * E * H, "router weight"},
        {reinterpret_cast<void **>(&L->bias), sizeof(float) * E, "router bias"},
        {reinterpret_cast<void **>(&L->table_dev), sizeof(void *) * (E + 1), "expert table"},
        {reinterpret_cast<void **>(&L->logits), sizeof(float) * T * E, "logits scratch"},
        {reinterpret_cast<void **>(&L->h), sizeof(_Float16) * (rows + 2) * I, "hidden scratch"},
        {reinterpret_cast<void **>(&L->xh), sizeof(_Float16) * (T + 1) * H, "fp16 activation scratch"},
        {reinterpret_cast<void **>(&L->ys), sizeof(float) * (rows + 1) * H, "per-entry output scratch"},
        {reinterpret_cast<void **>(&L->chunks), sizeof(ChunkDesc) * L->max_chunks, "work list"},
        {reinterpret_cast<void **>(&L->n_chunks), sizeof(int32_t), "work count"},
        {reinterpret_cast<void **>(&L->err), sizeof(int32_t), "error flags"},
        {reinterpret_cast<void **>(&L->sync_counters), sizeof(int32_t) * (1 + H / 32 + route_topk_counters()),
         "arrival counters"},
        {reinterpret_cast<void **>(&L->queues), sizeof(int32_t) * kQueueInts, "work-queue counters"},
        {reinterpret_cast<void **>(&L->union_blk), sizeof(int32_t) * (kUnionMaxBlocks * E + 64), "union slab counts"},
        {reinterpret_cast<void **>(&L->union_rank), sizeof(int32_t) * T * dims->top_k, "union ranks"},
        {reinterpret_cast<void **>(&L->units), sizeof(UnitDesc) * (E + 1), "unit descriptors"},
    };
    for (auto &a : allocs) {
        if ((he = dev_alloc(a.p, a.n)) != hipSuccess) {
            coli_status st = he == hipErrorOutOfMemory ? COLI_E_NOMEM : COLI_E_DEVICE;
            fail(nullptr, st, "hipMalloc %s (%zu bytes): %s", a.what, a.n, hipGetErrorString(he));
            free_layer(L);
            return st;
        }
    }
    if ((he = hipMemset(L->h + (rows + 1) * I, 0, sizeof(_Float16) * I)) != hipSuccess ||
        (he = hipMemset(L->xh + T * H, 0, sizeof(_Float16) * H)) != hipSuccess ||
        (he = hipMemset(L->table_dev, 0, sizeof(void *) * (E + 1))) != hipSuccess ||
        (he = hipMemset(L->err, 0, sizeof(int32_t))) != hipSuccess ||
        (he = hipMemset(L->sync_counters, 0, sizeof(int32_t) * (1 + H / 32 + route_topk_counters()))) != hipSuccess ||
        (he = hipMemset(L->queues, 0, sizeof(int32_t) * kQueueInts)) != hipSuccess ||
        (he = hipMemset(L->union_blk, 0, sizeof(int32_t) * (kUnionMaxBlocks * E + 64))) != hipSuccess ||
        (he = hipMemset(L->bias, 0, sizeof(float) * E)) != hipSuccess ||
        (he = host_alloc(&L->pin_stage, L->lay.total)) != hipSuccess ||
        (he = host_alloc(&L->pin_union, sizeof(int32_t) * (E + 1))) != hipSuccess ||
        (he = hipDeviceSynchronize()) != hipSuccess) {
        coli_status st = he == hipErrorOutOfMemory ? COLI_E_NOMEM : COLI_E_DEVICE;
        fail(nullptr, st, "layer setup: %s", hipGetErrorString(he));
        free_layer(L);
        return st;
    }
    void *static_ptr = nullptr;
    if ((he = static_scratch_setup(device, &static_ptr)) != hipSuccess) {
        fail(nullptr, COLI_E_DEVICE, "static scratch setup: %s", hipGetErrorString(he));
        free_layer(L);
        return COLI_E_DEVICE;
    }
    *out = L;
    return COLI_OK;
}

coli_status coli_layer_destroy(coli_layer *L) {
    if (!L) return COLI_OK;
    DeviceGuard guard(L->device);
    free_layer(L);
    return COLI_OK;
}

coli_status coli_layer_set_path(coli_layer *L, int32_t path) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    if (path < COLI_PATH_AUTO || path > COLI_PATH_GROUPED) return fail(L, COLI_E_INVALID, "bad path %d", path);
    if (path == COLI_PATH_GROUPED && L->d.weight_bits == 8)
        return fail(L, COLI_E_UNSUPPORTED, "int8 experts run on the GEMV path only");
    L->path = path;
    return COLI_OK;
}

coli_status coli_router_set(coli_layer *L, const float *w_host, const float *bias_host) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    if (!w_host) return fail(L, COLI_E_INVALID, "w_host is NULL");
    const int E = L->d.n_experts, H = L->d.hidden;
    std::vector<float> wt(static_cast<size_t>(E) * H);
    for (int k = 0; k < H; ++k)
        for (int e = 0; e < E; ++e) wt[static_cast<size_t>(e) * H + k] = w_host[static_cast<size_t>(k) * E + e];
    std::vector<float> b(E, 0.0f);
    if (bias_host) std::memcpy(b.data(), bias_host, sizeof(float) * E);
    DeviceGuard guard(L->device);
    // Work already queued on any stream may still read the old router.
    HIP_TRY(L, hipDeviceSynchronize(), "sync before the router update");
    HIP_TRY(L, hipMemcpy(L->wt, wt.data(), sizeof(float) * wt.size(), hipMemcpyHostToDevice), "router upload");
    HIP_TRY(L, hipMemcpy(L->bias, b.data(), sizeof(float) * E, hipMemcpyHostToDevice), "bias upload");
    L->router_set = true;
    return COLI_OK;
}

coli_status coli_expert_place(coli_layer *L, int32_t expert, const void *blob_host, size_t blob_bytes,
                              coli_tier tier) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    if (!blob_host) return fail(L, COLI_E_INVALID, "blob_host is NULL");
    if (expert != COLI_SHARED && (expert < 0 || expert >= L->d.n_experts))
        return fail(L, COLI_E_INVALID, "expert %d out of range", expert);
    if (expert == COLI_SHARED && !L->d.has_shared) return fail(L, COLI_E_INVALID, "layer has no shared expert");
    if (blob_bytes != L->lay.total)
        return fail(L, COLI_E_INVALID, "blob_bytes %zu != %zu", blob_bytes, L->lay.total);
    if (tier != COLI_TIER_VRAM && tier != COLI_TIER_HOST) return fail(L, COLI_E_INVALID, "bad tier %d", tier);
    if (expert == COLI_SHARED && tier != COLI_TIER_VRAM)
        return fail(L, COLI_E_INVALID, "the shared expert must be VRAM-resident");
    const int idx = expert == COLI_SHARED ? L->d.n_experts : expert;
    ExpertSlot &x = L->experts[idx];
    DeviceGuard guard(L->device);
    // Work already queued on any stream (caller streams, the side stream of
    // the tiered path, prefetch copies) may still read this expert's blob,
    // table entry or cached copy: let it finish before anything changes.
    HIP_TRY(L, hipDeviceSynchronize(), "sync before placement");
    const uint8_t *src = static_cast<const uint8_t *>(blob_host);
    if (tier == COLI_TIER_VRAM) {
        repack_blob(src, L->pin_stage, L->d.hidden, L->d.inter, L->d.group, L->d.weight_bits);
        if (!x.dev) HIP_TRY(L, dev_alloc(&x.dev, L->lay.total), "expert VRAM");
        HIP_TRY(L, hipMemcpy(x.dev, L->pin_stage, L->lay.total, hipMemcpyHostToDevice), "expert upload");
        if (x.host) {
            host_free(x.host);
            x.host = nullptr;
        }
        L->table_host[idx] = x.dev;
    } else {
        if (!x.host) HIP_TRY(L, host_alloc(&x.host, L->lay.total), "expert pinned host");
        repack_blob(src, x.host, L->d.hidden, L->d.inter, L->d.group, L->d.weight_bits);
        L->table_host[idx] = nullptr;
    }
    x.tier = tier;
    if (idx < L->d.n_experts && L->expert_slot[idx] >= 0) {   // a cached copy is stale now
        L->slot_expert[L->expert_slot[idx]] = -1;
        L->slot_pending[L->expert_slot[idx]] = 0;
        L->expert_slot[idx] = -1;
    }
    HIP_TRY(L, hipMemcpy(L->table_dev + idx, &L->table_host[idx], sizeof(void *), hipMemcpyHostToDevice), "table update");
    if (tier == COLI_TIER_HOST && x.dev) {
        HIP_TRY(L, hipDeviceSynchronize(), "sync before free");
        dev_free(x.dev);
        x.dev = nullptr;
    }
    return COLI_OK;
}

static coli_status check_tokens(coli_layer *L, int32_t n_tok) {
    if (n_tok < 0 || n_tok > L->d.max_tokens)
        return fail(L, COLI_E_INVALID, "n_tok %d outside [0, %d]", n_tok, L->d.max_tokens);
    return COLI_OK;
}

coli_status coli_moe_router_logits(coli_layer *L, const void *x, int32_t n_tok, float *logits, void *stream) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    coli_status st = check_tokens(L, n_tok);
    if (st != COLI_OK) return st;
    if (n_tok == 0) return COLI_OK;
    if (!x || !logits) return fail(L, COLI_E_INVALID, "NULL device pointer");
    if (!L->router_set) return fail(L, COLI_E_STATE, "router weight not set");
    DeviceGuard guard(L->device);
    KernelMark m(L, COLI_K_ROUTER, static_cast<hipStream_t>(stream));
    HIP_TRY(L, launch_router_logits(x, L->d.act == COLI_ACT_BF16, L->wt, L->bias, n_tok, L->d.hidden,
                                    L->d.n_experts, logits, static_cast<hipStream_t>(stream)),
            "router logits launch");
    return COLI_OK;
}

coli_status coli_moe_route(coli_layer *L, const void *x, int32_t n_tok, int32_t *topk_idx, float *topk_w,
                           void *stream) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    coli_status st = check_tokens(L, n_tok);
    if (st != COLI_OK) return st;
    if (n_tok == 0) return COLI_OK;
    if (!x || !topk_idx || !topk_w) return fail(L, COLI_E_INVALID, "NULL device pointer");
    if (!L->router_set) return fail(L, COLI_E_STATE, "router weight not set");
    DeviceGuard guard(L->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        // 3 to 128 tokens: router and top-k in one launch (counted as the router).
        KernelMark m(L, COLI_K_ROUTER, s);
        const hipError_t e = launch_router_topk(x, L->d.act == COLI_ACT_BF16, L->wt, L->bias, n_tok, L->d.hidden,
                                                L->d.n_experts, L->d.top_k, L->logits,
                                                L->sync_counters + 1 + L->d.hidden / 32, topk_idx, topk_w, s);
        if (e == hipSuccess) return COLI_OK;
        if (e != hipErrorNotSupported) return hip_fail(L, e, "router and top-k launch");
        (void)hipGetLastError();
        HIP_TRY(L, launch_router_logits(x, L->d.act == COLI_ACT_BF16, L->wt, L->bias, n_tok, L->d.hidden,
                                        L->d.n_experts, L->logits, s),
                "router logits launch");
    }
    KernelMark m(L, COLI_K_TOPK, s);
    HIP_TRY(L, launch_topk(L->logits, n_tok, L->d.n_experts, L->d.top_k, topk_idx, topk_w, s), "top-k launch");
    return COLI_OK;
}

// The union of a call.  Up to kUnionSmallEntries entries it is one launch;
// with `work` (the arguments of the forward that follows, grouped strategy)
// that launch also writes the work list and the fp16 copy of x, and
// *planned says so.
coli_status union_impl(coli_layer *L, const int32_t *topk_idx, int32_t n_tok, int32_t *n_union,
                       int32_t *union_ids, int32_t *counts, int32_t *offsets, int32_t *gather, hipStream_t s,
                       const FwdArgs *work, bool *planned) {
    if (planned) *planned = false;
    if (n_tok > 0 && n_tok * L->d.top_k <= kUnionSmallEntries) {
        KernelMark m(L, COLI_K_UNION, s);
        FwdArgs a{};
        if (work) a = *work;
        a.err = L->err;
        HIP_TRY(L, launch_union_small(topk_idx, n_tok, L->d.top_k, L->d.n_experts, n_union, union_ids, counts,
                                      offsets, gather, a, work ? L->chunks : nullptr, work ? L->n_chunks : nullptr,
                                      s),
                "union launch");
        if (planned) *planned = work != nullptr;
        return COLI_OK;
    }
    const UnionScratch ws{L->union_blk, L->union_blk + kUnionMaxBlocks * L->d.n_experts, L->union_rank};
    {
        KernelMark m(L, COLI_K_UNION, s);
        HIP_TRY(L, launch_union_rank(topk_idx, n_tok, L->d.top_k, L->d.n_experts, ws, n_union, union_ids, counts,
                                     offsets, L->err, s),
                "union launch");
    }
    KernelMark m(L, COLI_K_UNION, s);
    HIP_TRY(L, launch_union_scatter(topk_idx, n_tok, L->d.top_k, L->d.n_experts, ws, offsets, gather, s),
            "union scatter launch");
    return COLI_OK;
}

coli_status coli_moe_union(coli_layer *L, const int32_t *topk_idx, int32_t n_tok, int32_t *n_union,
                           int32_t *union_ids, int32_t *counts, int32_t *offsets, int32_t *gather,
                           void *stream) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    coli_status st = check_tokens(L, n_tok);
    if (st != COLI_OK) return st;
    if (!n_union || !union_ids || !counts || !offsets || (n_tok > 0 && (!topk_idx || !gather)))
        return fail(L, COLI_E_INVALID, "NULL device pointer");
    DeviceGuard guard(L->device);
    return union_impl(L, topk_idx, n_tok, n_union, union_ids, counts, offsets, gather,
                      static_cast<hipStream_t>(stream), nullptr, nullptr);
}

// The expert FFNs and the combine of one call whose routing and union are
// already on the device.  `planned`: the union launch also wrote the grouped
// work list and the fp16 copy of x (union_impl with a work list).
coli_status forward_impl(coli_layer *L, const void *x, int32_t n_tok, const float *topk_w,
                         const int32_t *n_union, const int32_t *union_ids, const int32_t *counts,
                         const int32_t *offsets, const int32_t *gather, float *y, hipStream_t s, bool planned) {
    coli_status st = COLI_OK;
    const int path = choose_path(L, n_tok);

    FwdArgs a = make_args(L, x, n_tok, topk_w, n_union, union_ids, counts, offsets, gather, y);

    L->last_streamed = 0;
    L->last_bytes = 0;
    L->last_hits = 0;
    std::vector<int> streamed;
    if (!all_routed_resident(L)) {
        // Read the union back to find the experts that are not in VRAM.
        const int E = L->d.n_experts;
        HIP_TRY(L, hipMemcpyAsync(L->pin_union, n_union, sizeof(int32_t), hipMemcpyDeviceToHost, s), "union readback");
        HIP_TRY(L, hipMemcpyAsync(L->pin_union + 1, union_ids, sizeof(int32_t) * E, hipMemcpyDeviceToHost, s),
                "union readback");
        HIP_TRY(L, hipStreamSynchronize(s), "union readback sync");
        const int nu = L->pin_union[0];
        if (nu < 0 || nu > E) return fail(L, COLI_E_INVALID, "n_union %d out of range", nu);
        for (int u = 0; u < nu; ++u) {
            const int e = L->pin_union[1 + u];
            if (e < 0 || e >= E) return fail(L, COLI_E_INVALID, "union id %d out of range", e);
            if (L->experts[e].tier < 0) return fail(L, COLI_E_STATE, "expert %d is routed to but not placed", e);
            if (L->experts[e].tier == COLI_TIER_HOST) streamed.push_back(e);
        }
    }

    // Host-tier experts already in the stream cache form the first batch (no
    // copy); the others are copied into slots in batches of kBatchExperts,
    // each batch computed once its copies have landed.  The slots, tables and
    // events are allocated before any launch, so a failed allocation leaves
    // no work behind.
    const bool cache = L->cache_slots > 0;
    std::vector<int> hits, misses;
    for (int e : streamed) (cache && L->expert_slot[e] >= 0 ? hits : misses).push_back(e);
    const int n_hit_batches = hits.empty() ? 0 : 1;
    const int n_batches = n_hit_batches + (static_cast<int>(misses.size()) + kBatchExperts - 1) / kBatchExperts;
    if (!streamed.empty() && (st = ensure_stream_resources(L, n_batches)) != COLI_OK) return st;

    if (path == COLI_PATH_GROUPED && !planned) {
        {
            KernelMark m(L, COLI_K_PLAN, s);
            HIP_TRY(L, launch_plan(a, L->chunks, L->n_chunks, s), "plan launch");
        }
        KernelMark m(L, COLI_K_PLAN, s);
        HIP_TRY(L, launch_to_half(a, s), "fp16 activation launch");
    }
    // Resident experts (the table holds NULL for pinned-host experts).
    if ((st = launch_experts(L, a, path, s)) != COLI_OK) return st;

    if (!streamed.empty()) {
        // Every earlier call ended with a stream synchronisation, so only
        // slots read earlier in this call, or filled by a prefetch, can
        // still be in use.
        const int64_t call = ++L->call_no;
        const int n_slots = cache ? L->cache_slots : kSlotCount;
        const size_t bytes = L->lay.total;
        const size_t tbytes = sizeof(uint8_t *) * (L->d.n_experts + 1);
        // Batch of this call that last read each slot (-1: none yet).
        std::vector<int> slot_batch(L->slots.size(), -1);
        // A slot for a copy in batch b: a slot not read yet in this call (the
        // least recently used one with the cache); when every slot was, the
        // one read earliest, never one of batch b itself (n_slots >=
        // kBatchExperts, so such a slot exists), after its kernels.
        auto pick_slot = [&](int b) {
            int best = -1;
            for (int q = 0; q < n_slots; ++q)
                if (slot_batch[q] < 0 && (best < 0 || (cache && L->slot_stamp[q] < L->slot_stamp[best]))) best = q;
            if (best >= 0) return best;
            for (int q = 0; q < n_slots; ++q)
                if (slot_batch[q] < b && (best < 0 || slot_batch[q] < slot_batch[best])) best = q;
            return best;
        };
        for (int b = 0; b < n_batches; ++b) {
            const uint8_t **pt = L->pin_tables[b];
            std::memset(pt, 0, tbytes);
            std::vector<int> batch_slots;
            if (b < n_hit_batches) {
                for (int e : hits) {
                    const int slot = L->expert_slot[e];
                    if (L->slot_pending[slot]) {     // filled by a prefetch: after its copy
                        HIP_TRY(L, hipStreamWaitEvent(s, L->slot_ready[slot], 0), "prefetch wait");
                        L->slot_pending[slot] = 0;
                    }
                    pt[e] = L->slots[slot];
                    slot_batch[slot] = b;
                    batch_slots.push_back(slot);
                }
            } else {
                const int first = (b - n_hit_batches) * kBatchExperts;
                const int last = std::min<int>(static_cast<int>(misses.size()), first + kBatchExperts);
                for (int i = first; i < last; ++i) {
                    const int e = misses[i];
                    const int slot = pick_slot(b);
                    if (slot_batch[slot] >= 0)       // read earlier in this call: after those kernels
                        HIP_TRY(L, hipStreamWaitEvent(L->side, L->slot_free[slot], 0), "slot wait");
                    if (L->slot_expert[slot] >= 0) L->expert_slot[L->slot_expert[slot]] = -1;
                    L->slot_expert[slot] = -1;
                    L->slot_pending[slot] = 0;     // a prefetch copy into it is ordered before this one
                    HIP_TRY(L, hipMemcpyAsync(L->slots[slot], L->experts[e].host, bytes, hipMemcpyHostToDevice,
                                              L->side),
                            "expert H2D");
                    if (cache) {
                        L->slot_expert[slot] = e;
                        L->expert_slot[e] = slot;
                    }
                    pt[e] = L->slots[slot];
                    slot_batch[slot] = b;
                    batch_slots.push_back(slot);
                    L->last_bytes += static_cast<int64_t>(bytes);
                }
                HIP_TRY(L, hipEventRecord(L->batch_ready[b], L->side), "batch event");
                HIP_TRY(L, hipStreamWaitEvent(s, L->batch_ready[b], 0), "batch wait");
            }
            HIP_TRY(L, hipMemcpyAsync(L->dev_tables[b], pt, tbytes, hipMemcpyHostToDevice, s), "batch table");
            FwdArgs ab = a;
            ab.table = L->dev_tables[b];
            if ((st = launch_experts(L, ab, path, s)) != COLI_OK) return st;
            for (int slot : batch_slots) {
                HIP_TRY(L, hipEventRecord(L->slot_free[slot], s), "slot event");
                L->slot_stamp[slot] = call;
            }
        }
        L->last_streamed = static_cast<int32_t>(misses.size());
        L->last_hits = static_cast<int32_t>(hits.size());
    }
    {
        KernelMark m(L, COLI_K_COMBINE, s);
        HIP_TRY(L, launch_combine(a, s), "combine launch");
    }
    if (!streamed.empty() || !all_routed_resident(L)) HIP_TRY(L, hipStreamSynchronize(s), "tiered forward sync");
    return COLI_OK;
}

coli_status coli_moe_forward(coli_layer *L, const void *x, int32_t n_tok, const int32_t *topk_idx,
                             const float *topk_w, const int32_t *n_union, const int32_t *union_ids,
                             const int32_t *counts, const int32_t *offsets, const int32_t *gather, float *y,
                             void *stream) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    coli_status st = check_tokens(L, n_tok);
    if (st != COLI_OK) return st;
    if (n_tok == 0) return COLI_OK;
    if (!x || !topk_idx || !topk_w || !n_union || !union_ids || !counts || !offsets || !gather || !y)
        return fail(L, COLI_E_INVALID, "NULL device pointer");
    if (L->d.has_shared && L->experts[L->d.n_experts].tier != COLI_TIER_VRAM)
        return fail(L, COLI_E_STATE, "shared expert not placed");
    DeviceGuard guard(L->device);
    return forward_impl(L, x, n_tok, topk_w, n_union, union_ids, counts, offsets, gather, y,
                        static_cast<hipStream_t>(stream), false);
}

coli_status coli_moe_layer(coli_layer *L, const void *x, int32_t n_tok, int32_t *topk_idx, float *topk_w,
                           int32_t *n_union, int32_t *union_ids, int32_t *counts, int32_t *offsets,
                           int32_t *gather, float *y, void *stream) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    coli_status st = check_tokens(L, n_tok);
    if (st != COLI_OK) return st;
    if (n_tok == 0) return COLI_OK;
    if (!x || !topk_idx || !topk_w || !n_union || !union_ids || !counts || !offsets || !gather || !y)
        return fail(L, COLI_E_INVALID, "NULL device pointer");
    if (!fused_path(L, n_tok)) {
        if (L->d.has_shared && L->experts[L->d.n_experts].tier != COLI_TIER_VRAM)
            return fail(L, COLI_E_STATE, "shared expert not placed");
        if ((st = coli_moe_route(L, x, n_tok, topk_idx, topk_w, stream)) != COLI_OK) return st;
        DeviceGuard guard(L->device);
        hipStream_t s = static_cast<hipStream_t>(stream);
        // A grouped call hands its work list and fp16 copy to the union launch.
        const FwdArgs work = make_args(L, x, n_tok, topk_w, n_union, union_ids, counts, offsets, gather, y);
        const bool grouped = choose_path(L, n_tok) == COLI_PATH_GROUPED;
        bool planned = false;
        if ((st = union_impl(L, topk_idx, n_tok, n_union, union_ids, counts, offsets, gather, s,
                             grouped ? &work : nullptr, &planned)) != COLI_OK)
            return st;
        return forward_impl(L, x, n_tok, topk_w, n_union, union_ids, counts, offsets, gather, y, s, planned);
    }
    DeviceGuard guard(L->device);
    const FusedScratch w{L->logits, L->h, L->ys, L->sync_counters,
                         static_cast<int>(L->d.max_tokens) * (L->d.top_k + 1), L->units};
    return run_fused(L, w, true, x, n_tok, topk_idx, topk_w, n_union, union_ids, counts, offsets, gather, y,
                     static_cast<hipStream_t>(stream));
}

coli_status coli_moe_layer_static(coli_layer *L, const void *x, int32_t n_tok, int32_t *topk_idx, float *topk_w,
                                  int32_t *n_union, int32_t *union_ids, int32_t *counts, int32_t *offsets,
                                  int32_t *gather, float *y, void *stream) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    coli_status st = check_tokens(L, n_tok);
    if (st != COLI_OK) return st;
    if (n_tok == 0) return COLI_OK;
    if (!x || !topk_idx || !topk_w || !n_union || !union_ids || !counts || !offsets || !gather || !y)
        return fail(L, COLI_E_INVALID, "NULL device pointer");
    // Layout of this call in the static scratch: counters first (the same
    // place for every call, zero at rest), then logits, h, ys, unit descriptors.
    const size_t H = static_cast<size_t>(L->d.hidden), I = static_cast<size_t>(L->d.inter);
    const size_t rows = static_cast<size_t>(n_tok) * (L->d.top_k + 1) + 1;   // + the discard row
    const size_t o_logits = align256(sizeof(int32_t) * (1 + H / 32));
    const size_t o_h = o_logits + align256(sizeof(float) * n_tok * L->d.n_experts);
    const size_t o_ys = o_h + align256(sizeof(_Float16) * rows * I);
    const size_t o_units = o_ys + align256(sizeof(float) * rows * H);
    const size_t need = o_units + sizeof(UnitDesc) * (L->d.n_experts + 1);
    if (need > kStaticScratchBytes)
        return fail(L, COLI_E_UNSUPPORTED, "this call needs %zu bytes of static scratch; the maximum is %zu",
                    need, kStaticScratchBytes);
    if (!fused_path(L, n_tok))
        return fail(L, COLI_E_UNSUPPORTED,
                    "the allocation-free call runs the fused small-batch path only: 1..%d tokens, <= 256 "
                    "experts all in VRAM, router set, GEMV strategy",
                    kFrontMaxTok);
    uint8_t *base = static_cast<uint8_t *>(static_scratch_ptr(L->device));
    if (!base) return fail(L, COLI_E_UNSUPPORTED, "no static scratch on device %d", L->device);
    DeviceGuard guard(L->device);
    const FusedScratch w{reinterpret_cast<float *>(base + o_logits), reinterpret_cast<_Float16 *>(base + o_h),
                         reinterpret_cast<float *>(base + o_ys), reinterpret_cast<int32_t *>(base),
                         static_cast<int>(rows) - 1, reinterpret_cast<UnitDesc *>(base + o_units)};
    return run_fused(L, w, false, x, n_tok, topk_idx, topk_w, n_union, union_ids, counts, offsets, gather, y,
                     static_cast<hipStream_t>(stream));
}

coli_status coli_layer_set_timing(coli_layer *L, int32_t enable) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    L->timing = enable != 0;
    return COLI_OK;
}

coli_status coli_layer_kernel_times(coli_layer *L, double *ms_total, int64_t *launches) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    DeviceGuard guard(L->device);
    HIP_TRY(L, hipDeviceSynchronize(), "sync");
    double t[COLI_KERNEL_KINDS] = {0};
    int64_t n[COLI_KERNEL_KINDS] = {0};
    for (auto &mk : L->marks) {
        float ms = 0.0f;
        HIP_TRY(L, hipEventElapsedTime(&ms, mk.a, mk.b), "event elapsed");
        t[mk.kind] += ms;
        n[mk.kind] += 1;
        L->ev_pool.push_back(mk.a);
        L->ev_pool.push_back(mk.b);
    }
    L->marks.clear();
    for (int k = 0; k < COLI_KERNEL_KINDS; ++k) {
        if (ms_total) ms_total[k] = t[k];
        if (launches) launches[k] = n[k];
    }
    return COLI_OK;
}

coli_status coli_layer_stream_stats(const coli_layer *L, int32_t *n_streamed, int64_t *bytes) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    if (n_streamed) *n_streamed = L->last_streamed;
    if (bytes) *bytes = L->last_bytes;
    return COLI_OK;
}

coli_status coli_layer_set_stream_cache(coli_layer *L, int32_t n_slots) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    if (n_slots != 0 && (n_slots < kBatchExperts || n_slots > L->d.n_experts))
        return fail(L, COLI_E_INVALID, "n_slots %d: 0 or %d..%d", n_slots, kBatchExperts, L->d.n_experts);
    DeviceGuard guard(L->device);
    // Prefetch copies may still be in flight into the slots; every tiered
    // forward call ended with a synchronisation.
    if (L->side) HIP_TRY(L, hipStreamSynchronize(L->side), "side stream sync");
    L->cache_slots = n_slots;
    // Slots past the new need are released.
    const size_t keep = static_cast<size_t>(std::max(kSlotCount, n_slots));
    while (L->slots.size() > keep) {
        dev_free(L->slots.back());
        (void)hipEventDestroy(L->slot_free.back());
        (void)hipEventDestroy(L->slot_ready.back());
        L->slots.pop_back();
        L->slot_free.pop_back();
        L->slot_ready.pop_back();
        L->slot_expert.pop_back();
        L->slot_stamp.pop_back();
        L->slot_pending.pop_back();
    }
    for (auto &x : L->slot_expert) x = -1;
    for (auto &x : L->slot_stamp) x = 0;
    for (auto &x : L->slot_pending) x = 0;
    for (auto &x : L->expert_slot) x = -1;
    return COLI_OK;
}

coli_status coli_layer_stream_hits(const coli_layer *L, int32_t *hits) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    if (!hits) return fail(const_cast<coli_layer *>(L), COLI_E_INVALID, "hits is NULL");
    *hits = L->last_hits;
    return COLI_OK;
}

coli_status coli_layer_prefetch_union(coli_layer *L, const int32_t *n_union, const int32_t *union_ids,
                                      void *stream, int32_t *n_started) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    if (!n_union || !union_ids) return fail(L, COLI_E_INVALID, "NULL device pointer");
    if (L->cache_slots <= 0) return fail(L, COLI_E_STATE, "prefetch needs the stream cache (coli_layer_set_stream_cache)");
    DeviceGuard guard(L->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int E = L->d.n_experts;
    if (n_started) *n_started = 0;
    coli_status st;
    if ((st = ensure_stream_resources(L, 0)) != COLI_OK) return st;
    HIP_TRY(L, hipMemcpyAsync(L->pin_union, n_union, sizeof(int32_t), hipMemcpyDeviceToHost, s), "union readback");
    HIP_TRY(L, hipMemcpyAsync(L->pin_union + 1, union_ids, sizeof(int32_t) * E, hipMemcpyDeviceToHost, s),
            "union readback");
    HIP_TRY(L, hipStreamSynchronize(s), "union readback sync");
    const int nu = L->pin_union[0];
    if (nu < 0 || nu > E) return fail(L, COLI_E_INVALID, "n_union %d out of range", nu);
    for (int u = 0; u < nu; ++u) {
        const int e = L->pin_union[1 + u];
        if (e < 0 || e >= E) return fail(L, COLI_E_INVALID, "union id %d out of range", e);
    }
    const int n_slots = L->cache_slots;
    const size_t bytes = L->lay.total;
    const int64_t stamp = ++L->call_no;
    int started = 0;
    for (int u = 0; u < nu; ++u) {
        const int e = L->pin_union[1 + u];
        if (L->experts[e].tier != COLI_TIER_HOST || L->expert_slot[e] >= 0) continue;
        // An empty slot, else the least recently used one; never a slot
        // filled by this call, nor one whose earlier prefetch copy is still
        // in flight.  None left: the rest of the union is not prefetched.
        int best = -1;
        for (int q = 0; q < n_slots; ++q) {
            if (L->slot_stamp[q] == stamp) continue;
            if (L->slot_pending[q]) {
                if (hipEventQuery(L->slot_ready[q]) != hipSuccess) continue;
                L->slot_pending[q] = 0;        // landed: no forward call needs to wait for it
            }
            if (best < 0 || (L->slot_expert[q] < 0 && L->slot_expert[best] >= 0) ||
                ((L->slot_expert[q] < 0) == (L->slot_expert[best] < 0) && L->slot_stamp[q] < L->slot_stamp[best]))
                best = q;
        }
        if (best < 0) break;
        if (L->slot_expert[best] >= 0) L->expert_slot[L->slot_expert[best]] = -1;
        HIP_TRY(L, hipMemcpyAsync(L->slots[best], L->experts[e].host, bytes, hipMemcpyHostToDevice, L->side),
                "prefetch H2D");
        HIP_TRY(L, hipEventRecord(L->slot_ready[best], L->side), "prefetch event");
        L->slot_expert[best] = e;
        L->expert_slot[e] = best;
        L->slot_stamp[best] = stamp;
        L->slot_pending[best] = 1;
        ++started;
    }
    if (n_started) *n_started = started;
    return COLI_OK;
}

coli_status coli_layer_device_errors(coli_layer *L, int32_t *flags) {
    if (!L) return fail(nullptr, COLI_E_INVALID, "layer is NULL");
    if (!flags) return fail(L, COLI_E_INVALID, "flags is NULL");
    DeviceGuard guard(L->device);
    HIP_TRY(L, hipDeviceSynchronize(), "sync");
    HIP_TRY(L, hipMemcpy(flags, L->err, sizeof(int32_t), hipMemcpyDeviceToHost), "error flag readback");
    HIP_TRY(L, hipMemset(L->err, 0, sizeof(int32_t)), "error flag clear");
    HIP_TRY(L, hipDeviceSynchronize(), "sync");
    return COLI_OK;
}

}  // extern "C"
