// dev_common.h -- small device helpers shared by the kernel files.
#pragma once

#include "internal.h"

namespace coli {
namespace dev {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Load through a global-address-space pointer.  Expert weights are reached
// through pointers read from the device expert table, which the compiler
// cannot prove to be global; plain dereferences would become flat loads,
// which also count against the LDS wait counter and serialise LDS traffic
// behind the weight stream.
template <typename T>
__device__ __forceinline__ T gload(const void *p) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    if constexpr (sizeof(T) == 16) {
        const v4u v = *(const __attribute__((address_space(1))) v4u *)(p);
        return __builtin_bit_cast(T, v);
    } else if constexpr (sizeof(T) == 8) {
        const v2u v = *(const __attribute__((address_space(1))) v2u *)(p);
        return __builtin_bit_cast(T, v);
    } else {
        static_assert(sizeof(T) == 4, "gload: 4, 8 or 16 bytes");
        const uint32_t v = *(const __attribute__((address_space(1))) uint32_t *)(p);
        return __builtin_bit_cast(T, v);
    }
}

// Buffer loads: base and size in a resource descriptor (scalar registers),
// the per-lane offset in one vector register and the wave-uniform part of the
// offset in a scalar register, so a stream of loads needs no per-load vector
// address arithmetic.  Reads past `bytes` return zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}
// Cache policy of a buffer load: kLoadDefault, or kLoadStream (the nt bit,
// non-temporal) for data read exactly once, every byte of it by the
// instruction that fetches it -- the GEMV weight and scale streams: they then
// do not displace the data the L2 serves again (measured: decode B=1 layer
// call 52.0 -> 49 us).  The grouped GEMMs read each 16-byte weight slot in two
// halves one K step apart and keep the default (with nt they ran 25% slower).
constexpr int kLoadDefault = 0;
constexpr int kLoadStream = 2;

template <typename T, int AUX = kLoadDefault>
__device__ __forceinline__ T bload(rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (sizeof(T) == 16) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                                                           static_cast<int>(soff), AUX));
    } else if constexpr (sizeof(T) == 8) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(voff),
                                                                          static_cast<int>(soff), AUX));
    } else {
        static_assert(sizeof(T) == 4, "bload: 4, 8 or 16 bytes");
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff),
                                                                          static_cast<int>(soff), AUX));
    }
}

// SwiGLU of one gate/up pair, silu(g) * v = g * v / (1 + e^-g), with e^-g as
// 2^(-g log2 e) on the hardware base-2 exponential and the quotient through
// the hardware reciprocal (each about one ulp in fp32; h is then rounded to
// fp16, whose step is 2^11 ulp of fp32).  Large negative g gives e^-g = inf,
// reciprocal 0 and h = -0 or 0, the limit of the exact function.
__device__ __forceinline__ float swiglu(float g, float v) {
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * v;
}

// True when v is NaN or rounds to an infinite fp16 (|v| >= 65520, the
// midpoint between the largest half, 65504, and 2^16).
__device__ __forceinline__ bool outside_half(float v) { return !(__builtin_fabsf(v) < 65520.0f); }

// True when an fp16 value is inf or NaN (all exponent bits set): the result
// of rounding a value outside the fp16 range, or of a non-finite input.
__device__ __forceinline__ bool half_nonfinite(_Float16 h) {
    return (__builtin_bit_cast(uint16_t, h) & 0x7C00u) == 0x7C00u;
}

// Sets `bit` in the device error flags when `bad` holds in any active lane
// of the wave: one atomic from the lowest such lane, and none in the usual
// case.  Call it where the lanes that matter are active.
__device__ __forceinline__ void flag_if(bool bad, int32_t *err, int32_t bit) {
    const uint64_t m = __ballot(bad);
    if (__builtin_expect(m != 0, 0) && __lane_id() == static_cast<unsigned>(__ffsll(static_cast<unsigned long long>(m)) - 1))
        __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fp16 copy of the 8 activations x[8i .. 8i+7] (bf16 or fp32) into xh, the A
// operand of the grouped gate/up GEMM; values outside the fp16 range set a
// device error flag.  Threads with i >= n8 do nothing.
__device__ __forceinline__ void to_half8(const void *x, int act_bf16, size_t i, size_t n8, _Float16 *xh,
                                         int32_t *err) {
    if (i >= n8) return;
    typedef _Float16 half8x __attribute__((ext_vector_type(8)));
    float v[8];
    if (act_bf16) {
        const uint4 raw = reinterpret_cast<const uint4 *>(x)[i];
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float((w4[j] & 0xFFFFu) << 16);
            v[2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
        }
    } else {
        const float4 lo = reinterpret_cast<const float4 *>(x)[2 * i];
        const float4 hi = reinterpret_cast<const float4 *>(x)[2 * i + 1];
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    }
    half8x h;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        h[j] = static_cast<_Float16>(v[j]);
        bad = bad || outside_half(v[j]);
    }
    reinterpret_cast<half8x *>(xh)[i] = h;
    flag_if(bad, err, kErrActRange);
}

// Wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6); }

// Thread index the optimiser cannot hoist computations of out of a
// persistent loop (keeps per-item address math from holding registers).
__device__ __forceinline__ int opaque_tid() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h16)));
}

// Keeps a constant in a VGPR so the compiler can use three-operand
// v_and_or_b32 (VOP3 cannot encode literals on this ISA).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
    asm volatile("" : "+v"(c));
    return c;
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c, false);
}

// Load through the scalar data cache: a wave-uniform address read as
// constant memory becomes s_load, which waits on its own counter (not behind
// vector loads in flight) and skips the vector cache path.  Only for data no
// workgroup of the running launch writes (the routing arrays, written by
// earlier launches; the scalar cache is invalidated at every launch).
template <typename T>
__device__ __forceinline__ T ld_uniform(const T *p) {
    return *(const __attribute__((address_space(4))) T *)(p);
}

// Work unit u of a forward call: routed union entry (u < n_union) or the
// shared expert (u == n_union), with its blob pointer.  Returns false when u
// is past the last unit.  With a.units (a fused small-batch call) the unit
// comes resolved; otherwise the loads come in two rounds, not four: the union
// size and the union entry at u are read together (the entry speculatively,
// at an in-range index), then the entry's offset, count and blob together.
// u must be wave-uniform and the routing arrays written by earlier launches.
__device__ __forceinline__ bool resolve(const FwdArgs &a, int u, int &e, int &r0, int &m, const uint8_t *&blob) {
    if (a.units) {
        // Resolved by the decode front: one round of scalar loads.
        typedef int32_t int8v __attribute__((ext_vector_type(8)));
        const UnitDesc d = __builtin_bit_cast(UnitDesc, ld_uniform(reinterpret_cast<const int8v *>(a.units + u)));
        if (d.m < 0) return false;
        e = d.e;
        r0 = d.r0;
        m = d.m;
        blob = d.blob;
        return true;
    }
    const int E = a.n_experts;
    const int nu = ld_uniform(a.n_union);
    const int es = ld_uniform(a.union_ids + (u < E ? u : E - 1));
    asm volatile("" ::"s"(nu), "s"(es));   // both loads issued before the first use
    const bool routed = u < nu;
    if (!routed && !(u == nu && a.has_shared)) return false;
    const int ec = routed ? (es >= 0 && es < E ? es : 0) : 0;
    const int r0s = ld_uniform(a.offsets + ec), ms = ld_uniform(a.counts + ec);
    e = routed ? ec : E;
    blob = ld_uniform(a.table + e);
    r0 = routed ? r0s : a.n_tok * a.k;
    m = routed ? ms : a.n_tok;
    return true;
}

// Token of hidden-buffer row `row`: routed rows are in gather order, shared
// rows follow at n_tok*k + t.
__device__ __forceinline__ int token_of_row(const FwdArgs &a, int row) {
    if (a.n_tok == 1) return 0;   // one token: no lookup
    const int routed = a.n_tok * a.k;
    return row < routed ? ld_uniform(a.gather + row) / a.k : row - routed;
}

// Monotonic unsigned key of a finite float (larger float -> larger key);
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t float_key(float f) {
    const uint32_t b = __float_as_uint(f + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// LDS byte address of a __shared__ array (pass the array itself, not a
// pointer computed at run time, so the conversion folds to a constant).
template <typename T>
__device__ __forceinline__ uint32_t lds_address(T *shared_array) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) T *)(shared_array))));
}

// Direct global -> LDS copy of 16 bytes per lane: lane L's bytes land at
// LDS byte address lds_addr + 16 L (lds_addr wave-uniform; it goes to M0).
// Written as inline asm so that the compiler's wait insertion does not see an
// LDS write in flight: it would otherwise make every LDS read wait for all
// copies, including the lookahead stages.  The caller waits for a stage's
// copies explicitly (s_waitcnt vmcnt) before reading it; the copy has no
// output register, and its address operands are consumed at issue.
__device__ __forceinline__ void copy16_to_lds(const void *src, uint32_t lds_addr) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_addr) : "memory");
}

// Exclusive scan of one int per thread over a block of NT threads; *total
// gets the sum.  s_tmp needs NT/64 + 1 ints.  Contains __syncthreads().
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_tmp, int *total) {
    constexpr int kWaves = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) s_tmp[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int wv = lane < kWaves ? s_tmp[lane] : 0;
        int inc = wv;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        if (lane < kWaves) s_tmp[lane] = inc - wv;
        if (lane == kWaves - 1) s_tmp[kWaves] = inc;
    }
    __syncthreads();
    const int excl = s_tmp[wave] + x - v;
    *total = s_tmp[kWaves];
    __syncthreads();
    return excl;
}

// Device-coherent store / load of data handed from one workgroup to another
// inside a launch.  Relaxed atomics at agent scope compile to plain global
// stores/loads with the device-coherence bit (sc1): they bypass the per-XCD
// L2 without the whole-cache writeback and invalidate that a fence costs.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent(const int32_t *p) {
    return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(_Float16 *p, _Float16 v) {
    __hip_atomic_store(reinterpret_cast<uint16_t *>(p), __builtin_bit_cast(uint16_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true in exactly one workgroup: the last of `expected` workgroups
// to arrive at `counter` (which it resets to 0 for the next launch).  The
// data a workgroup hands over must have been written with store_coherent and
// must be read with load_coherent: each wave waits for its stores to complete
// before the workgroup arrives, so the last workgroup finds all of them.
// All threads of the workgroup must call it.
__device__ __forceinline__ bool arrive_last(int32_t *counter, int expected) {
    __shared__ int s_last;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == expected - 1) ? 1 : 0;
        if (s_last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return s_last != 0;
}

}  // namespace dev
}  // namespace coli
