// gemv.hip -- decode-shaped expert FFN kernels (VALU GEMV work items from
// dev_gemv.h), one workgroup per (unit, panel) or (unit, panel pair), for a
// forward call whose routing was computed by earlier launches.
//
// The down kernel can also finish the layer: with a per-panel-pair arrival
// counter, the last workgroup to finish a panel pair (over all units) sums
// the k routed rows and the shared row of every token for those columns and
// writes y, so no separate combine launch is needed.
#include "dev_gemv.h"

namespace coli {
namespace {

template <class F, int MAXM>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(FwdArgs a, int u_begin) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int P = a.inter / kPanel;
    const int u = u_begin + blockIdx.x / P, p = blockIdx.x % P;
    int e, r0, M;
    if (!dev::resolve(a, u, e, r0, M)) return;
    if (a.skip_shared && e == a.n_experts) return;
    const uint8_t *blob = a.table[e];
    if (!blob || M <= 0) return;
    dev::gateup_panel<F, MAXM>(a, dev::PlainRows{a}, blob, r0, M, p, lds, dev::lds_address(lds));
}

template <class F, int MAXM, bool FUSED_COMBINE>
__global__ __launch_bounds__(256) void gemv_down_kernel(FwdArgs a, int32_t *counters) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int PG = a.hidden / (2 * kPanel);
    const int u = blockIdx.x / PG, pg = blockIdx.x % PG;
    int e, r0, M;
    if (!dev::resolve(a, u, e, r0, M)) return;
    const uint8_t *blob = a.table[e];
    if (blob && M > 0)
        dev::down_panelgroup<F, MAXM, FUSED_COMBINE>(a, dev::PlainRows{a}, blob, r0, M, pg, lds, dev::lds_address(lds),
                                                  dev::NoWait{});
    if (FUSED_COMBINE) {
        const int units = *a.n_union + (a.has_shared ? 1 : 0);
        // The last workgroup of the panel pair reuses its (now idle) LDS.
        if (dev::arrive_last(counters + pg, units))
            dev::combine_panelgroup(
                a, pg, reinterpret_cast<float *>(lds),
                static_cast<int>(dev::combine_lds_floats(dev::down_lds_bytes(MAXM, a.inter), a.k, a.has_shared)));
    }
}

int units_bound(const FwdArgs &a) {
    const int routed = a.n_tok * a.k < a.n_experts ? a.n_tok * a.k : a.n_experts;
    return routed + (a.has_shared ? 1 : 0);
}

int pick_maxm(int n_tok) { return n_tok >= 4 ? 4 : (n_tok >= 2 ? 2 : 1); }

template <class F>
void launch_gateup_as(const FwdArgs &a, int maxm, int grid, size_t lds, hipStream_t s, int u_begin) {
    if (maxm == 4) launch(gemv_gateup_kernel<F, 4>, grid, 256, lds, s, a, u_begin);
    else if (maxm == 2) launch(gemv_gateup_kernel<F, 2>, grid, 256, lds, s, a, u_begin);
    else launch(gemv_gateup_kernel<F, 1>, grid, 256, lds, s, a, u_begin);
}

template <class F>
void launch_down_as(const FwdArgs &a, int maxm, int grid, size_t lds, hipStream_t s, int32_t *combine_counters) {
    if (combine_counters) {
        if (maxm == 4) launch(gemv_down_kernel<F, 4, true>, grid, 256, lds, s, a, combine_counters);
        else if (maxm == 2) launch(gemv_down_kernel<F, 2, true>, grid, 256, lds, s, a, combine_counters);
        else launch(gemv_down_kernel<F, 1, true>, grid, 256, lds, s, a, combine_counters);
    } else {
        if (maxm == 4) launch(gemv_down_kernel<F, 4, false>, grid, 256, lds, s, a, nullptr);
        else if (maxm == 2) launch(gemv_down_kernel<F, 2, false>, grid, 256, lds, s, a, nullptr);
        else launch(gemv_down_kernel<F, 1, false>, grid, 256, lds, s, a, nullptr);
    }
}

}  // namespace

hipError_t launch_gemv_gateup(const FwdArgs &a, size_t max_lds, hipStream_t s, int u_begin, int u_count) {
    int maxm = pick_maxm(a.n_tok);
    while (maxm > 1 && dev::gateup_lds_bytes(maxm, a.hidden) > max_lds) maxm >>= 1;
    const size_t lds = dev::gateup_lds_bytes(maxm, a.hidden);
    if (lds > max_lds) return hipErrorInvalidValue;
    const int units = u_count >= 0 ? u_count : units_bound(a) - u_begin;
    if (units <= 0) return hipSuccess;
    const int grid = units * (a.inter / kPanel);
    dev::dispatch_format(a.lay.group, a.lay.bits,
                         [&](auto f) { launch_gateup_as<decltype(f)>(a, maxm, grid, lds, s, u_begin); });
    return hipGetLastError();
}

hipError_t launch_gemv_down(const FwdArgs &a, size_t max_lds, hipStream_t s, int32_t *combine_counters) {
    int maxm = pick_maxm(a.n_tok);
    while (maxm > 1 && dev::down_lds_bytes(maxm, a.inter) > max_lds) maxm >>= 1;
    size_t lds = dev::down_lds_bytes(maxm, a.inter);
    if (combine_counters) lds = sizeof(float) * dev::combine_lds_floats(lds, a.k, a.has_shared);
    if (lds > max_lds) return hipErrorInvalidValue;
    const int grid = units_bound(a) * (a.hidden / (2 * kPanel));
    dev::dispatch_format(a.lay.group, a.lay.bits,
                         [&](auto f) { launch_down_as<decltype(f)>(a, maxm, grid, lds, s, combine_counters); });
    return hipGetLastError();
}

}  // namespace coli
