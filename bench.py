"""Benchmark of one int4 routed-expert MoE layer on one MI355X.

A step is one full pass of the layer (route -> union -> expert FFNs ->
combine) over one batch of synthetic tokens, through the C ABI.  The headline
workload is single-token decode: H=6144, I=2048, 256 routed experts (top-8)
plus one shared expert, int4 weights with fp16 group-32 scales, all experts in
VRAM.  To keep the 256 MB last-level cache from serving weights, steps rotate
over several layer instances (distinct copies of the experts), so every step
streams its experts from HBM.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (% peak) at decode B=1/64; prefill MFMA %"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def fused_decode(spec):
    """coli_moe_layer's small-batch path: the shared expert's gate/up runs in
    the router launch, so the gate/up kernel streams the routed experts only."""
    return spec.n_tok <= 4 and spec.n_experts <= 256


def algorithmic_bytes(spec, n_union, n_tok):
    """Bytes one layer call must move at minimum: each union expert's blob
    once, the shared expert's blob, the router weight, activations in, output
    out; and the share of them each expert kernel streams."""
    from int4_routed_expert_layer_amd import configs
    blob = configs.blob_bytes(spec.hidden, spec.inter, spec.group, spec.bits)
    experts = n_union + (1 if spec.has_shared else 0)
    h, i, g, b = spec.hidden, spec.inter, spec.group, spec.bits
    gu_experts = n_union if (fused_decode(spec) and spec.has_shared) else experts
    gateup = gu_experts * (2 * i * h * b // 8 + 2 * i * (h // g) * 2)
    down = experts * (h * i * b // 8 + h * (i // g) * 2)
    router = h * spec.n_experts * 4
    act = n_tok * h * spec.act_bytes + n_tok * h * 4
    return dict(total=experts * blob + router + act, gateup=gateup, down=down, router=router)


def expert_flops(spec, n_tok):
    rows = n_tok * spec.top_k + (n_tok if spec.has_shared else 0)
    return 2.0 * rows * 3 * spec.hidden * spec.inter


class Workload:
    def __init__(self, name, spec, layers, steps, warmup, graph_steps):
        self.name, self.spec, self.layers = name, spec, layers
        self.steps, self.warmup, self.graph_steps = steps, warmup, graph_steps


def make_layers(B, spec, blobs, shared, n_inst, max_tokens, w, b):
    layers = []
    for r in range(n_inst):
        L = B.MoELayer.from_spec(spec, max_tokens=max_tokens)
        L.set_router(w, b)
        for e in range(spec.n_experts):
            L.place(e, blobs[e])
        if shared is not None:
            L.place(B.SHARED, shared)
        layers.append(L)
        log(f"  layer instance {r + 1}/{n_inst} placed")
    return layers


def run_workload(B, torch, wl, x_all, use_graph=True):
    """Time `steps` steps; returns timing, union sizes and per-kernel times."""
    spec, layers = wl.spec, wl.layers
    n_tok = spec.n_tok
    R = len(layers)
    n_slices = x_all.shape[0] // n_tok
    dev = "cuda:0"
    k, E, H = spec.top_k, spec.n_experts, spec.hidden

    # Static buffers, one set per (instance) so graph replays reuse addresses.
    bufs = []
    for r in range(R):
        bufs.append(dict(
            idx=torch.empty((n_tok, k), dtype=torch.int32, device=dev),
            w=torch.empty((n_tok, k), dtype=torch.float32, device=dev),
            n_union=torch.empty(1, dtype=torch.int32, device=dev),
            union_ids=torch.empty(E, dtype=torch.int32, device=dev),
            counts=torch.empty(E, dtype=torch.int32, device=dev),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            gather=torch.empty(n_tok * k, dtype=torch.int32, device=dev),
            y=torch.empty((n_tok, H), dtype=torch.float32, device=dev)))

    C = B.C
    lib = B.lib

    def step(s):
        r = s % R
        L, bf = layers[r], bufs[r]
        x = x_all[(s % n_slices) * n_tok:(s % n_slices + 1) * n_tok]
        st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        p = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731
        B._check(lib.coli_moe_layer(L.handle, p(x), n_tok, p(bf["idx"]), p(bf["w"]), p(bf["n_union"]),
                                    p(bf["union_ids"]), p(bf["counts"]), p(bf["offsets"]),
                                    p(bf["gather"]), p(bf["y"]), st), L.handle)
        return bf

    # 1) eager pass with per-kernel events (roofline of the dominant kernel).
    # A bounded GPU sleep is queued first so the host has enqueued every step
    # before the GPU reaches them: kernels then run back to back and each
    # event pair brackets its kernel without host gaps.
    for s in range(wl.warmup):
        step(s)
    torch.cuda.synchronize()
    for L in layers:
        L.kernel_times()
        L.set_timing(True)
    unions = []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(wl.steps + 1)]   # one per step boundary
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * max(0.02, 1e-4 * wl.steps)))   # ~20+ ms of GPU clock cycles
    for s in range(wl.steps):
        evs[s].record()
        bf = step(s)
    evs[-1].record()
    torch.cuda.synchronize()
    eager_ms = evs[0].elapsed_time(evs[-1]) / wl.steps
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(wl.steps)]
    kt = {}
    for L in layers:
        L.set_timing(False)
        for kind, (ms, n) in L.kernel_times().items():
            a = kt.setdefault(kind, [0.0, 0])
            a[0] += ms
            a[1] += n
    # union sizes over one rotation of inputs
    for s in range(min(wl.steps, n_slices)):
        bf = step(s)
        unions.append(int(bf["n_union"].cpu()[0]))
    torch.cuda.synchronize()

    # Kernel time per step (a kind may launch more than once per step).
    res = dict(eager_ms_per_step=eager_ms, eager_ms_p50=float(np.median(per_step)),
               eager_ms_p90=float(np.percentile(per_step, 90)),
               kernel_ms={k_: v[0] / wl.steps for k_, v in kt.items() if v[1]},
               kernel_launches={k_: v[1] / wl.steps for k_, v in kt.items() if v[1]},
               union_mean=float(np.mean(unions)), union_min=int(np.min(unions)),
               union_max=int(np.max(unions)))

    # 2) graph pass: capture G steps once, replay it `steps // G` times
    if use_graph:
        G = max(1, min(wl.graph_steps, wl.steps))
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step(0)   # warm the capture stream
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for s in range(G):
                step(s)
        reps = max(1, wl.steps // G)
        for _ in range(max(1, wl.warmup // G)):
            g.replay()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        res["graph_ms_per_step"] = ev0.elapsed_time(ev1) / (reps * G)
        res["graph_steps_timed"] = reps * G
    return res


def hbm_reference(B, torch, reps=5):
    """Streaming rates on this GPU, as a reference for the expert kernels'
    bandwidth: the library's plain read (coli_probe_read, 16-byte loads) over
    2 GiB, torch's sum over 2 GiB of fp32 (reads only) and a 1 GiB
    device-to-device copy (read + write bytes), best of `reps`.  All sizes
    are far above the 256 MB last-level cache.  Run before the layers are
    placed."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    src = torch.ones(512 << 20, dtype=torch.float32, device="cuda:0")
    out = {}
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    best = 0.0
    for _ in range(reps):
        torch.cuda.synchronize()
        ev0.record()
        B.probe_read(src, sink)
        ev1.record()
        torch.cuda.synchronize()
        best = max(best, src.numel() * 4 / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
    out["stream_read_GBs"] = best
    best = 0.0
    for _ in range(reps):
        torch.cuda.synchronize()
        ev0.record()
        src.sum()
        ev1.record()
        torch.cuda.synchronize()
        best = max(best, src.numel() * 4 / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
    out["sum_read_GBs"] = best
    del src
    a = torch.ones(256 << 20, dtype=torch.float32, device="cuda:0")
    bdst = torch.empty_like(a)
    best = 0.0
    for _ in range(reps):
        torch.cuda.synchronize()
        ev0.record()
        bdst.copy_(a)
        ev1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * a.numel() * 4 / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
    out["copy_read_write_GBs"] = best
    del a, bdst
    torch.cuda.empty_cache()
    return out


def mfma_reference(torch, sizes=(8192, 16384), reps=5):
    """Dense matrix-core rate of the platform's own GEMM (torch.matmul on
    hipBLASLt) for fp16 and bf16 n x n x n products, the best over `sizes`
    and `reps`: the achievable figure beside the 2.5 PFLOP/s nominal peak."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for name, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        for n in sizes:
            a = torch.randn(n, n, device="cuda:0").to(dt).contiguous()
            b = torch.randn(n, n, device="cuda:0").to(dt).contiguous()
            c = torch.matmul(a, b)
            best = 0.0
            for _ in range(reps):
                torch.cuda.synchronize()
                ev0.record()
                torch.matmul(a, b, out=c)
                ev1.record()
                torch.cuda.synchronize()
                best = max(best, 2.0 * n ** 3 / (ev0.elapsed_time(ev1) / 1e3) / 1e12)
            out[f"{name}_{n}_TFLOPs"] = best
            out[f"{name}_TFLOPs"] = max(out.get(f"{name}_TFLOPs", 0.0), best)
            del a, b, c
            torch.cuda.empty_cache()
    out["shapes"] = " and ".join(f"{n} x {n} x {n}" for n in sizes) + ", torch.matmul (hipBLASLt)"
    return out


def run_stack(B, torch, blobs, shared, steps=8, warmup=2, cache_slots=48):
    """The tiered 12-layer stack (the a7 step and its placement policy):
    12 layers of the decode shape, each with its own seeded router (Zipf
    popularity), inputs and tier mask (a seeded 154 of 256 experts in VRAM,
    the rest in pinned host memory).  A step runs one batch of 16 tokens
    through the 12 layers in order.  Flows, each timed over `steps` steps by
    the host clock around the step (a tiered call synchronises):
      stream     every host-tier expert of a union is copied per call;
      cache      each layer keeps up to `cache_slots` host-tier experts in VRAM
                 between calls (least recently used replaced);
      lookahead  cache, plus: before layer l runs, layer l+1's route and
                 union are computed on a second stream and its host-tier
                 experts prefetched (coli_layer_prefetch_union), so their
                 copies overlap layer l;
      all_vram   every expert in VRAM (the same layers, re-placed).
    Expert contents are the decode workload's for every layer (timing does
    not depend on them); each layer holds its own copies."""
    from int4_routed_expert_layer_amd import configs, inputs
    spec = configs.TIERED_12L
    n_tok, NL, E, H = spec.n_tok, spec.n_layers, spec.n_experts, spec.hidden
    n_batches = steps + warmup
    layers, xs, masks = [], [], []
    for li in range(NL):
        L = B.MoELayer.from_spec(spec, max_tokens=n_tok)
        L.set_router(inputs.router_weight(spec, li), inputs.router_bias(spec, li))
        mask = inputs.resident_mask(spec, li)
        for e in range(E):
            L.place(e, blobs[e], B.TIER_VRAM if mask[e] else B.TIER_HOST)
        L.place(B.SHARED, shared)
        layers.append(L)
        masks.append(mask)
        xs.append(B.activations_to_device(inputs.activations(spec, li, n_tok * n_batches)))
        log(f"  stack layer {li + 1}/{NL} placed ({int(mask.sum())} resident)")
    blob = configs.blob_bytes(spec.hidden, spec.inter, spec.group, spec.bits)
    main = torch.cuda.current_stream()
    ahead = torch.cuda.Stream()

    def bufs():
        return dict(idx=torch.empty((n_tok, spec.top_k), dtype=torch.int32, device="cuda:0"),
                    w=torch.empty((n_tok, spec.top_k), dtype=torch.float32, device="cuda:0"),
                    u=dict(n_union=torch.empty(1, dtype=torch.int32, device="cuda:0"),
                           union_ids=torch.empty(E, dtype=torch.int32, device="cuda:0"),
                           counts=torch.empty(E, dtype=torch.int32, device="cuda:0"),
                           offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda:0"),
                           gather=torch.empty(n_tok * spec.top_k, dtype=torch.int32, device="cuda:0")),
                    y=torch.empty((n_tok, H), dtype=torch.float32, device="cuda:0"))
    rb = [bufs() for _ in range(NL)]
    C, lib = B.C, B.lib
    p = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731

    def route(li, b, stream):
        L, r = layers[li], rb[li]
        x = xs[li][b * n_tok:(b + 1) * n_tok]
        st = C.c_void_p(stream.cuda_stream)
        u = r["u"]
        B._check(lib.coli_moe_route(L.handle, p(x), n_tok, p(r["idx"]), p(r["w"]), st), L.handle)
        B._check(lib.coli_moe_union(L.handle, p(r["idx"]), n_tok, p(u["n_union"]), p(u["union_ids"]),
                                    p(u["counts"]), p(u["offsets"]), p(u["gather"]), st), L.handle)

    def forward(li, b):
        L, r = layers[li], rb[li]
        x = xs[li][b * n_tok:(b + 1) * n_tok]
        u = r["u"]
        B._check(lib.coli_moe_forward(L.handle, p(x), n_tok, p(r["idx"]), p(r["w"]), p(u["n_union"]),
                                      p(u["union_ids"]), p(u["counts"]), p(u["offsets"]), p(u["gather"]),
                                      p(r["y"]), C.c_void_p(main.cuda_stream)), L.handle)

    def flow(kind):
        times, streamed, hits, prefetched, host_union, unions = [], 0, 0, 0, 0, []
        for b in range(n_batches):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            st = dict(streamed=0, hits=0, prefetched=0)
            if kind == "lookahead":
                route(0, b, main)
            for li in range(NL):
                if kind == "lookahead":
                    if li + 1 < NL:
                        route(li + 1, b, ahead)
                        with torch.cuda.stream(ahead):
                            st["prefetched"] += layers[li + 1].prefetch_union(rb[li + 1]["u"])
                else:
                    route(li, b, main)
                forward(li, b)
                n, _ = layers[li].stream_stats()
                st["streamed"] += n
                st["hits"] += layers[li].stream_hits()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            if b >= warmup:
                times.append((t1 - t0) * 1e3)
                streamed += st["streamed"]
                hits += st["hits"]
                prefetched += st["prefetched"]
                for li in range(NL):
                    nu = int(rb[li]["u"]["n_union"].cpu()[0])
                    ids = rb[li]["u"]["union_ids"].cpu().numpy()[:nu]
                    unions.append(nu)
                    host_union += int(np.sum(~masks[li][ids]))
        ms = float(np.median(times))
        copied = (streamed + prefetched) * blob / steps
        out = dict(ms_per_step=ms, ms_p90=float(np.percentile(times, 90)),
                   tokens_per_s=n_tok / (ms / 1e3), union_mean=float(np.mean(unions)),
                   host_experts_per_step=host_union / steps,
                   copied_experts_per_step=(streamed + prefetched) / steps,
                   pcie_MB_per_step=copied / 1e6, pcie_GBs=copied / (ms / 1e3) / 1e9)
        if kind != "stream":
            out["hit_rate"] = hits / max(1, host_union)
        if kind == "lookahead":
            out["prefetched_experts_per_step"] = prefetched / steps
        return out

    res = {}
    log("  stack: stream")
    res["stream"] = flow("stream")
    for L in layers:
        L.set_stream_cache(cache_slots)
    log("  stack: cache")
    res["cache"] = flow("cache")
    for L in layers:
        L.set_stream_cache(0)
        L.set_stream_cache(cache_slots)        # empty cache: the lookahead starts cold too
    log("  stack: lookahead")
    res["lookahead"] = flow("lookahead")
    for L in layers:
        L.set_stream_cache(0)
    log("  stack: moving the host tier to VRAM")
    for li, L in enumerate(layers):
        for e in range(E):
            if not masks[li][e]:
                L.place(e, blobs[e], B.TIER_VRAM)
    res["all_vram"] = flow("stream")
    for L in layers:
        L.close()
    # plain pinned-host -> device copy rate at one expert blob per copy
    src = torch.empty(blob * 4, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(blob * 4, dtype=torch.uint8, device="cuda:0")
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    h2d = blob * 4 * 5 / (time.perf_counter() - t0) / 1e9
    del src, dst
    # Overlap: time the copies alone would take at the plain rate, plus the
    # all-VRAM step, against the measured step; 100% = fully hidden.
    t_vram = res["all_vram"]["ms_per_step"]
    resident_bytes = (res["all_vram"]["union_mean"] + 1) * blob + H * E * 4
    res["all_vram"]["hbm_GBs"] = NL * resident_bytes / (t_vram / 1e3) / 1e9
    for k in ("stream", "cache", "lookahead"):
        r = res[k]
        t_copy = r["pcie_MB_per_step"] * 1e6 / (h2d * 1e9) * 1e3
        r["ms_copy_at_plain_rate"] = t_copy
        hidden = t_copy + t_vram - r["ms_per_step"]
        r["overlap_pct"] = 100.0 * max(0.0, hidden) / max(1e-9, min(t_copy, t_vram))
        res_bytes = NL * ((r["union_mean"] + 1) * blob - r["host_experts_per_step"] / NL * blob + H * E * 4)
        r["resident_hbm_GBs"] = res_bytes / (r["ms_per_step"] / 1e3) / 1e9
    res.update(layers=NL, tokens_per_step=n_tok, steps=steps, cache_slots=cache_slots,
               resident_per_layer=int(masks[0].sum()), h2d_copy_GBs=h2d,
               timing="host clock around each 12-layer step (tiered calls synchronise); median over steps")
    return res


KERNEL_SOURCES = ["int4_routed_expert_layer_amd/csrc/dev_gemv.h", "int4_routed_expert_layer_amd/csrc/gemv.hip",
                  "int4_routed_expert_layer_amd/csrc/dev_common.h", "int4_routed_expert_layer_amd/csrc/internal.h"]


def kernel_source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the gate/up GEMV from the committed rocprofv3
    counter runs (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known
    size), or None when the kernel sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic_gemv_gateup_decode_b1.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != kernel_source_sha():
        return None
    return t["hbm_bytes_per_launch"]


def host_description():
    """CPU model and core counts of the host the oracle runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(cpu_model=model, logical_cpus=os.cpu_count(), cpus_available=len(os.sched_getaffinity(0)))


def cpu_baseline(spec, x, w, b, blobs, shared, seconds):
    """The oracle (plain C, one thread) on single-token decode calls of the
    headline layer: route + union + 8 routed + 1 shared expert, fp64."""
    from oracle import oracle as orc
    n = 0
    t0 = time.perf_counter()
    while True:
        xt = x[n:n + 1]
        logits = orc.router_logits(xt, w, b)
        idx, wt = orc.topk(logits, spec.top_k)
        orc.union(idx, spec.n_experts)
        need = {int(e): blobs[int(e)] for e in idx[0]}
        orc.layer_tokens(xt, spec.hidden, spec.inter, idx, wt, need, shared, [0], spec.group, spec.bits)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= x.shape[0]:
            break
    return dict(value=n / el, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{n} single-token decode calls of the same layer (route + union + 8 routed "
                       f"+ 1 shared int4 SwiGLU experts, fp64), {el:.1f} s on 1 host core")


def oracle_batch_rate(spec, x, w, b, blobs, shared, seconds, route_sample=None):
    """The oracle on one batch of a config: the router, top-k and union over
    `route_sample` tokens (all when None; the rate is then scaled to the whole
    batch, the router being linear in tokens), then the expert FFNs token by
    token for about `seconds`.  Returns the batch's extrapolated tokens/s:
    n_tok / (route time + n_tok * time per token)."""
    from oracle import oracle as orc
    n_tok = x.shape[0]
    m = n_tok if route_sample is None else min(route_sample, n_tok)
    t0 = time.perf_counter()
    logits = orc.router_logits(x[:m], w, b)
    idx, wt = orc.topk(logits, spec.top_k)
    orc.union(idx, spec.n_experts)
    t_route = (time.perf_counter() - t0) * n_tok / m
    n = 0
    t0 = time.perf_counter()
    while n < m:
        need = {int(e): blobs[int(e)] for e in idx[n]}
        orc.layer_tokens(x, spec.hidden, spec.inter, idx, wt, need, shared, [n], spec.group, spec.bits)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    t_tok = (time.perf_counter() - t0) / n
    total = t_route + n_tok * t_tok
    return dict(tokens_per_s=n_tok / total, route_s_per_batch=t_route, ffn_s_per_token=t_tok,
                sample=f"router, top-k and union over {m} of {n_tok} tokens"
                       f"{' (scaled to the batch)' if m < n_tok else ''}; expert FFNs of {n} tokens; "
                       f"1 host core")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--instances", type=int, default=8, help="layer copies rotated per step")
    ap.add_argument("--workloads", default="decode_b1,decode_b4,decode_b64,prefill_b4096,tiered_12l,"
                                           "decode_b1_g64,prefill_b4096_g64,decode_b1_i8")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy 4 times (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one MoE layer on one GPU; the library has no multi-GPU "
              "(expert-parallel) path, so runs on more than one GPU are not supported.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from int4_routed_expert_layer_amd import binding as B
    from int4_routed_expert_layer_amd import configs, inputs

    torch.cuda.init()
    # The reference rates first, before the layers' allocations fill the device.
    log("timing the HBM and matrix-core reference kernels")
    hbm_ref = hbm_reference(B, torch, reps=10)
    mfma_ref = mfma_reference(torch)
    wanted = args.workloads.split(",")
    spec1 = configs.DECODE_B1
    log(f"generating experts of {spec1.name}")
    blobs = inputs.expert_blobs(spec1, 0, range(spec1.n_experts), threads=8)
    shared = inputs.expert_blob(spec1, 0, inputs.SHARED)
    w1, b1 = inputs.router_weight(spec1), inputs.router_bias(spec1)

    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 4 x 256 MiB read + 256 MiB write")
        del src, dst

    results = {}
    specs = {"decode_b1": spec1, "decode_b4": configs.DECODE_B4, "decode_b64": configs.DECODE_B64,
             "prefill_b4096": configs.PREFILL_B4096}
    decode_layers = []
    if "decode_b1" in wanted or "decode_b4" in wanted or "decode_b64" in wanted:
        log(f"placing {args.instances} decode layer instances")
        decode_layers = make_layers(B, spec1, blobs, shared, args.instances, 64, w1, b1)

    if "decode_b1" in wanted:
        n_x = 256
        x = B.activations_to_device(inputs.activations(spec1, 0, n_x))
        wl = Workload("decode_b1", spec1, decode_layers, args.steps, args.warmup, graph_steps=64)
        log("timing decode_b1")
        results["decode_b1"] = run_workload(B, torch, wl, x, use_graph=not args.no_graph)

    if "decode_b4" in wanted:
        # the speculative-verify shape: four tokens of one sequence per call
        spec4 = configs.DECODE_B4
        x = B.activations_to_device(inputs.activations(spec4, 0, 4 * 64))
        wl = Workload("decode_b4", spec4, decode_layers, args.steps, args.warmup, graph_steps=64)
        log("timing decode_b4")
        results["decode_b4"] = run_workload(B, torch, wl, x, use_graph=not args.no_graph)

    if "decode_b64" in wanted:
        spec2 = configs.DECODE_B64
        for L in decode_layers:
            L.set_router(inputs.router_weight(spec2), inputs.router_bias(spec2))
        x = B.activations_to_device(inputs.activations(spec2, 0, 64 * 16))
        wl = Workload("decode_b64", spec2, decode_layers, max(16, args.steps // 8),
                      max(4, args.warmup // 8), graph_steps=16)
        log("timing decode_b64")
        results["decode_b64"] = run_workload(B, torch, wl, x, use_graph=not args.no_graph)
    for L in decode_layers:
        L.close()
    decode_layers = []
    torch.cuda.empty_cache()

    if "prefill_b4096" in wanted:
        spec3 = configs.PREFILL_B4096
        log("placing the prefill layer")
        (L3,) = make_layers(B, spec3, blobs, shared, 1, spec3.n_tok, inputs.router_weight(spec3),
                            inputs.router_bias(spec3))
        x = B.activations_to_device(inputs.activations(spec3, 0))
        wl = Workload("prefill_b4096", spec3, [L3], max(4, args.steps // 32), 2, graph_steps=1)
        log("timing prefill_b4096")
        results["prefill_b4096"] = run_workload(B, torch, wl, x, use_graph=False)
        L3.close()

    tiered = None
    if "tiered_12l" in wanted:
        log("placing and timing the tiered 12-layer stack")
        tiered = run_stack(B, torch, blobs, shared)
        torch.cuda.empty_cache()

    # The same layer with one scale per 64 reduction elements (the group
    # size of the README's shipped int4 container): 5.6% fewer bytes.
    if "decode_b1_g64" in wanted or "prefill_b4096_g64" in wanted:
        spec1g = spec1.with_(name="decode_b1_g64_h6144_i2048_e256_k8", group=64)
        log(f"generating experts of {spec1g.name}")
        blobs_g = inputs.expert_blobs(spec1g, 0, range(spec1g.n_experts), threads=8)
        shared_g = inputs.expert_blob(spec1g, 0, inputs.SHARED)
        if "decode_b1_g64" in wanted:
            specs["decode_b1_g64"] = spec1g
            log(f"placing {args.instances} g64 decode layer instances")
            layers_g = make_layers(B, spec1g, blobs_g, shared_g, args.instances, 64, w1, b1)
            x = B.activations_to_device(inputs.activations(spec1g, 0, 256))
            wl = Workload("decode_b1_g64", spec1g, layers_g, args.steps, args.warmup, graph_steps=64)
            log("timing decode_b1_g64")
            results["decode_b1_g64"] = run_workload(B, torch, wl, x, use_graph=not args.no_graph)
            for L in layers_g:
                L.close()
            del layers_g
            torch.cuda.empty_cache()
        if "prefill_b4096_g64" in wanted:
            spec3g = configs.PREFILL_B4096.with_(name="prefill_b4096_g64_h6144_i2048_e256_k8", group=64)
            specs["prefill_b4096_g64"] = spec3g
            log("placing the g64 prefill layer")
            (L3,) = make_layers(B, spec3g, blobs_g, shared_g, 1, spec3g.n_tok, inputs.router_weight(spec3g),
                                inputs.router_bias(spec3g))
            x = B.activations_to_device(inputs.activations(spec3g, 0))
            wl = Workload("prefill_b4096_g64", spec3g, [L3], max(4, args.steps // 32), 2, graph_steps=1)
            log("timing prefill_b4096_g64")
            results["prefill_b4096_g64"] = run_workload(B, torch, wl, x, use_graph=False)
            L3.close()
        del blobs_g, shared_g

    # Int8 experts with group-64 scales (the format the pages require for the
    # MTP head), decode B=1: twice the weight bytes of int4.
    if "decode_b1_i8" in wanted:
        spec1i = spec1.with_(name="decode_b1_i8_g64_h6144_i2048_e256_k8", group=64, bits=8)
        specs["decode_b1_i8"] = spec1i
        log(f"generating experts of {spec1i.name}")
        blobs_i = inputs.expert_blobs(spec1i, 0, range(spec1i.n_experts), threads=8)
        shared_i = inputs.expert_blob(spec1i, 0, inputs.SHARED)
        log(f"placing {args.instances} int8 decode layer instances")
        layers_i = make_layers(B, spec1i, blobs_i, shared_i, args.instances, 64, w1, b1)
        del blobs_i, shared_i
        x = B.activations_to_device(inputs.activations(spec1i, 0, 256))
        wl = Workload("decode_b1_i8", spec1i, layers_i, args.steps, args.warmup, graph_steps=64)
        log("timing decode_b1_i8")
        results["decode_b1_i8"] = run_workload(B, torch, wl, x, use_graph=not args.no_graph)
        for L in layers_i:
            L.close()
        del layers_i
        torch.cuda.empty_cache()


    # ---- report
    out_also = {}
    for name, r in results.items():
        spec = specs[name]
        ms = r.get("graph_ms_per_step", r["eager_ms_per_step"])
        nb = algorithmic_bytes(spec, r["union_mean"], spec.n_tok)
        entry = dict(tokens_per_s=spec.n_tok / (ms / 1e3), ms_per_step=ms,
                     eager_ms_per_step=r["eager_ms_per_step"], eager_ms_p50=r["eager_ms_p50"],
                     eager_ms_p90=r["eager_ms_p90"],
                     union_mean=r["union_mean"], union_min=r["union_min"], union_max=r["union_max"],
                     step_GBs=nb["total"] / (ms / 1e3) / 1e9,
                     step_frac_hbm=nb["total"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                     step_frac_stream_read=nb["total"] / (ms / 1e3) / 1e9 / hbm_ref["stream_read_GBs"],
                     kernel_us={k: v * 1e3 for k, v in r["kernel_ms"].items()})
        kg, kd = r["kernel_ms"].get("gateup"), r["kernel_ms"].get("down")
        if kg:
            entry["gateup_GBs"] = nb["gateup"] / (kg / 1e3) / 1e9
        if kd:
            entry["down_GBs"] = nb["down"] / (kd / 1e3) / 1e9
        if name.startswith("prefill") and kg and kd:
            fl = expert_flops(spec, spec.n_tok)
            entry["expert_gemm_TFLOPs"] = fl / ((kg + kd) / 1e3) / 1e12
            entry["expert_gemm_frac_mfma"] = entry["expert_gemm_TFLOPs"] / MFMA_F16_PEAK_TFLOPS
            entry["expert_gemm_frac_library_gemm"] = entry["expert_gemm_TFLOPs"] / mfma_ref["f16_TFLOPs"]
        out_also[name] = entry
    if tiered is not None:
        out_also["tiered_12l"] = tiered
    out_also["hbm_reference"] = hbm_ref
    out_also["mfma_reference"] = mfma_ref
    if "decode_b1" in out_also and out_also["decode_b1"].get("gateup_GBs"):
        g = out_also["decode_b1"]["gateup_GBs"]
        out_also["decode_b1"]["gateup_vs_sum_read"] = g / hbm_ref["sum_read_GBs"]
        out_also["decode_b1"]["gateup_vs_copy"] = g / hbm_ref["copy_read_write_GBs"]

    kernel_names = [n for n in ("decode_b1", "decode_b4", "decode_b64", "prefill_b4096", "decode_b1_g64",
                                "prefill_b4096_g64", "decode_b1_i8") if n in out_also]
    if not kernel_names:        # the tiered measurement alone
        best = tiered["lookahead"]
        print(json.dumps({"metric": METRIC, "value": best["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                          "steps": tiered["steps"], "warmup": 2, "ms_per_step": best["ms_per_step"],
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
                          "data": "synthetic", "config": {"workload": "tiered_12l_b16_lookahead"},
                          "roofline": None, "also": out_also}), flush=True)
        return
    head_name = kernel_names[0]
    head = out_also[head_name]
    head_spec = specs[head_name]
    r = results[head_name]
    nb = algorithmic_bytes(head_spec, r["union_mean"], head_spec.n_tok)
    kname = ("gemv_gateup_kernel (routed gate/up + SwiGLU)" if fused_decode(head_spec)
             else "gate/up expert kernel")
    kbytes, kt = nb["gateup"], r["kernel_ms"]["gateup"]
    achieved = kbytes / (kt / 1e3) / 1e9
    step_bytes = nb["total"]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": r.get("graph_steps_timed", args.steps),
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": head_spec.name + "+shared", "tokens_per_step": head_spec.n_tok,
                   "layer_instances_rotated": args.instances, "hip_graph": not args.no_graph,
                   "all_experts_vram": True},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic() if head_name == "decode_b1" else None,
                     "kernel": kname, "bytes_per_launch": kbytes, "avg_launch_us": kt * 1e3,
                     # the whole layer step: its algorithmic bytes over ms_per_step
                     "step_bytes": step_bytes, "step_achieved": step_bytes / (head["ms_per_step"] / 1e3) / 1e9,
                     "step_frac": step_bytes / (head["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                     # the plain read's rate on this part (coli_probe_read over 2 GiB), and both
                     # rates as fractions of it
                     "stream_read_GBs": hbm_ref["stream_read_GBs"],
                     "frac_of_stream_read": achieved / hbm_ref["stream_read_GBs"],
                     "step_frac_of_stream_read": step_bytes / (head["ms_per_step"] / 1e3) / 1e9
                     / hbm_ref["stream_read_GBs"]},
        "also": out_also,
    }
    if not args.no_cpu_baseline and head_name == "decode_b1":
        log("timing the CPU oracle")
        xs = inputs.activations(spec1, 0, 64)
        cb = cpu_baseline(spec1, xs, w1, b1, blobs, shared, args.cpu_seconds)
        cb["host"] = host_description()
        per = {"decode_b1": dict(tokens_per_s=cb["value"], gpu_over_oracle=head["tokens_per_s"] / cb["value"])}
        for name, spec, route_sample in (("decode_b64", configs.DECODE_B64, None),
                                         ("prefill_b4096", configs.PREFILL_B4096, 256)):
            log(f"timing the CPU oracle on {name}")
            o = oracle_batch_rate(spec, inputs.activations(spec, 0), inputs.router_weight(spec),
                                  inputs.router_bias(spec), blobs, shared, args.cpu_seconds / 2, route_sample)
            if name in out_also:
                o["gpu_over_oracle"] = out_also[name]["tokens_per_s"] / o["tokens_per_s"]
            per[name] = o
        cb["per_config"] = per
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
