"""Shared helpers of the GPU parity tests: build a layer from a workload
spec, run it through the C ABI, run the CPU oracle on the same seeded
inputs, and compare (bit-exact routing and union, output within
2e-3 * max|ref|)."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from int4_routed_expert_layer_amd import inputs
from oracle import oracle as orc

TOL = 2e-3          # max|y_gpu - y_ref| <= TOL * max|y_ref|
# Oracle worker threads: the host's cores, at most 16 (the CPU share of a
# one-GPU machine).
THREADS = max(1, min(16, os.cpu_count() or 1))
# Rows per grouped-GEMM work chunk (five 32-row MFMA tiles): experts with
# more rows are split into several chunks.
CHUNK_ROWS = 160


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class Data:
    """Seeded inputs of one layer of a spec (blobs drawn lazily)."""

    def __init__(self, spec, layer=0, n_tok=None):
        self.spec, self.layer = spec, layer
        self.x = inputs.activations(spec, layer, n_tok)
        self.w = inputs.router_weight(spec, layer)
        self.b = inputs.router_bias(spec, layer)
        self._blobs = {}
        self.shared = inputs.expert_blob(spec, layer, inputs.SHARED) if spec.has_shared else None

    def blobs(self, experts):
        need = [e for e in experts if e not in self._blobs]
        if need:
            self._blobs.update(inputs.expert_blobs(self.spec, self.layer, need, THREADS))
        return {e: self._blobs[e] for e in experts}

    def drop_blobs(self):
        self._blobs.clear()


def make_layer(B, data, tiers=None, place=None, max_tokens=None, path=None):
    """MoELayer with router and experts placed (all VRAM unless tiers says)."""
    spec = data.spec
    L = B.MoELayer.from_spec(spec, max_tokens=max_tokens or data.x.shape[0])
    L.set_router(data.w, data.b)
    experts = range(spec.n_experts) if place is None else place
    chunk = 32
    ex = list(experts)
    for i in range(0, len(ex), chunk):
        part = ex[i:i + chunk]
        for e, blob in data.blobs(part).items():
            tier = B.TIER_VRAM if tiers is None else tiers[e]
            L.place(e, blob, tier)
        data.drop_blobs()
    if data.shared is not None:
        L.place(B.SHARED, data.shared, B.TIER_VRAM)
    if path is not None:
        L.set_path(path)
    return L


def gpu_run(B, L, data, with_logits=True):
    import torch
    x = B.activations_to_device(data.x)
    out = {}
    if with_logits:
        out["logits"] = L.router_logits(x)
    y, idx, w, u = L(x)
    torch.cuda.synchronize()
    out.update(idx=idx.cpu().numpy(), weight=w.cpu().numpy(), y=y.cpu().numpy(),
               n_union=int(u["n_union"].cpu()[0]), counts=u["counts"].cpu().numpy(),
               offsets=u["offsets"].cpu().numpy(), gather=u["gather"].cpu().numpy())
    out["union_ids"] = u["union_ids"].cpu().numpy()[:out["n_union"]]
    if with_logits:
        out["logits"] = out["logits"].cpu().numpy()
    return out


def oracle_route(data):
    """Logits, top-k and union of the whole batch (threads over tokens)."""
    x, n = data.x, data.x.shape[0]
    parts = max(1, min(THREADS, n // 64))
    bounds = np.linspace(0, n, parts + 1).astype(int)
    with ThreadPoolExecutor(parts) as ex:
        chunks = list(ex.map(lambda i: orc.router_logits(x[bounds[i]:bounds[i + 1]], data.w, data.b),
                             range(parts)))
    logits = np.concatenate(chunks, 0)
    idx, w = orc.topk(logits, data.spec.top_k)
    un = orc.union(idx, data.spec.n_experts)
    return dict(logits=logits, idx=idx, weight=w, **un)


def oracle_y(data, ref, tokens):
    spec = data.spec
    tokens = list(tokens)
    need = sorted({int(e) for t in tokens for e in ref["idx"][t]})
    blobs = data.blobs(need)

    def one(t):
        return orc.layer_tokens(data.x, spec.hidden, spec.inter, ref["idx"], ref["weight"],
                                blobs, data.shared, [t], spec.group, spec.bits)[0]
    with ThreadPoolExecutor(THREADS) as ex:
        ys = list(ex.map(one, tokens))
    return np.stack(ys)


def check_routing(gpu, ref, check_logits=True):
    if check_logits and "logits" in gpu:
        assert np.array_equal(gpu["logits"].view(np.uint32), ref["logits"].view(np.uint32)), \
            "router logits differ bitwise"
    np.testing.assert_array_equal(gpu["idx"], ref["idx"])
    np.testing.assert_allclose(gpu["weight"], ref["weight"], rtol=2e-6, atol=1e-7)
    assert gpu["n_union"] == ref["n_union"]
    np.testing.assert_array_equal(gpu["union_ids"], ref["union_ids"])
    np.testing.assert_array_equal(gpu["counts"], ref["counts"])
    np.testing.assert_array_equal(gpu["offsets"], ref["offsets"])
    np.testing.assert_array_equal(gpu["gather"][:len(ref["gather"])], ref["gather"])


def check_outputs(y_gpu, y_ref, what=""):
    scale = float(np.max(np.abs(y_ref)))
    err = float(np.max(np.abs(y_gpu.astype(np.float64) - y_ref)))
    log(f"  {what} max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio = {err / scale:.3e}")
    assert np.all(np.isfinite(y_gpu))
    assert err <= TOL * scale, f"{what}: {err / scale:.3e} > {TOL}"
    return err / scale


def edge_tokens(ref, k, extra=()):
    """Tokens whose outputs cover every union expert's grouped work: the
    tokens on the first and last gather row of each expert and on both sides
    of every CHUNK_ROWS boundary inside an expert's rows, plus ``extra``.
    Comparing these checks each expert's first and last MFMA tile of every
    chunk the grouped path cuts it into."""
    gather, counts, offsets = ref["gather"], ref["counts"], ref["offsets"]
    rows = set()
    for e in np.nonzero(counts)[0]:
        r0, m = int(offsets[e]), int(counts[e])
        rows.update((r0, r0 + m - 1))
        for b in range(CHUNK_ROWS, m, CHUNK_ROWS):
            rows.update((r0 + b - 1, r0 + b))
    toks = {int(gather[r]) // k for r in rows}
    toks.update(int(t) for t in extra)
    return sorted(toks)


def planted_routing(n_experts, top_k, counts, n_tok, seed):
    """Token sets S_t (n_tok x top_k expert ids, each row distinct) in which
    expert e is chosen by exactly counts[e] tokens.  Experts are laid out one
    after another on a cycle over the tokens, so an expert's counts[e] <=
    n_tok entries land on distinct tokens and every token gets exactly top_k
    entries (sum(counts) must be n_tok * top_k)."""
    counts = np.asarray(counts, dtype=np.int64)
    assert counts.shape == (n_experts,) and counts.sum() == n_tok * top_k
    assert counts.max() <= n_tok
    order = np.random.default_rng(seed).permutation(n_experts)
    slots = [[] for _ in range(n_tok)]
    pos = 0
    for e in order:
        for i in range(int(counts[e])):
            slots[(pos + i) % n_tok].append(int(e))
        pos += int(counts[e])
    sets = np.array(slots, dtype=np.int32)
    assert sets.shape == (n_tok, top_k)
    return sets


def planted_inputs(spec, sets, seed):
    """Activations (bf16 bits) and router weight under which the oracle's
    top-k of token t is exactly the set sets[t]: W_r[:, e] is the unit vector
    of row e plus N(0, 0.01^2) on the rows past E, x[t, e] lies in [2, 3) for
    chosen experts and in (-3, -2] otherwise, and the other columns are
    N(0, 1).  A logit is then x[t, e] plus noise of deviation
    0.01 sqrt(H - E) (0.32 at H = 1024), against a gap of 4 between chosen
    and other experts."""
    from int4_routed_expert_layer_amd.inputs import f32_to_bf16_bits
    g = np.random.default_rng(seed)
    n_tok, E, H = sets.shape[0], spec.n_experts, spec.hidden
    assert H > E
    x = g.standard_normal((n_tok, H)).astype(np.float32)
    chosen = np.zeros((n_tok, E), dtype=bool)
    chosen[np.arange(n_tok)[:, None], sets] = True
    mag = 2.0 + g.random((n_tok, E))
    x[:, :E] = np.where(chosen, mag, -mag).astype(np.float32)
    w = (g.standard_normal((H, E)) * 0.01).astype(np.float32)
    w[:E, :] = 0.0
    w[np.arange(E), np.arange(E)] = 1.0
    return f32_to_bf16_bits(x), w
