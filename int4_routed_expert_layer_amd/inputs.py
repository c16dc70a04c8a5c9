"""Seeded synthetic inputs for the MoE layer (test and benchmark data only).

Nothing here computes any part of the layer: it draws activations, router
weights, router bias, int4 expert blobs and tier assignments from numpy
``SeedSequence`` streams keyed by (seed, layer, stream), so each expert can be
regenerated on its own without materialising a whole multi-GB layer.

Recipe (the pages name the model, GLM-5.2, and its sizes but print no tensor):
  * activations: N(0,1); fp32 for ``act == "f32"``, otherwise rounded to bf16
    (round to nearest even) and returned as raw uint16 bit patterns;
  * router weight W_r [H x E] fp32 ~ N(0, 1/H), so every logit is ~N(0,1);
  * router bias: 0 for "gauss" routing; for "zipf" routing expert e gets
    gamma * ln p_rank(e), p_r proportional to r^-s over ranks r=1..E, ranks
    taken from a seeded permutation, so expert popularity falls off like a
    Zipf law (gamma=0.648 makes the realised rank-frequency slope about -s
    for top-8 of 256);
  * expert weights: uniform over the 16 int4 codes (uniform bytes), or for
    int8 experts over the 256 int8 codes;
  * expert scales: U[0.005, 0.02] rounded to fp16 (int4), or U[0.005, 0.02]/16
    for int8 (the same real weight range at 16 times the resolution);
  * tiers: the first round(resident_frac * E) experts of a seeded
    permutation are VRAM-resident, the rest live in pinned host memory.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Spec, blob_sections

SHARED = -1

# Stream ids beyond the routed experts' own ids (0..E-1).
def _streams(spec: Spec) -> dict:
    e = spec.n_experts
    return dict(shared=e, router_w=e + 1, router_b=e + 2, act=e + 3,
                tier=e + 4)


def rng(spec: Spec, layer: int, stream: int) -> np.random.Generator:
    ss = np.random.SeedSequence(spec.seed, spawn_key=(layer, stream))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(spec: Spec, layer: int = 0, n_tok: int | None = None) -> np.ndarray:
    """[B x H] activations: float32, or uint16 bf16 bits when act == "bf16"."""
    n = spec.n_tok if n_tok is None else n_tok
    g = rng(spec, layer, _streams(spec)["act"])
    x = g.standard_normal((n, spec.hidden), dtype=np.float32)
    return x if spec.act == "f32" else f32_to_bf16_bits(x)


def router_weight(spec: Spec, layer: int = 0) -> np.ndarray:
    """W_r [H x E] fp32 (reduction axis outer), entries ~ N(0, 1/H)."""
    g = rng(spec, layer, _streams(spec)["router_w"])
    w = g.standard_normal((spec.hidden, spec.n_experts), dtype=np.float32)
    return (w * np.float32(1.0 / np.sqrt(spec.hidden))).astype(np.float32)


def zipf_ranks(spec: Spec, layer: int = 0) -> np.ndarray:
    """rank[e] in 1..E: the popularity rank of expert e (1 = most popular)."""
    g = rng(spec, layer, _streams(spec)["router_b"])
    perm = g.permutation(spec.n_experts)
    rank = np.empty(spec.n_experts, dtype=np.int64)
    rank[perm] = np.arange(1, spec.n_experts + 1)
    return rank


def router_bias(spec: Spec, layer: int = 0) -> np.ndarray:
    if spec.routing == "gauss":
        return np.zeros(spec.n_experts, dtype=np.float32)
    if spec.routing != "zipf":
        raise ValueError(spec.routing)
    r = np.arange(1, spec.n_experts + 1, dtype=np.float64)
    p = r ** (-spec.zipf_s)
    p /= p.sum()
    rank = zipf_ranks(spec, layer)
    return (spec.zipf_gamma * np.log(p[rank - 1])).astype(np.float32)


def resident_mask(spec: Spec, layer: int = 0) -> np.ndarray:
    """True for experts that live in VRAM, False for pinned-host experts."""
    n_res = int(round(spec.resident_frac * spec.n_experts))
    g = rng(spec, layer, _streams(spec)["tier"])
    perm = g.permutation(spec.n_experts)
    mask = np.zeros(spec.n_experts, dtype=bool)
    mask[perm[:n_res]] = True
    return mask


def expert_blob(spec: Spec, layer: int, expert: int) -> np.ndarray:
    """Canonical blob (uint8) of routed expert ``expert`` or of SHARED."""
    stream = _streams(spec)["shared"] if expert == SHARED else expert
    if not (0 <= stream <= spec.n_experts):
        raise ValueError(f"expert {expert} out of range")
    if expert == SHARED and not spec.has_shared:
        raise ValueError("spec has no shared expert")
    sec = blob_sections(spec.hidden, spec.inter, spec.group, spec.bits)
    blob = np.zeros(sec["total"][1], dtype=np.uint8)
    g = rng(spec, layer, stream)
    for name in ("gate_q", "up_q", "down_q"):
        off, size = sec[name]
        blob[off:off + size] = g.integers(0, 256, size=size, dtype=np.uint8)
    for name in ("gate_s", "up_s", "down_s"):
        off, size = sec[name]
        lo, hi = (0.005, 0.02) if spec.bits == 4 else (0.005 / 16, 0.02 / 16)
        s = g.uniform(lo, hi, size=size // 2).astype(np.float16)
        blob[off:off + size] = s.view(np.uint8)
    return blob


def expert_blobs(spec: Spec, layer: int, experts, threads: int = 8) -> dict:
    """{expert: blob} for several experts, drawn on a thread pool."""
    experts = list(experts)
    if threads <= 1 or len(experts) <= 1:
        return {e: expert_blob(spec, layer, e) for e in experts}
    with ThreadPoolExecutor(threads) as ex:
        blobs = list(ex.map(lambda e: expert_blob(spec, layer, e), experts))
    return dict(zip(experts, blobs))
