"""Workload shapes for one int4 routed-expert MoE layer.

The Colibri pages (README "L'idea", the per-token path of the getting-started
page) describe GLM-5.2 layers with 256 routed experts of roughly 19 MB of int4
each and about 11 GB of routed weights touched per token over 75 layers, which
fixes top-8 and, with H=6144 and I=2048, 3*H*I/2 = 18.9 MB of nibbles per
expert.  The pages give no shape for a layer; the five workloads below are the
ones this library is measured and checked on.

A ``Spec`` is pure data: sizes, dtypes, the routing recipe and the seed.  The
arithmetic of the layer lives in the HIP library; the random inputs are drawn
by ``inputs.py``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

# Int4 weights carry one fp16 scale per GROUP consecutive reduction elements
# (32 in the fixed workloads; the container the README's "Scarica il modello"
# section ships uses 64, which GROUPS also allows).
GROUP = 32
GROUPS = (32, 64)
# Every section of an expert blob starts on a 256-byte boundary.
BLOB_ALIGN = 256


@dataclass(frozen=True)
class Spec:
    name: str
    hidden: int            # H, model width
    inter: int             # I, expert intermediate width
    n_experts: int         # E, routed experts per layer
    top_k: int             # k, experts per token
    n_tok: int             # B, tokens per call
    act: str               # "f32" or "bf16" activations
    has_shared: bool       # one always-on shared expert of the same shape
    routing: str           # "gauss" (bias 0) or "zipf" (popularity bias)
    n_layers: int = 1
    resident_frac: float = 1.0   # share of routed experts kept in VRAM
    seed: int = 20261203
    zipf_s: float = 1.1
    zipf_gamma: float = 0.648
    group: int = GROUP           # reduction elements per fp16 weight scale
    bits: int = 4                # weight width: 4 (int4) or 8 (int8)

    @property
    def act_bytes(self) -> int:
        return 4 if self.act == "f32" else 2

    def with_(self, **kw) -> "Spec":
        return replace(self, **kw)


def _align(n: int) -> int:
    return (n + BLOB_ALIGN - 1) // BLOB_ALIGN * BLOB_ALIGN


def blob_sections(hidden: int, inter: int, group: int = GROUP, bits: int = 4) -> dict:
    """Byte offset and size of each section of one expert blob.

    Order: gate nibbles, up nibbles, down nibbles, gate scales, up scales,
    down scales.  Gate and up are [I x H] (output rows x reduction), down is
    [H x I]; weights are row-major along the reduction axis, int4 two per
    byte (element 2j in the low nibble) or int8 one per byte; scales are fp16
    [rows x K/group].
    """
    h, i = hidden, inter
    sizes = [
        ("gate_q", i * h * bits // 8), ("up_q", i * h * bits // 8), ("down_q", h * i * bits // 8),
        ("gate_s", i * (h // group) * 2), ("up_s", i * (h // group) * 2),
        ("down_s", h * (i // group) * 2),
    ]
    out, off = {}, 0
    for name, size in sizes:
        out[name] = (off, size)
        off = _align(off + size)
    out["total"] = (0, off)
    return out


def blob_bytes(hidden: int, inter: int, group: int = GROUP, bits: int = 4) -> int:
    return blob_sections(hidden, inter, group, bits)["total"][1]


_BIG = dict(hidden=6144, inter=2048, n_experts=256, top_k=8, act="bf16",
            has_shared=True)

TINY = Spec("tiny_h256_i128_e16_k4_b8", 256, 128, 16, 4, 8, "f32", False,
            "gauss", seed=20261203 + 0)
DECODE_B1 = Spec("decode_b1_h6144_i2048_e256_k8", n_tok=1, routing="gauss",
                 seed=20261203 + 1, **_BIG)
# Four tokens of one sequence per call: the speculative-verify batch.
DECODE_B4 = Spec("decode_b4_h6144_i2048_e256_k8", n_tok=4, routing="gauss",
                 seed=20261203 + 1, **_BIG)
DECODE_B64 = Spec("decode_b64_zipf_h6144_i2048_e256_k8", n_tok=64,
                  routing="zipf", seed=20261203 + 2, **_BIG)
PREFILL_B4096 = Spec("prefill_b4096_h6144_i2048_e256_k8", n_tok=4096,
                     routing="gauss", seed=20261203 + 3, **_BIG)
TIERED_12L = Spec("tiered_12l_b16_zipf_h6144_i2048_e256_k8", n_tok=16,
                  routing="zipf", n_layers=12, resident_frac=0.6,
                  seed=20261203 + 4, **_BIG)

WORKLOADS = [TINY, DECODE_B1, DECODE_B64, PREFILL_B4096, TIERED_12L]
