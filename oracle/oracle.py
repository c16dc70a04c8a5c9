"""ctypes wrapper over the plain-C CPU oracle (coli_oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, the smoke check and
the benchmark's CPU-baseline leg import this module.  It imports nothing from
the HIP library and the HIP library imports nothing from it.

Every function takes and returns numpy arrays; the arithmetic is all in the C
file (see its header for the definition of the layer and the readings of the
Colibri pages that it follows).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "coli_oracle.c")
LIB = os.path.join(HERE, "libcoli_oracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (single-threaded, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        L = C.CDLL(LIB)
        p = C.c_void_p
        i = C.c_int
        L.coli_oracle_version.restype = i
        L.coli_oracle_half_to_double.argtypes = [C.c_uint16]
        L.coli_oracle_half_to_double.restype = C.c_double
        L.coli_oracle_nibble.argtypes = [p, i]
        L.coli_oracle_nibble.restype = i
        L.coli_oracle_router.argtypes = [p, i, p, p, i, i, i, p]
        L.coli_oracle_topk.argtypes = [p, i, i, i, p, p]
        L.coli_oracle_union.argtypes = [p, i, i, i, p, p, p, p, p]
        L.coli_oracle_blob_bytes.argtypes = [i, i, i, i]
        L.coli_oracle_blob_bytes.restype = C.c_size_t
        L.coli_oracle_expert_ffn.argtypes = [p, i, i, i, i, p, p]
        L.coli_oracle_dequant.argtypes = [p, i, i, i, i, i, p]
        L.coli_oracle_layer_tokens.argtypes = [p, i, i, i, i, i, i, p, p, p, p, p, i, p]
        for f in ("router", "topk", "union", "expert_ffn", "dequant",
                  "layer_tokens"):
            getattr(L, "coli_oracle_" + f).restype = i
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> C.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return C.c_void_p(a.ctypes.data)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def _x_args(x: np.ndarray):
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), 0
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    raise TypeError("activations must be float32 or uint16 bf16 bits")


def half_to_double(bits: int) -> float:
    return lib().coli_oracle_half_to_double(bits)


def nibble(row: np.ndarray, k: int) -> int:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    return lib().coli_oracle_nibble(_ptr(row), k)


def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """[B x E] fp32 logits in the canonical summation order."""
    x, bf = _x_args(x)
    n_tok, hidden = x.shape
    w = np.ascontiguousarray(w_router, dtype=np.float32)
    assert w.shape[0] == hidden
    n_exp = w.shape[1]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((n_tok, n_exp), dtype=np.float32)
    _check(lib().coli_oracle_router(_ptr(x), bf, _ptr(w),
                                    None if b is None else _ptr(b),
                                    n_tok, hidden, n_exp, _ptr(out)), "router")
    return out


def topk(logits: np.ndarray, k: int):
    """(idx [B x k] int32 in rank order, weights [B x k] fp64)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    n_tok, n_exp = lg.shape
    idx = np.empty((n_tok, k), dtype=np.int32)
    w = np.empty((n_tok, k), dtype=np.float64)
    _check(lib().coli_oracle_topk(_ptr(lg), n_tok, n_exp, k, _ptr(idx), _ptr(w)),
           "topk")
    return idx, w


def union(idx: np.ndarray, n_experts: int) -> dict:
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n_tok, k = idx.shape
    nu = np.zeros(1, dtype=np.int32)
    ids = np.zeros(n_experts, dtype=np.int32)
    counts = np.zeros(n_experts, dtype=np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    gather = np.zeros(n_tok * k, dtype=np.int32)
    _check(lib().coli_oracle_union(_ptr(idx), n_tok, k, n_experts, _ptr(nu),
                                   _ptr(ids), _ptr(counts), _ptr(offsets),
                                   _ptr(gather)), "union")
    n = int(nu[0])
    return dict(n_union=n, union_ids=ids[:n].copy(), counts=counts,
                offsets=offsets, gather=gather)


def blob_bytes(hidden: int, inter: int, group: int = 32, bits: int = 4) -> int:
    n = int(lib().coli_oracle_blob_bytes(hidden, inter, group, bits))
    if n == 0:
        raise ValueError(f"no {bits}-bit layout with group {group} for hidden {hidden}, inter {inter}")
    return n


def dequant(blob: np.ndarray, hidden: int, inter: int, which: str, group: int = 32,
            bits: int = 4) -> np.ndarray:
    """One matrix of a canonical blob as fp64 [rows x K] (``bits``-bit
    weights, one fp16 scale per ``group`` consecutive reduction elements)."""
    w = {"gate": 0, "up": 1, "down": 2}[which]
    rows, K = (hidden, inter) if w == 2 else (inter, hidden)
    out = np.empty((rows, K), dtype=np.float64)
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    _check(lib().coli_oracle_dequant(_ptr(blob), hidden, inter, group, bits, w, _ptr(out)),
           "dequant")
    return out


def expert_ffn(blob: np.ndarray, hidden: int, inter: int, x: np.ndarray, group: int = 32,
               bits: int = 4) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(hidden, dtype=np.float64)
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    _check(lib().coli_oracle_expert_ffn(_ptr(blob), hidden, inter, group, bits, _ptr(x), _ptr(y)),
           "expert_ffn")
    return y


def layer_tokens(x: np.ndarray, hidden: int, inter: int, idx: np.ndarray,
                 weight: np.ndarray, blobs: dict, shared, tokens, group: int = 32,
                 bits: int = 4) -> np.ndarray:
    """y [len(tokens) x H] fp64 for the listed tokens.

    blobs maps expert id -> canonical blob and must cover every expert the
    listed tokens route to; shared is the shared expert's blob or None.
    """
    x, bf = _x_args(x)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    weight = np.ascontiguousarray(weight, dtype=np.float64)
    k = idx.shape[1]
    n_exp = max(max(blobs) + 1 if blobs else 0, int(idx.max()) + 1)
    keep = [np.ascontiguousarray(b, dtype=np.uint8) for b in blobs.values()]
    table = (C.c_void_p * n_exp)()
    for e, b in zip(blobs.keys(), keep):
        table[e] = b.ctypes.data
    sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.uint8)
    sel = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    y = np.empty((len(sel), hidden), dtype=np.float64)
    _check(lib().coli_oracle_layer_tokens(
        _ptr(x), bf, hidden, inter, group, bits, k, _ptr(idx), _ptr(weight), table,
        None if sh is None else _ptr(sh), _ptr(sel), len(sel), _ptr(y)),
        "layer_tokens (missing expert blob?)")
    return y


def run_layer(x, w_router, bias, k, blobs, shared, hidden, inter, tokens=None, group=32, bits=4):
    """Route, union and (for ``tokens``, default all) the layer output."""
    logits = router_logits(x, w_router, bias)
    idx, w = topk(logits, k)
    un = union(idx, w_router.shape[1])
    if tokens is None:
        tokens = range(x.shape[0])
    y = layer_tokens(x, hidden, inter, idx, w, blobs, shared, tokens, group, bits)
    return dict(logits=logits, idx=idx, weight=w, y=y, **un)
