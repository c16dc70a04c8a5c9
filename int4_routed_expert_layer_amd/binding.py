"""Thin ctypes binding over the C ABI in include/coli_moe.h.

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch provides device memory (output tensors) and the current HIP stream.
Importing this module fails loudly if the library has not been built; there
is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcoli_moe.so")

OK, E_INVALID, E_NOMEM, E_DEVICE, E_STATE, E_UNSUPPORTED = range(6)
ACT_F32, ACT_BF16 = 0, 1
TIER_VRAM, TIER_HOST = 0, 1
PATH_AUTO, PATH_GEMV, PATH_GROUPED = 0, 1, 2
SHARED = -1

# Every function the header declares, with (restype, argtypes).
_p, _i32, _sz, _i64 = C.c_void_p, C.c_int32, C.c_size_t, C.c_int64
SIGNATURES = {
    "coli_abi_version": (_i32, []),
    "coli_status_str": (C.c_char_p, [C.c_int]),
    "coli_last_error": (C.c_char_p, [_p]),
    "coli_expert_blob_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "coli_expert_repack": (C.c_int, [_p, _p, _i32, _i32, _i32, _i32]),
    "coli_layer_create": (C.c_int, [_p, C.c_int, _p]),
    "coli_layer_destroy": (C.c_int, [_p]),
    "coli_router_set": (C.c_int, [_p, _p, _p]),
    "coli_expert_place": (C.c_int, [_p, _i32, _p, _sz, C.c_int]),
    "coli_moe_route": (C.c_int, [_p, _p, _i32, _p, _p, _p]),
    "coli_moe_router_logits": (C.c_int, [_p, _p, _i32, _p, _p]),
    "coli_moe_union": (C.c_int, [_p, _p, _i32, _p, _p, _p, _p, _p, _p]),
    "coli_moe_forward": (C.c_int, [_p, _p, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "coli_layer_set_path": (C.c_int, [_p, _i32]),
    "coli_moe_layer": (C.c_int, [_p, _p, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "coli_moe_layer_static": (C.c_int, [_p, _p, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "coli_layer_stream_stats": (C.c_int, [_p, _p, _p]),
    "coli_layer_set_stream_cache": (C.c_int, [_p, _i32]),
    "coli_layer_stream_hits": (C.c_int, [_p, _p]),
    "coli_layer_prefetch_union": (C.c_int, [_p, _p, _p, _p, _p]),
    "coli_layer_device_errors": (C.c_int, [_p, _p]),
    "coli_layer_set_timing": (C.c_int, [_p, _i32]),
    "coli_layer_kernel_times": (C.c_int, [_p, _p, _p]),
    "coli_set_alloc_limit": (C.c_int, [_i64]),
    "coli_alloc_bytes": (_i64, []),
    "coli_probe_read": (C.c_int, [_p, _sz, _p, _p]),
}
KERNEL_KINDS = ["router", "topk", "union", "plan", "gateup", "down", "combine"]


class Dims(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("inter", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("has_shared", C.c_int32), ("max_tokens", C.c_int32),
                ("act", C.c_int32), ("group", C.c_int32), ("weight_bits", C.c_int32)]


class ColiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)}: {msg}")
        self.status = status


def _load():
    # torch carries its own HIP runtime under the soname libamdhip64.so.7.
    # Importing it first makes the library bind to that same copy, so the
    # process holds one HIP runtime: a second runtime loaded beside it finds
    # no device once torch's has claimed the GPU.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: the HIP library must be built "
            "(python -m int4_routed_expert_layer_amd.build); there is no CPU fallback")
    L = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def status_str(st: int) -> str:
    return lib.coli_status_str(st).decode()


def blob_bytes(hidden: int, inter: int, group: int = 32, bits: int = 4) -> int:
    return int(lib.coli_expert_blob_bytes(hidden, inter, group, bits))


def repack(blob: np.ndarray, hidden: int, inter: int, group: int = 32, bits: int = 4) -> np.ndarray:
    """Device-layout bytes of a canonical expert blob (host-side repack)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    out = np.empty_like(blob)
    _check(lib.coli_expert_repack(blob.ctypes.data, out.ctypes.data, hidden, inter, group, bits))
    return out


def _check(st: int, handle=None) -> None:
    if st != OK:
        raise ColiError(st, lib.coli_last_error(handle).decode())


def _stream():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dptr(t) -> C.c_void_p:
    return C.c_void_p(t.data_ptr())


class MoELayer:
    """One MoE layer living on a HIP device (owns its router and experts)."""

    def __init__(self, hidden, inter, n_experts, top_k, has_shared, max_tokens,
                 act="bf16", device=0, group=32, bits=4):
        self.dims = Dims(hidden, inter, n_experts, top_k, int(bool(has_shared)),
                         max_tokens, ACT_BF16 if act == "bf16" else ACT_F32, group, bits)
        self.device = device
        h = C.c_void_p()
        _check(lib.coli_layer_create(C.byref(self.dims), device, C.byref(h)))
        self.handle = h

    @classmethod
    def from_spec(cls, spec, max_tokens=None, device=0):
        return cls(spec.hidden, spec.inter, spec.n_experts, spec.top_k, spec.has_shared,
                   max_tokens or spec.n_tok, spec.act, device, spec.group, spec.bits)

    def close(self):
        if getattr(self, "handle", None):
            lib.coli_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- setup -------------------------------------------------------------
    def set_router(self, w: np.ndarray, bias=None):
        w = np.ascontiguousarray(w, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        _check(lib.coli_router_set(self.handle, w.ctypes.data,
                                   None if b is None else b.ctypes.data), self.handle)

    def place(self, expert: int, blob: np.ndarray, tier: int = TIER_VRAM):
        blob = np.ascontiguousarray(blob, dtype=np.uint8)
        _check(lib.coli_expert_place(self.handle, expert, blob.ctypes.data, blob.nbytes, tier),
               self.handle)

    def set_path(self, path: int):
        _check(lib.coli_layer_set_path(self.handle, path), self.handle)

    # -- per call ----------------------------------------------------------
    def _new(self, shape, dtype):
        import torch
        return torch.empty(shape, dtype=dtype, device=f"cuda:{self.device}")

    def router_logits(self, x):
        import torch
        n = x.shape[0]
        out = self._new((n, self.dims.n_experts), torch.float32)
        _check(lib.coli_moe_router_logits(self.handle, _dptr(x), n, _dptr(out), _stream()),
               self.handle)
        return out

    def route(self, x):
        import torch
        n, k = x.shape[0], self.dims.top_k
        idx = self._new((n, k), torch.int32)
        w = self._new((n, k), torch.float32)
        _check(lib.coli_moe_route(self.handle, _dptr(x), n, _dptr(idx), _dptr(w), _stream()),
               self.handle)
        return idx, w

    def union(self, idx):
        import torch
        n, E = idx.shape[0], self.dims.n_experts
        u = dict(n_union=self._new((1,), torch.int32),
                 union_ids=self._new((E,), torch.int32),
                 counts=self._new((E,), torch.int32),
                 offsets=self._new((E + 1,), torch.int32),
                 gather=self._new((max(n * self.dims.top_k, 1),), torch.int32))
        _check(lib.coli_moe_union(self.handle, _dptr(idx), n, _dptr(u["n_union"]),
                                  _dptr(u["union_ids"]), _dptr(u["counts"]), _dptr(u["offsets"]),
                                  _dptr(u["gather"]), _stream()), self.handle)
        return u

    def forward(self, x, idx, w, u, y=None):
        import torch
        n = x.shape[0]
        if y is None:
            y = self._new((n, self.dims.hidden), torch.float32)
        _check(lib.coli_moe_forward(self.handle, _dptr(x), n, _dptr(idx), _dptr(w),
                                    _dptr(u["n_union"]), _dptr(u["union_ids"]), _dptr(u["counts"]),
                                    _dptr(u["offsets"]), _dptr(u["gather"]), _dptr(y), _stream()),
               self.handle)
        return y

    def _union_bufs(self, n):
        import torch
        E = self.dims.n_experts
        return dict(n_union=self._new((1,), torch.int32),
                    union_ids=self._new((E,), torch.int32),
                    counts=self._new((E,), torch.int32),
                    offsets=self._new((E + 1,), torch.int32),
                    gather=self._new((max(n * self.dims.top_k, 1),), torch.int32))

    def layer(self, x):
        """Route, union and forward in one call (coli_moe_layer)."""
        import torch
        n, k = x.shape[0], self.dims.top_k
        idx = self._new((n, k), torch.int32)
        w = self._new((n, k), torch.float32)
        u = self._union_bufs(n)
        y = self._new((n, self.dims.hidden), torch.float32)
        _check(lib.coli_moe_layer(self.handle, _dptr(x), n, _dptr(idx), _dptr(w), _dptr(u["n_union"]),
                                  _dptr(u["union_ids"]), _dptr(u["counts"]), _dptr(u["offsets"]),
                                  _dptr(u["gather"]), _dptr(y), _stream()), self.handle)
        return y, idx, w, u

    def layer_static(self, x, out=None):
        """coli_moe_layer_static: the fused small-batch call on the library's
        static scratch.  ``out`` (optional) is a dict of preallocated outputs
        with the keys layer() returns (y, idx, w, u)."""
        import torch
        n, k = x.shape[0], self.dims.top_k
        if out is None:
            out = dict(y=self._new((n, self.dims.hidden), torch.float32), idx=self._new((n, k), torch.int32),
                       w=self._new((n, k), torch.float32), u=self._union_bufs(n))
        u = out["u"]
        _check(lib.coli_moe_layer_static(self.handle, _dptr(x), n, _dptr(out["idx"]), _dptr(out["w"]),
                                         _dptr(u["n_union"]), _dptr(u["union_ids"]), _dptr(u["counts"]),
                                         _dptr(u["offsets"]), _dptr(u["gather"]), _dptr(out["y"]), _stream()),
               self.handle)
        return out["y"], out["idx"], out["w"], u

    def __call__(self, x):
        idx, w = self.route(x)
        u = self.union(idx)
        return self.forward(x, idx, w, u), idx, w, u

    def set_stream_cache(self, n_slots: int):
        _check(lib.coli_layer_set_stream_cache(self.handle, n_slots), self.handle)

    def prefetch_union(self, u) -> int:
        """Start copies of the host-tier experts of union ``u`` (the dict
        union() returns) into the stream cache; returns the copies started."""
        n = C.c_int32()
        _check(lib.coli_layer_prefetch_union(self.handle, _dptr(u["n_union"]), _dptr(u["union_ids"]),
                                             _stream(), C.byref(n)), self.handle)
        return n.value

    def stream_hits(self) -> int:
        h = C.c_int32()
        _check(lib.coli_layer_stream_hits(self.handle, C.byref(h)), self.handle)
        return h.value

    def stream_stats(self):
        n = C.c_int32()
        b = C.c_int64()
        _check(lib.coli_layer_stream_stats(self.handle, C.byref(n), C.byref(b)), self.handle)
        return n.value, b.value

    def set_timing(self, enable: bool):
        _check(lib.coli_layer_set_timing(self.handle, int(bool(enable))), self.handle)

    def kernel_times(self) -> dict:
        """{kind: (total ms, launches)} since the last read; resets them."""
        ms = (C.c_double * len(KERNEL_KINDS))()
        n = (C.c_int64 * len(KERNEL_KINDS))()
        _check(lib.coli_layer_kernel_times(self.handle, ms, n), self.handle)
        return {k: (ms[i], n[i]) for i, k in enumerate(KERNEL_KINDS)}

    def device_errors(self) -> int:
        f = C.c_int32()
        _check(lib.coli_layer_device_errors(self.handle, C.byref(f)), self.handle)
        return f.value


def set_alloc_limit(nbytes: int) -> None:
    """Cap the device + pinned host bytes the library may hold (-1: none)."""
    _check(lib.coli_set_alloc_limit(int(nbytes)))


def alloc_bytes() -> int:
    return int(lib.coli_alloc_bytes())


def probe_read(buf, sink, stream=None):
    """coli_probe_read over the bytes of device tensor `buf` on `stream`
    (default: torch's current stream); XORs its 32-bit words into the
    one-element int32 device tensor `sink`."""
    import torch
    st = stream if stream is not None else torch.cuda.current_stream()
    _check(lib.coli_probe_read(C.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                               C.c_void_p(sink.data_ptr()), C.c_void_p(st.cuda_stream)))


def activations_to_device(x: np.ndarray, device=0):
    """numpy activations (float32, or uint16 bf16 bits) -> torch tensor on the GPU."""
    import torch
    if x.dtype == np.uint16:
        t = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(f"cuda:{device}")
