"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the header declares, validates arguments before touching a
device, and its host repack writes the documented device layout."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

from int4_routed_expert_layer_amd import binding as B
from int4_routed_expert_layer_amd import configs, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coli_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coli_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 16
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(coli_\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(B.SIGNATURES)


def test_abi_version_and_status_strings():
    assert B.lib.coli_abi_version() == 5
    for st, name in enumerate(["COLI_OK", "COLI_E_INVALID", "COLI_E_NOMEM", "COLI_E_DEVICE",
                               "COLI_E_STATE", "COLI_E_UNSUPPORTED"]):
        assert B.status_str(st) == name


def test_blob_bytes_matches_layout():
    for g in (32, 64):
        for bits in (4, 8):
            for h, i in ((6144, 2048), (256, 128), (512, 256), (384, 640)):
                assert B.blob_bytes(h, i, g, bits) == configs.blob_bytes(h, i, g, bits)
    assert B.blob_bytes(6144, 2048, 64, 8) == 3 * 6144 * 2048 + 3 * 6144 * 2048 // 64 * 2
    assert B.blob_bytes(6144, 2048, 32, 6) == 0
    assert B.blob_bytes(6144, 2048) == 21233664
    assert B.blob_bytes(6144, 2048, 64) == 20054016
    assert B.blob_bytes(0, 128) == 0 and B.blob_bytes(100, 128) == 0
    assert B.blob_bytes(6144, 2048, 16) == 0 and B.blob_bytes(6144, 2048, 128) == 0
    assert B.blob_bytes(6144, 2080, 64) == 0


def create(**kw):
    d = dict(hidden=256, inter=128, n_experts=16, top_k=4, has_shared=0, max_tokens=8, act=0, group=32,
             weight_bits=4)
    d.update(kw)
    h = C.c_void_p()
    st = B.lib.coli_layer_create(C.byref(B.Dims(**d)), 0, C.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=17), B.E_INVALID),
    (dict(top_k=0), B.E_INVALID),
    (dict(top_k=33, n_experts=64), B.E_INVALID),
    (dict(max_tokens=0), B.E_INVALID),
    (dict(has_shared=2), B.E_INVALID),
    (dict(act=7), B.E_INVALID),
    (dict(group=0), B.E_INVALID),
    (dict(group=128), B.E_INVALID),
    (dict(weight_bits=2), B.E_INVALID),
    (dict(hidden=192), B.E_UNSUPPORTED),
    (dict(inter=96), B.E_UNSUPPORTED),
    (dict(n_experts=1024, has_shared=1), B.E_UNSUPPORTED),
])
def test_create_validates_dims_before_the_device(kw, status):
    st, h = create(**kw)
    assert st == status
    assert not h.value
    assert B.lib.coli_last_error(None)


def test_create_without_a_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, h = create()
    assert st == B.E_DEVICE and not h.value


def test_null_layer_calls_are_invalid():
    L = B.lib
    assert L.coli_router_set(None, None, None) == B.E_INVALID
    assert L.coli_expert_place(None, 0, None, 0, 0) == B.E_INVALID
    assert L.coli_moe_route(None, None, 1, None, None, None) == B.E_INVALID
    assert L.coli_moe_router_logits(None, None, 1, None, None) == B.E_INVALID
    assert L.coli_moe_union(None, None, 1, None, None, None, None, None, None) == B.E_INVALID
    assert L.coli_moe_forward(None, None, 1, *([None] * 8), None, None) == B.E_INVALID
    assert L.coli_layer_set_path(None, 0) == B.E_INVALID
    assert L.coli_layer_stream_stats(None, None, None) == B.E_INVALID
    assert L.coli_layer_device_errors(None, None) == B.E_INVALID
    assert L.coli_layer_destroy(None) == B.OK


def test_probe_read_validates_before_the_device():
    import ctypes as C
    L = B.lib
    fake, sink = C.c_void_p(4096), C.c_void_p(8192)     # never dereferenced on the host
    assert L.coli_probe_read(None, 16, sink, None) == B.E_INVALID
    assert L.coli_probe_read(fake, 16, None, None) == B.E_INVALID
    assert L.coli_probe_read(fake, 24, sink, None) == B.E_INVALID          # not a multiple of 16
    assert L.coli_probe_read(C.c_void_p(4100), 16, sink, None) == B.E_INVALID   # misaligned


def documented_layout_i8(blob, H, I, group):
    """The int8 device layout described in coli_moe.h, written with numpy."""
    sec = configs.blob_sections(H, I, group, 8)
    per = 64 // group
    out = np.zeros_like(blob)
    for name, rows, K in (("gate", I, H), ("up", I, H), ("down", H, I)):
        qo, qs = sec[name + "_q"]
        so, ss = sec[name + "_s"]
        u = blob[qo:qo + qs].reshape(rows, K) ^ 0x80             # q + 128
        P, Cn = rows // 16, K // 64
        L = np.arange(64)
        s = np.arange(4)
        order = np.array([0, 2, 1, 3])                         # byte b holds column k0 + order[b]
        r = np.arange(P)[:, None, None, None, None] * 16 + (L % 16)[None, None, :, None, None]
        k = (np.arange(Cn)[None, :, None, None, None] * 64 + 32 * (s // 2)[None, None, None, :, None]
             + 8 * (L // 16)[None, None, :, None, None] + 4 * (s % 2)[None, None, None, :, None]
             + order[None, None, None, None, :])
        out[qo:qo + qs] = u[r, k].astype(np.uint8).reshape(-1)      # [P, C, lane, dword, byte]
        sc = blob[so:so + ss].view(np.uint16).reshape(rows, K // group)
        tiles = sc.reshape(P, 16, Cn, per).transpose(0, 2, 1, 3)
        out[so:so + ss] = np.ascontiguousarray(tiles).reshape(-1).view(np.uint8)
    return out


def documented_layout(blob, H, I, group=32, bits=4):
    """The device layout described in coli_moe.h, written with numpy."""
    if bits == 8:
        return documented_layout_i8(blob, H, I, group)
    sec = configs.blob_sections(H, I, group)
    per = 128 // group                                      # scales per row of a tile
    out = np.zeros_like(blob)
    for name, rows, K in (("gate", I, H), ("up", I, H), ("down", H, I)):
        qo, qs = sec[name + "_q"]
        so, ss = sec[name + "_s"]
        b = blob[qo:qo + qs].reshape(rows, K // 2)
        q = np.empty((rows, K), np.int64)
        q[:, 0::2] = b & 15
        q[:, 1::2] = b >> 4
        u = q ^ 8                                           # q + 8 for two's complement
        P, Cn = rows // 16, K // 128
        L = np.arange(64)
        s = np.arange(4)
        i = np.arange(8)
        r = (np.arange(P)[:, None, None, None, None] * 16 + (L % 16)[None, None, :, None, None])
        k = (np.arange(Cn)[None, :, None, None, None] * 128 + 32 * s[None, None, None, :, None]
             + 8 * (L // 16)[None, None, :, None, None] + i[None, None, None, None, :])
        vals = u[r, k]                                      # [P, C, 64, 4, 8]
        slot = np.where(i % 2 == 0, i // 2, 4 + i // 2)
        words = (vals << (4 * slot)).sum(-1).astype(np.uint32)
        out[qo:qo + qs] = words.reshape(-1).view(np.uint8)
        sc = blob[so:so + ss].view(np.uint16).reshape(rows, K // group)
        tiles = sc.reshape(P, 16, Cn, per).transpose(0, 2, 1, 3)   # [P, C, row, group]
        out[so:so + ss] = np.ascontiguousarray(tiles).reshape(-1).view(np.uint8)
    return out


@pytest.mark.parametrize("group,bits", [(32, 4), (64, 4), (32, 8), (64, 8)])
@pytest.mark.parametrize("spec", [configs.TINY, configs.TINY.with_(hidden=512, inter=384)])
def test_repack_writes_the_documented_layout(spec, group, bits):
    spec = spec.with_(group=group, bits=bits)
    blob = inputs.expert_blob(spec, 0, 2)
    got = B.repack(blob, spec.hidden, spec.inter, group, bits)
    np.testing.assert_array_equal(got, documented_layout(blob, spec.hidden, spec.inter, group, bits))


def test_repack_rejects_bad_sizes():
    buf = np.zeros(1024, np.uint8)
    assert B.lib.coli_expert_repack(buf.ctypes.data, buf.ctypes.data, 96, 128, 32, 4) == B.E_INVALID
    assert B.lib.coli_expert_repack(None, buf.ctypes.data, 128, 128, 32, 4) == B.E_INVALID
    assert B.lib.coli_expert_repack(buf.ctypes.data, buf.ctypes.data, 128, 128, 48, 4) == B.E_INVALID
    assert B.lib.coli_expert_repack(buf.ctypes.data, buf.ctypes.data, 128, 128, 32, 16) == B.E_INVALID


def test_create_refuses_shapes_past_32_bit_row_offsets():
    # The grouped kernels index activation and h rows with 32-bit element
    # offsets: (max_tokens * (k + 1) + 2) * max(H, I) (the rows of a call, the
    # discard row and the zero row) must stay below 2^32.
    st, h = create(hidden=2048, inter=1024, n_experts=16, top_k=8, max_tokens=262144)
    assert st == B.E_UNSUPPORTED and not h.value
    assert b"2^32" in B.lib.coli_last_error(None)
    # The exact boundary: 2^32 / 2048 = 2^21 rows; with k = 2, 699050 tokens
    # make 3 * 699050 + 2 = 2^21 rows.  With the allocation cap far below the
    # layer's scratch, an accepted shape stops at the cap (E_NOMEM, before any
    # device call) and a refused one at the shape check.
    assert 3 * 699050 + 2 == 2 ** 21
    B.set_alloc_limit(1 << 20)
    try:
        st, h = create(hidden=2048, inter=1024, n_experts=16, top_k=2, max_tokens=699049)
        assert st == B.E_NOMEM and not h.value
        st, h = create(hidden=2048, inter=1024, n_experts=16, top_k=2, max_tokens=699050)
        assert st == B.E_UNSUPPORTED and not h.value
    finally:
        B.set_alloc_limit(-1)


def test_alloc_cap_fails_create_with_nomem_before_the_device():
    assert B.alloc_bytes() == 0
    B.set_alloc_limit(1 << 20)      # far below the layer's scratch
    try:
        st, h = create(max_tokens=4096)
        assert st == B.E_NOMEM and not h.value
        assert b"allocation cap" in B.lib.coli_last_error(None)
    finally:
        B.set_alloc_limit(-1)
    assert B.lib.coli_set_alloc_limit(-2) == B.E_INVALID
    assert B.alloc_bytes() == 0
