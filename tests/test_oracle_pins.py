"""Pins for the CPU oracle against things other than itself.

Each test ties one step of the oracle to a closed form, a library routine, a
brute-force enumeration, an invariant, or a hand-worked fixture under
tests/golden/, so that a dropped term, a wrong sign or index, or a transposed
operand anywhere in the oracle fails at least one of them.  No GPU involved.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

from int4_routed_expert_layer_amd import configs, inputs
from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_spec(**kw):
    return configs.TINY.with_(**kw)


# ------------------------------------------------------------------ scalars

def test_half_to_double_matches_numpy_for_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    got = np.array([orc.half_to_double(int(b)) for b in bits[finite][::7]])
    np.testing.assert_array_equal(got, ref[finite][::7])
    for b in (0x0001, 0x03FF, 0x0400, 0x7BFF, 0x8001, 0xFBFF, 0x3C00, 0xBC00):
        assert orc.half_to_double(b) == float(np.array([b], np.uint16).view(np.float16)[0])


def test_nibble_decode_of_all_256_bytes():
    for b in range(256):
        lo, hi = b & 15, b >> 4
        lo = lo - 16 if lo >= 8 else lo
        hi = hi - 16 if hi >= 8 else hi
        row = np.array([b], np.uint8)
        assert orc.nibble(row, 0) == lo
        assert orc.nibble(row, 1) == hi


def test_nibble_encode_roundtrip_over_all_int4_pairs():
    # Element 2j sits in the low nibble, 2j+1 in the high nibble.
    for a in range(-8, 8):
        for b in range(-8, 8):
            byte = ((b & 15) << 4) | (a & 15)
            row = np.array([byte], np.uint8)
            assert (orc.nibble(row, 0), orc.nibble(row, 1)) == (a, b)


# ------------------------------------------------------------------ route

def test_router_unit_vector_selects_one_row_of_w():
    rng = np.random.default_rng(1)
    H, E = 256, 16
    w = rng.standard_normal((H, E)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    for j in (0, 1, 63, 64, 130, 255):
        x = np.zeros((1, H), np.float32)
        x[0, j] = 1.0
        got = orc.router_logits(x, w, b)[0]
        np.testing.assert_array_equal(got, (w[j] + b).astype(np.float32))


def test_router_exact_on_small_integers():
    # All partial sums are small integers, so fp32 is exact in any order.
    rng = np.random.default_rng(2)
    H, E, B = 512, 24, 5
    x = rng.integers(-4, 5, (B, H)).astype(np.float32)
    w = rng.integers(-4, 5, (H, E)).astype(np.float32)
    ref = x.astype(np.int64) @ w.astype(np.int64)
    np.testing.assert_array_equal(orc.router_logits(x, w), ref.astype(np.float32))


def test_router_within_higham_bound_of_fp64_dot():
    spec = configs.DECODE_B1
    x = inputs.activations(spec.with_(n_tok=3))
    w = inputs.router_weight(spec)
    got = orc.router_logits(x, w).astype(np.float64)
    xf = inputs.bf16_bits_to_f32(x).astype(np.float64)
    exact = xf @ w.astype(np.float64)
    absdot = np.abs(xf) @ np.abs(w.astype(np.float64))
    n = spec.hidden // 64 + 6
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    assert np.all(np.abs(got - exact) <= gamma * absdot)
    # and the order is not plain fp64 (a wrong-precision oracle would pass
    # the bound trivially): at least some logits differ from fp64-rounded.
    assert np.any(got != exact.astype(np.float32).astype(np.float64))


def test_router_canonical_order_worked_example():
    with open(os.path.join(GOLDEN, "router_order_example.json")) as f:
        g = json.load(f)
    H = g["hidden"]
    x = np.zeros((1, H), np.float32)
    w = np.zeros((H, 1), np.float32)
    for k, v in g["nonzero_x"].items():
        x[0, int(k)] = v
    for k, v in g["nonzero_w"].items():
        w[int(k), 0] = v
    got = float(orc.router_logits(x, w)[0, 0])
    assert got == g["expected_canonical"]
    assert got != g["left_to_right_fp32"] and got != g["exact"]


def test_router_bf16_activations_equal_fp32_of_same_values():
    rng = np.random.default_rng(3)
    H, E = 256, 8
    bits = inputs.f32_to_bf16_bits(rng.standard_normal((4, H)).astype(np.float32))
    w = rng.standard_normal((H, E)).astype(np.float32)
    np.testing.assert_array_equal(orc.router_logits(bits, w),
                                  orc.router_logits(inputs.bf16_bits_to_f32(bits), w))


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0).
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-39], np.float32)
    got = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(v))
    np.testing.assert_array_equal(got[:3], np.array([1.0, 1.0 + 2 ** -6, -2.5], np.float32))


# ------------------------------------------------------------------ top-k

def key_better(la, a, lb, b):
    return la > lb or (la == lb and a < b)


def test_topk_brute_force_over_all_subsets_tiny():
    spec = configs.TINY
    x = inputs.activations(spec)
    w = inputs.router_weight(spec)
    logits = orc.router_logits(x, w)
    idx, _ = orc.topk(logits, spec.top_k)
    E, k = spec.n_experts, spec.top_k
    for t in range(spec.n_tok):
        l = logits[t]
        winners = []
        for S in itertools.combinations(range(E), k):
            rest = [e for e in range(E) if e not in S]
            if all(key_better(l[i], i, l[j], j) for i in S for j in rest):
                winners.append(set(S))
        assert len(winners) == 1
        assert set(idx[t].tolist()) == winners[0]
        # slot order is rank order
        for a, b in zip(idx[t][:-1], idx[t][1:]):
            assert key_better(l[a], a, l[b], b)


def test_topk_matches_numpy_lexsort():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((50, 64)).astype(np.float32)
    logits[:, 10] = logits[:, 3]            # exact ties
    idx, _ = orc.topk(logits, 8)
    for t in range(50):
        order = np.lexsort((np.arange(64), -logits[t].astype(np.float64)))
        np.testing.assert_array_equal(idx[t], order[:8])


def test_topk_ties_and_signed_zero_prefer_lower_id():
    logits = np.array([[0.0, -0.0, 0.0, -1.0, 5.0, 5.0]], np.float32)
    logits[0, 0] = -0.0
    idx, _ = orc.topk(logits, 4)
    assert idx[0].tolist() == [4, 5, 0, 1]


def test_topk_weights_are_normalised_sigmoids():
    rng = np.random.default_rng(5)
    logits = (3 * rng.standard_normal((40, 32))).astype(np.float32)
    idx, w = orc.topk(logits, 6)
    sel = np.take_along_axis(logits, idx, 1).astype(np.float64)
    ref = expit(sel)
    ref /= ref.sum(1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=1e-14, atol=0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=8 * 2.0 ** -52)


def test_topk_k_equals_e_is_a_full_sort():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((3, 16)).astype(np.float32)
    idx, w = orc.topk(logits, 16)
    for t in range(3):
        np.testing.assert_array_equal(idx[t], np.argsort(-logits[t], kind="stable"))
    s = expit(logits.astype(np.float64))
    np.testing.assert_allclose(np.take_along_axis(w, np.argsort(idx, 1), 1),
                               s / s.sum(1, keepdims=True), rtol=1e-14)


def test_topk_rejects_non_finite():
    with pytest.raises(RuntimeError):
        orc.topk(np.array([[0.0, np.nan, 1.0]], np.float32), 1)


# ------------------------------------------------------------------ union

def brute_union(idx, E):
    pairs = sorted((int(e), t, j) for t, row in enumerate(idx) for j, e in enumerate(row))
    k = idx.shape[1]
    ids = sorted({p[0] for p in pairs})
    counts = np.bincount([p[0] for p in pairs], minlength=E)
    return ids, counts, [t * k + j for _, t, j in pairs]


@pytest.mark.parametrize("seed,B,E,k", [(7, 8, 16, 4), (8, 1, 256, 8), (9, 37, 64, 6), (10, 0, 8, 2)])
def test_union_matches_brute_force(seed, B, E, k):
    rng = np.random.default_rng(seed)
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(B)], np.int32).reshape(B, k)
    u = orc.union(idx, E)
    ids, counts, gather = brute_union(idx, E)
    assert u["n_union"] == len(ids)
    np.testing.assert_array_equal(u["union_ids"], ids)
    np.testing.assert_array_equal(u["counts"], counts)
    np.testing.assert_array_equal(u["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(u["gather"], gather)
    assert sorted(u["gather"].tolist()) == list(range(B * k))


# ------------------------------------------------------------------ experts

def numpy_dequant(blob, H, I, which, group=32, bits=4):
    sec = configs.blob_sections(H, I, group, bits)
    rows, K = (H, I) if which == "down" else (I, H)
    off, size = sec[which + "_q"]
    if bits == 8:
        q = blob[off:off + size].view(np.int8).reshape(rows, K).astype(np.int64)
    else:
        b = blob[off:off + size].reshape(rows, K // 2)
        lo = (b & 15).astype(np.int64)
        hi = (b >> 4).astype(np.int64)
        q = np.empty((rows, K), np.int64)
        q[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
        q[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    soff, ssize = sec[which + "_s"]
    s = blob[soff:soff + ssize].view(np.float16).reshape(rows, K // group).astype(np.float64)
    return q * np.repeat(s, group, axis=1)


def test_blob_size_matches_pages_scale():
    # 3*H*I/2 nibble bytes = 18.9 MB, "~19 MB per expert" on the README.
    assert orc.blob_bytes(6144, 2048) == configs.blob_bytes(6144, 2048) == 21233664
    assert orc.blob_bytes(256, 128) == configs.blob_bytes(256, 128)


def test_group64_blob_size():
    # Group 64 halves the scale sections: 3*H*I/2 nibble bytes plus
    # 3*H*I/64 fp16 scales (every section already 256-byte aligned here).
    H, I = 6144, 2048
    assert orc.blob_bytes(H, I, 64) == configs.blob_bytes(H, I, 64) == 3 * H * I // 2 + 3 * H * I // 64 * 2
    assert orc.blob_bytes(384, 640, 64) == configs.blob_bytes(384, 640, 64)
    with pytest.raises(ValueError):
        orc.blob_bytes(6144, 2048, 48)      # 48 does not divide 2048


FORMATS = [(32, 4), (64, 4), (32, 8), (64, 8)]


@pytest.mark.parametrize("group,bits", FORMATS)
@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_dequant_matches_numpy(which, group, bits):
    spec = configs.TINY.with_(group=group, bits=bits)
    blob = inputs.expert_blob(spec, 0, 3)
    np.testing.assert_array_equal(orc.dequant(blob, spec.hidden, spec.inter, which, group, bits),
                                  numpy_dequant(blob, spec.hidden, spec.inter, which, group, bits))


def numpy_ffn(blob, H, I, x, group=32, bits=4):
    g = numpy_dequant(blob, H, I, "gate", group, bits) @ x
    v = numpy_dequant(blob, H, I, "up", group, bits) @ x
    h = g * expit(g) * v
    return numpy_dequant(blob, H, I, "down", group, bits) @ h


@pytest.mark.parametrize("group,bits", FORMATS)
def test_expert_ffn_matches_numpy_matmul(group, bits):
    spec = configs.TINY.with_(group=group, bits=bits)
    rng = np.random.default_rng(11)
    for e in (0, 5):
        blob = inputs.expert_blob(spec, 0, e)
        x = rng.standard_normal(spec.hidden)
        got = orc.expert_ffn(blob, spec.hidden, spec.inter, x, group, bits)
        ref = numpy_ffn(blob, spec.hidden, spec.inter, x, group, bits)
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def make_blob(H, I, gate_q, up_q, down_q, gate_s, up_s, down_s, group=32, bits=4):
    """Canonical blob from explicit int4 or int8 matrices and fp16 scales."""
    sec = configs.blob_sections(H, I, group, bits)
    blob = np.zeros(sec["total"][1], np.uint8)
    for name, q in (("gate_q", gate_q), ("up_q", up_q), ("down_q", down_q)):
        q = np.asarray(q, np.int64)
        packed = (q & 255) if bits == 8 else ((q[:, 1::2] & 15) << 4) | (q[:, 0::2] & 15)
        off, size = sec[name]
        blob[off:off + size] = packed.astype(np.uint8).ravel()
    for name, s in (("gate_s", gate_s), ("up_s", up_s), ("down_s", down_s)):
        off, size = sec[name]
        blob[off:off + size] = np.asarray(s, np.float16).ravel().view(np.uint8)
    return blob


def test_swiglu_closed_form_with_permutation_weights():
    # gate = P (row r reads x[pi(r)]), up = identity, down = identity, scales
    # 2^g per 32-group of the gate, 1 elsewhere:
    #   y[n] = silu(x[pi(n)] * 2^(pi(n)//32)) * x[n].
    H = I = 64
    rng = np.random.default_rng(12)
    pi = rng.permutation(H)
    gq = np.zeros((I, H), np.int64)
    gq[np.arange(I), pi] = 1
    eye = np.eye(H, dtype=np.int64)
    gs = np.tile(np.array([1.0, 2.0]), (I, 1))
    ones = np.ones((I, H // 32))
    blob = make_blob(H, I, gq, eye, eye, gs, ones, np.ones((H, I // 32)))
    x = rng.standard_normal(H)
    z = x[pi] * 2.0 ** (pi // 32)
    ref = z * expit(z) * x
    np.testing.assert_allclose(orc.expert_ffn(blob, H, I, x), ref, rtol=1e-15, atol=1e-300)


def test_swiglu_closed_form_group64():
    # As above with one scale per 64 columns: gate scales 1, 2, 4, 8 over
    # the four 64-column groups of a 256-wide row, so
    #   y[n] = silu(x[pi(n)] * 2^(pi(n)//64)) * x[n].
    H = I = 256
    rng = np.random.default_rng(13)
    pi = rng.permutation(H)
    gq = np.zeros((I, H), np.int64)
    gq[np.arange(I), pi] = 1
    eye = np.eye(H, dtype=np.int64)
    gs = np.tile(np.array([1.0, 2.0, 4.0, 8.0]), (I, 1))
    ones = np.ones((I, H // 64))
    blob = make_blob(H, I, gq, eye, eye, gs, ones, np.ones((H, I // 64)), group=64)
    x = rng.standard_normal(H)
    z = x[pi] * 2.0 ** (pi // 64)
    ref = z * expit(z) * x
    np.testing.assert_allclose(orc.expert_ffn(blob, H, I, x, 64), ref, rtol=1e-15, atol=1e-300)


def test_group64_is_group32_with_each_scale_repeated():
    # A group-64 matrix is the group-32 matrix whose scale pairs are equal:
    # same nibbles, each 64-group scale written twice, gives the same
    # dequantised weights and the same FFN output, bit for bit.
    H, I = 256, 128
    rng = np.random.default_rng(14)
    q = {n: rng.integers(-8, 8, size=sh) for n, sh in (("g", (I, H)), ("u", (I, H)), ("d", (H, I)))}
    s64 = {n: rng.uniform(0.005, 0.02, size=(sh[0], sh[1] // 64)).astype(np.float16)
           for n, sh in (("g", (I, H)), ("u", (I, H)), ("d", (H, I)))}
    b64 = make_blob(H, I, q["g"], q["u"], q["d"], s64["g"], s64["u"], s64["d"], group=64)
    b32 = make_blob(H, I, q["g"], q["u"], q["d"], *(np.repeat(s64[n], 2, axis=1) for n in "gud"))
    for which in ("gate", "up", "down"):
        np.testing.assert_array_equal(orc.dequant(b64, H, I, which, 64), orc.dequant(b32, H, I, which, 32))
    x = rng.standard_normal(H)
    np.testing.assert_array_equal(orc.expert_ffn(b64, H, I, x, 64), orc.expert_ffn(b32, H, I, x, 32))


def test_int8_blob_size_and_extremes():
    # int8: one byte per weight, the same scale sections as int4.
    H, I = 6144, 2048
    assert orc.blob_bytes(H, I, 32, 8) == configs.blob_bytes(H, I, 32, 8) == 3 * H * I + 3 * H * I // 32 * 2
    assert orc.blob_bytes(H, I, 64, 8) == configs.blob_bytes(H, I, 64, 8) == 3 * H * I + 3 * H * I // 64 * 2
    with pytest.raises(ValueError):
        orc.blob_bytes(H, I, 32, 6)
    H = I = 64
    gq = np.tile(np.array([-128, 127, -1, 0]), (I, H // 4))
    s = np.full((I, 2), 0.0009765625)  # 2^-10, exact in fp16
    blob = make_blob(H, I, gq, gq, gq.T, s, s, s, bits=8)
    d = orc.dequant(blob, H, I, "gate", 32, 8)
    assert d[0, 0] == -128 * 2.0 ** -10 and d[0, 1] == 127 * 2.0 ** -10 and d[0, 2] == -2.0 ** -10


def test_int8_holding_int4_values_equals_int4():
    # The same integers in [-8, 7] stored one per byte and two per byte, with
    # the same scales, are the same matrices and the same expert, bit for bit.
    H, I = 256, 128
    rng = np.random.default_rng(15)
    q = {n: rng.integers(-8, 8, size=sh) for n, sh in (("g", (I, H)), ("u", (I, H)), ("d", (H, I)))}
    sc = {n: rng.uniform(0.005, 0.02, size=(sh[0], sh[1] // 32)).astype(np.float16)
          for n, sh in (("g", (I, H)), ("u", (I, H)), ("d", (H, I)))}
    b4 = make_blob(H, I, q["g"], q["u"], q["d"], sc["g"], sc["u"], sc["d"])
    b8 = make_blob(H, I, q["g"], q["u"], q["d"], sc["g"], sc["u"], sc["d"], bits=8)
    for which in ("gate", "up", "down"):
        np.testing.assert_array_equal(orc.dequant(b8, H, I, which, 32, 8), orc.dequant(b4, H, I, which, 32, 4))
    x = rng.standard_normal(H)
    np.testing.assert_array_equal(orc.expert_ffn(b8, H, I, x, 32, 8), orc.expert_ffn(b4, H, I, x, 32, 4))


def test_int4_extremes_and_scale_product_are_exact():
    H = I = 32
    gq = np.full((I, H), -8)
    gq[:, 1::2] = 7
    s = np.full((I, 1), 0.0126953125)  # exactly representable in fp16
    blob = make_blob(H, I, gq, gq, gq.T, s, s, s)
    d = orc.dequant(blob, H, I, "gate")
    assert d[0, 0] == -8 * 0.0126953125 and d[0, 1] == 7 * 0.0126953125


# ------------------------------------------------------------------ layer

def layer_inputs(spec, layer=0):
    x = inputs.activations(spec, layer)
    w = inputs.router_weight(spec, layer)
    b = inputs.router_bias(spec, layer)
    blobs = inputs.expert_blobs(spec, layer, range(spec.n_experts), threads=1)
    shared = inputs.expert_blob(spec, layer, inputs.SHARED) if spec.has_shared else None
    return x, w, b, blobs, shared


def x64(x):
    return (inputs.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)


def test_layer_single_expert_is_plain_swiglu():
    spec = tiny_spec(n_experts=1, top_k=1)
    x, w, b, blobs, _ = layer_inputs(spec)
    r = orc.run_layer(x, w, b, 1, blobs, None, spec.hidden, spec.inter)
    assert np.all(r["weight"] == 1.0)
    for t in range(spec.n_tok):
        ref = numpy_ffn(blobs[0], spec.hidden, spec.inter, x64(x)[t])
        assert np.max(np.abs(r["y"][t] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_layer_k_equals_e_is_dense_soft_moe():
    spec = tiny_spec(n_experts=6, top_k=6, n_tok=3)
    x, w, b, blobs, _ = layer_inputs(spec)
    r = orc.run_layer(x, w, b, 6, blobs, None, spec.hidden, spec.inter)
    xf = x64(x)
    logits = xf @ w.astype(np.float64)
    gate = expit(logits)
    gate /= gate.sum(1, keepdims=True)
    for t in range(3):
        ref = sum(gate[t, e] * numpy_ffn(blobs[e], spec.hidden, spec.inter, xf[t])
                  for e in range(6))
        assert np.max(np.abs(r["y"][t] - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_layer_shared_expert_adds_with_weight_one():
    spec = tiny_spec(has_shared=True)
    x, w, b, blobs, shared = layer_inputs(spec)
    zero = {e: make_blob(spec.hidden, spec.inter,
                         np.zeros((spec.inter, spec.hidden)), np.zeros((spec.inter, spec.hidden)),
                         np.zeros((spec.hidden, spec.inter)),
                         np.ones((spec.inter, spec.hidden // 32)),
                         np.ones((spec.inter, spec.hidden // 32)),
                         np.ones((spec.hidden, spec.inter // 32)))
            for e in range(spec.n_experts)}
    r = orc.run_layer(x, w, b, spec.top_k, zero, shared, spec.hidden, spec.inter)
    for t in range(spec.n_tok):
        ref = numpy_ffn(shared, spec.hidden, spec.inter, x64(x)[t])
        assert np.max(np.abs(r["y"][t] - ref)) <= 1e-12 * np.max(np.abs(ref))
    full = orc.run_layer(x, w, b, spec.top_k, blobs, shared, spec.hidden, spec.inter)
    none = orc.run_layer(x, w, b, spec.top_k, blobs, None, spec.hidden, spec.inter)
    np.testing.assert_allclose(full["y"] - none["y"], r["y"], rtol=1e-12, atol=1e-12)


def test_layer_doubling_down_scales_doubles_output_exactly():
    spec = configs.TINY
    x, w, b, blobs, _ = layer_inputs(spec)
    sec = configs.blob_sections(spec.hidden, spec.inter)
    off, size = sec["down_s"]
    doubled = {}
    for e, blob in blobs.items():
        d = blob.copy()
        s = d[off:off + size].view(np.float16) * np.float16(2)
        d[off:off + size] = s.view(np.uint8)
        doubled[e] = d
    r1 = orc.run_layer(x, w, b, spec.top_k, blobs, None, spec.hidden, spec.inter)
    r2 = orc.run_layer(x, w, b, spec.top_k, doubled, None, spec.hidden, spec.inter)
    np.testing.assert_array_equal(r2["y"], 2 * r1["y"])


def test_layer_expert_relabelling_is_invariant():
    spec = configs.TINY
    x, w, b, blobs, _ = layer_inputs(spec)
    perm = np.random.default_rng(13).permutation(spec.n_experts)   # new id -> old id
    w2 = w[:, perm].copy()
    blobs2 = {new: blobs[int(old)] for new, old in enumerate(perm)}
    r1 = orc.run_layer(x, w, b, spec.top_k, blobs, None, spec.hidden, spec.inter)
    r2 = orc.run_layer(x, w2, b, spec.top_k, blobs2, None, spec.hidden, spec.inter)
    np.testing.assert_array_equal(perm[r2["idx"]], r1["idx"])
    np.testing.assert_array_equal(r2["y"], r1["y"])


@pytest.mark.parametrize("group,bits", FORMATS)
def test_layer_matches_numpy_composition_on_tiny(group, bits):
    spec = configs.TINY.with_(group=group, bits=bits)
    x, w, b, blobs, _ = layer_inputs(spec)
    r = orc.run_layer(x, w, b, spec.top_k, blobs, None, spec.hidden, spec.inter, group=group, bits=bits)
    xf = x64(x)
    for t in range(spec.n_tok):
        ref = sum(r["weight"][t, j] * numpy_ffn(blobs[int(e)], spec.hidden, spec.inter, xf[t], group, bits)
                  for j, e in enumerate(r["idx"][t]))
        assert np.max(np.abs(r["y"][t] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_layer_token_subset_equals_full_rows():
    spec = configs.TINY
    x, w, b, blobs, _ = layer_inputs(spec)
    full = orc.run_layer(x, w, b, spec.top_k, blobs, None, spec.hidden, spec.inter)
    part = orc.layer_tokens(x, spec.hidden, spec.inter, full["idx"], full["weight"],
                            blobs, None, [6, 1])
    np.testing.assert_array_equal(part, full["y"][[6, 1]])


# ------------------------------------------------------------------ inputs

def test_generator_is_deterministic_and_per_expert():
    spec = configs.DECODE_B1.with_(hidden=256, inter=128)
    a = inputs.expert_blobs(spec, 2, [0, 5, inputs.SHARED], threads=3)
    for e in (0, 5, inputs.SHARED):
        np.testing.assert_array_equal(a[e], inputs.expert_blob(spec, 2, e))
    assert not np.array_equal(a[0], a[5])
    assert not np.array_equal(inputs.expert_blob(spec, 1, 0), a[0])
    np.testing.assert_array_equal(inputs.activations(spec, 0), inputs.activations(spec, 0))


def test_int8_generator_value_ranges():
    spec = configs.TINY.with_(bits=8)
    blob = inputs.expert_blob(spec, 0, 1)
    sec = configs.blob_sections(spec.hidden, spec.inter, spec.group, 8)
    for name in ("gate_s", "up_s", "down_s"):
        off, size = sec[name]
        s = blob[off:off + size].view(np.float16).astype(np.float64)
        assert s.min() >= 0.005 / 16 - 1e-6 and s.max() <= 0.02 / 16 + 1e-6
    off, size = sec["gate_q"]
    counts = np.bincount(blob[off:off + size], minlength=256)
    assert counts.min() > 0 and counts.max() < 3 * counts.mean()


def test_generator_value_ranges():
    spec = configs.TINY
    blob = inputs.expert_blob(spec, 0, 1)
    sec = configs.blob_sections(spec.hidden, spec.inter)
    for name in ("gate_s", "up_s", "down_s"):
        off, size = sec[name]
        s = blob[off:off + size].view(np.float16).astype(np.float64)
        assert s.min() >= 0.005 - 1e-5 and s.max() <= 0.02 + 1e-5
    off, size = sec["gate_q"]
    nib = np.concatenate([blob[off:off + size] & 15, blob[off:off + size] >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.8 * counts.mean()


def test_zipf_bias_gives_rank_frequency_slope_near_minus_s():
    # Logits x.W_r are N(0,1) by construction; draw them directly.
    spec = configs.DECODE_B64
    b = inputs.router_bias(spec).astype(np.float64)
    rank = inputs.zipf_ranks(spec)
    rng = np.random.default_rng(14)
    hits = np.zeros(spec.n_experts)
    for _ in range(20):
        l = rng.standard_normal((5000, spec.n_experts)) + b
        top = np.argpartition(-l, spec.top_k, axis=1)[:, :spec.top_k]
        hits += np.bincount(top.ravel(), minlength=spec.n_experts)
    freq = hits[np.argsort(rank)]
    r = np.arange(1, 65)
    slope = np.polyfit(np.log(r), np.log(freq[:64]), 1)[0]
    assert abs(slope + spec.zipf_s) < 0.08, slope


def test_resident_split_is_sixty_percent():
    spec = configs.TIERED_12L
    m = inputs.resident_mask(spec, 3)
    assert m.sum() == round(0.6 * 256)
    assert not np.array_equal(m, inputs.resident_mask(spec, 4))
