"""GPU parity: the HIP library against the CPU oracle on seeded inputs.

Routing (logits, top-k ids), the union (ids, counts, offsets, gather) are
compared bit for bit; routing weights to fp32 rounding; layer outputs to
max|y_gpu - y_ref| <= 2e-3 * max|y_ref|.  Every call goes through the C ABI.
"""
import numpy as np
import pytest

from int4_routed_expert_layer_amd import configs, inputs
from moe_case import (Data, check_outputs, check_routing, edge_tokens, gpu_run, log, make_layer,
                      oracle_route, oracle_y)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from int4_routed_expert_layer_amd import binding as B  # noqa: E402

PATHS = {"gemv": B.PATH_GEMV, "grouped": B.PATH_GROUPED}

MEDIUM = configs.Spec("medium_h512_i256_e32_k4_b37", 512, 256, 32, 4, 37, "bf16", True,
                      "zipf", seed=777)


def full_check(spec, path, tokens=None, n_tok=None):
    data = Data(spec, n_tok=n_tok)
    log(f"case {spec.name} path={path} n_tok={data.x.shape[0]}")
    L = make_layer(B, data, path=PATHS[path] if path else None)
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    toks = range(data.x.shape[0]) if tokens is None else tokens
    y_ref = oracle_y(data, ref, toks)
    check_outputs(gpu["y"][list(toks)], y_ref, f"{spec.name}/{path}")
    L.close()


@pytest.mark.parametrize("path", ["gemv", "grouped"])
def test_tiny_parity(path):
    full_check(configs.TINY, path)


@pytest.mark.parametrize("path", ["gemv", "grouped"])
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_medium_ragged_parity(path, act):
    full_check(MEDIUM.with_(act=act), path)


@pytest.mark.parametrize("path", ["gemv", "grouped"])
def test_medium_single_token(path):
    full_check(MEDIUM, path, n_tok=1)


@pytest.mark.parametrize("path", ["gemv", "grouped", None])
@pytest.mark.parametrize("hidden,inter,n_tok", [(384, 384, 3), (640, 128, 29), (384, 640, 45)])
def test_hidden_not_multiple_of_256(path, hidden, inter, n_tok):
    # A hidden width of 128 mod 256 leaves the grouped down pass a last
    # 256-column block that is half empty; odd multiples of 128 for the
    # intermediate width give gate/up an odd block count.
    spec = MEDIUM.with_(name=f"h{hidden}_i{inter}_e24_k6_b{n_tok}", hidden=hidden, inter=inter,
                        n_experts=24, top_k=6, n_tok=n_tok, has_shared=True, act="bf16")
    full_check(spec, path)


def test_special_case_e1_k1():
    full_check(configs.TINY.with_(n_experts=1, top_k=1, has_shared=True, act="bf16"), "gemv")
    full_check(configs.TINY.with_(n_experts=1, top_k=1, has_shared=True, act="bf16"), "grouped")


@pytest.mark.parametrize("path", ["gemv", "grouped"])
def test_special_case_k_equals_e(path):
    full_check(configs.TINY.with_(n_experts=8, top_k=8, n_tok=5), path)


@pytest.fixture(scope="module")
def decode_b1():
    data = Data(configs.DECODE_B1)
    log("case decode_b1: placing 257 experts")
    L = make_layer(B, data)
    yield data, L
    L.close()


@pytest.mark.parametrize("path", ["auto", "gemv", "grouped"])
def test_decode_b1_parity(decode_b1, path):
    data, L = decode_b1
    L.set_path({"auto": B.PATH_AUTO, **PATHS}[path])
    log(f"case decode_b1 path={path}")
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    check_outputs(gpu["y"], oracle_y(data, ref, [0]), f"decode_b1/{path}")


def test_decode_b1_fused_layer_call(decode_b1):
    data, L = decode_b1
    L.set_path(B.PATH_AUTO)
    x = B.activations_to_device(data.x)
    y, idx, w, u = L.layer(x)
    torch.cuda.synchronize()
    assert L.device_errors() == 0
    three = gpu_run(B, L, data, with_logits=False)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), three["y"].view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), three["idx"])
    assert np.array_equal(w.cpu().numpy().view(np.uint32), three["weight"].view(np.uint32))
    ref = oracle_route(data)
    check_outputs(y.cpu().numpy(), oracle_y(data, ref, [0]), "decode_b1/fused")


@pytest.mark.parametrize("n_tok", [1, 2, 3, 4])
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_fused_layer_small_batches(n_tok, act):
    spec = MEDIUM.with_(act=act)
    data = Data(spec, n_tok=n_tok)
    log(f"case fused layer {spec.name} n_tok={n_tok}")
    L = make_layer(B, data, path=B.PATH_GEMV)
    x = B.activations_to_device(data.x)
    outs = []
    for _ in range(2):      # twice: arrival counters must reset between calls
        y, idx, w, u = L.layer(x)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert L.device_errors() == 0
    three = gpu_run(B, L, data, with_logits=False)
    assert np.array_equal(outs[0].view(np.uint32), three["y"].view(np.uint32))
    nu = int(u["n_union"].cpu()[0])
    assert nu == three["n_union"]
    np.testing.assert_array_equal(u["union_ids"].cpu().numpy()[:nu], three["union_ids"])
    np.testing.assert_array_equal(u["gather"].cpu().numpy(), three["gather"])
    np.testing.assert_array_equal(u["offsets"].cpu().numpy(), three["offsets"])
    ref = oracle_route(data)
    check_routing(three, ref, check_logits=False)
    check_outputs(outs[0], oracle_y(data, ref, range(n_tok)), f"fused n_tok={n_tok}")
    L.close()


@pytest.mark.parametrize("E,k", [(37, 5), (100, 32), (256, 32), (256, 1)])
@pytest.mark.parametrize("n_tok", [1, 3, 4])
def test_fused_layer_odd_shapes(E, k, n_tok):
    """The one-launch front with expert counts that are not a multiple of the
    64-wide waves (partly empty router blocks and selection lanes) and with
    the largest k: bit-identical to the three separate calls, and routing and
    output against the oracle."""
    spec = MEDIUM.with_(name=f"fused_e{E}_k{k}", n_experts=E, top_k=k, routing="gauss")
    data = Data(spec, n_tok=n_tok)
    log(f"case fused odd shape E={E} k={k} n_tok={n_tok}")
    L = make_layer(B, data)
    x = B.activations_to_device(data.x)
    y, idx, w, u = L.layer(x)
    torch.cuda.synchronize()
    assert L.device_errors() == 0
    three = gpu_run(B, L, data, with_logits=False)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), three["y"].view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), three["idx"])
    assert np.array_equal(w.cpu().numpy().view(np.uint32), three["weight"].view(np.uint32))
    nu = int(u["n_union"].cpu()[0])
    assert nu == three["n_union"]
    np.testing.assert_array_equal(u["gather"].cpu().numpy(), three["gather"])
    np.testing.assert_array_equal(u["offsets"].cpu().numpy(), three["offsets"])
    np.testing.assert_array_equal(u["counts"].cpu().numpy(), three["counts"])
    ref = oracle_route(data)
    check_routing(three, ref, check_logits=False)
    check_outputs(y.cpu().numpy(), oracle_y(data, ref, range(n_tok)), f"fused E={E} k={k} n={n_tok}")
    L.close()


@pytest.mark.parametrize("path", ["auto", "gemv"])
@pytest.mark.parametrize("n_tok", [3, 4])
def test_fused_layer_identical_tokens(path, n_tok):
    """Tokens that route alike: every union expert gets all n_tok tokens, so
    the gate/up GEMV takes two passes per panel (two tokens per pass) and
    the front splits the shared gate/up over two blocks per panel.  The fused
    call is bit-identical to the three separate calls and within tolerance
    of the oracle."""
    data = Data(MEDIUM, n_tok=n_tok)
    data.x[:] = data.x[0]
    log(f"case fused identical tokens n_tok={n_tok} path={path}")
    L = make_layer(B, data, path=PATHS.get(path))
    x = B.activations_to_device(data.x)
    y, idx, w, u = L.layer(x)
    torch.cuda.synchronize()
    assert L.device_errors() == 0
    nu = int(u["n_union"].cpu()[0])
    assert nu == MEDIUM.top_k
    np.testing.assert_array_equal(u["counts"].cpu().numpy()[u["union_ids"].cpu().numpy()[:nu]], n_tok)
    three = gpu_run(B, L, data, with_logits=False)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), three["y"].view(np.uint32))
    ref = oracle_route(data)
    check_routing(three, ref, check_logits=False)
    y_ref = oracle_y(data, ref, range(n_tok))
    check_outputs(y.cpu().numpy(), y_ref, f"identical tokens n_tok={n_tok}")
    assert np.array_equal(y.cpu().numpy()[1:].view(np.uint32), np.repeat(y.cpu().numpy()[:1], n_tok - 1, 0).view(np.uint32))
    L.close()


def test_fused_layer_alternating_sizes():
    """One layer, fused calls of changing batch size back to back: the launch
    counters must be clean after every call."""
    spec = MEDIUM.with_(act="bf16")
    data = Data(spec, n_tok=4)
    L = make_layer(B, data, path=B.PATH_GEMV, max_tokens=4)
    ref = oracle_route(data)
    y_ref = oracle_y(data, ref, range(4))
    for n in (1, 4, 2, 3, 1, 4):
        x = B.activations_to_device(data.x[:n])
        y, idx, w, u = L.layer(x)
        torch.cuda.synchronize()
        log(f"  fused call n_tok={n}")
        assert L.device_errors() == 0
        # routing of a token does not depend on the other tokens of the batch
        np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"][:n])
        check_outputs(y.cpu().numpy(), y_ref[:n], f"alternating n_tok={n}")
    L.close()


def test_decode_b1_deterministic(decode_b1):
    data, L = decode_b1
    L.set_path(B.PATH_AUTO)
    a = gpu_run(B, L, data, with_logits=False)
    b = gpu_run(B, L, data, with_logits=False)
    assert np.array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32))


@pytest.mark.parametrize("path", ["auto", "gemv"])
def test_decode_b64_zipf_parity(path):
    spec = configs.DECODE_B64
    data = Data(spec)
    log(f"case decode_b64 path={path}")
    L = make_layer(B, data, path={"auto": B.PATH_AUTO, **PATHS}[path])
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    log(f"  union size {ref['n_union']} of {spec.n_tok * spec.top_k} selections")
    assert ref["n_union"] < spec.n_tok * spec.top_k // 2
    tokens = list(range(spec.n_tok))          # every token of the batch
    check_outputs(gpu["y"][tokens], oracle_y(data, ref, tokens), f"decode_b64/{path}")
    L.close()


def test_prefill_b4096_parity():
    spec = configs.PREFILL_B4096
    data = Data(spec)
    log("case prefill_b4096: placing 257 experts")
    L = make_layer(B, data)
    gpu = gpu_run(B, L, data)
    log("  oracle routing over 4096 tokens")
    ref = oracle_route(data)
    check_routing(gpu, ref)
    c = ref["counts"]
    log(f"  tokens per expert: min {c.min()} max {c.max()}")
    # Every expert's first and last gather row and both sides of each
    # 160-row chunk boundary: each grouped work chunk of every expert has
    # its first and last tile compared.
    tokens = edge_tokens(ref, spec.top_k, extra=[0, 1, 777, 2048, 3001, 4095])
    log(f"  comparing {len(tokens)} tokens")
    check_outputs(gpu["y"][tokens], oracle_y(data, ref, tokens), "prefill_b4096")
    L.close()


@pytest.mark.parametrize("layer", range(configs.TIERED_12L.n_layers))
def test_tiered_layer_matches_resident_and_oracle(layer):
    spec = configs.TIERED_12L
    data = Data(spec, layer)
    resident = inputs.resident_mask(spec, layer)
    log(f"case tiered layer {layer}: {resident.sum()} resident / {spec.n_experts}")
    L = make_layer(B, data)
    all_vram = gpu_run(B, L, data, with_logits=False)
    # Move the 40% host-tier experts to pinned host memory.
    host = [e for e in range(spec.n_experts) if not resident[e]]
    for i in range(0, len(host), 32):
        for e, blob in data.blobs(host[i:i + 32]).items():
            L.place(e, blob, B.TIER_HOST)
        data.drop_blobs()
    tiered = gpu_run(B, L, data, with_logits=False)
    n_streamed, nbytes = L.stream_stats()
    log(f"  streamed {n_streamed} experts, {nbytes / 1e6:.1f} MB")
    assert n_streamed == sum(1 for e in all_vram["union_ids"] if not resident[e])
    for key in ("idx", "weight", "union_ids", "counts", "offsets", "gather", "y"):
        assert np.array_equal(np.asarray(tiered[key]).view(np.uint8),
                              np.asarray(all_vram[key]).view(np.uint8)), key
    ref = oracle_route(data)
    check_routing(tiered, ref, check_logits=False)
    check_outputs(tiered["y"], oracle_y(data, ref, range(spec.n_tok)), f"tiered/L{layer}")
    L.close()


def test_tie_break_prefers_lower_expert_id():
    spec = configs.TINY.with_(act="bf16")
    data = Data(spec)
    data.w[:, 9] = data.w[:, 2]      # experts 2 and 9 always tie exactly
    data.w[:, 12] = data.w[:, 5]
    L = make_layer(B, data)
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    L.close()


def test_zero_tokens_is_a_no_op():
    data = Data(configs.TINY)
    L = make_layer(B, data)
    x = B.activations_to_device(data.x[:0])
    idx, w = L.route(x)
    u = L.union(idx)
    y = L.forward(x, idx, w, u)
    assert y.shape == (0, configs.TINY.hidden)
    L.close()


def test_unplaced_routed_expert_is_a_state_error():
    spec = configs.TINY
    data = Data(spec)
    ref = oracle_route(data)
    missing = int(ref["idx"][0, 0])
    L = make_layer(B, data, place=[e for e in range(spec.n_experts) if e != missing])
    x = B.activations_to_device(data.x)
    idx, w = L.route(x)
    u = L.union(idx)
    with pytest.raises(B.ColiError) as ei:
        L.forward(x, idx, w, u)
    assert ei.value.status == B.E_STATE
    # the layer stays usable once the expert is placed
    L.place(missing, data.blobs([missing])[missing])
    y = L.forward(x, idx, w, u)
    torch.cuda.synchronize()
    check_outputs(y.cpu().numpy(), oracle_y(data, ref, range(spec.n_tok)), "after placing")
    L.close()


def test_union_flags_out_of_range_ids():
    data = Data(configs.TINY)
    L = make_layer(B, data)
    bad = torch.tensor([[0, 1, 2, 99], [3, 4, 5, 6]], dtype=torch.int32, device="cuda")
    u = L.union(bad)
    torch.cuda.synchronize()
    assert L.device_errors() & 1
    assert int(u["n_union"].cpu()[0]) == 7
    assert L.device_errors() == 0
    L.close()


def test_max_tokens_is_enforced():
    data = Data(configs.TINY)
    L = make_layer(B, data, max_tokens=4)
    x = B.activations_to_device(data.x)          # 8 tokens > 4
    with pytest.raises(B.ColiError) as ei:
        L.route(x)
    assert ei.value.status == B.E_INVALID
    L.close()
