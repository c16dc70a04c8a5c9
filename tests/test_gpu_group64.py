"""GPU parity with one fp16 scale per 64 reduction elements (the group size of
the int4 container in the README's "Scarica il modello" section): every path
of the library (GEMV, grouped MFMA, the one-launch small-batch call, pinned
host placement) against the oracle at the same group size.  Routing and the
union bit for bit, outputs within 2e-3 * max|y_ref|, through the C ABI.
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

PATHS = {"gemv": B.PATH_GEMV, "grouped": B.PATH_GROUPED, "auto": B.PATH_AUTO}

MEDIUM64 = configs.Spec("medium_g64_h512_i256_e32_k4_b37", 512, 256, 32, 4, 37, "bf16", True,
                        "zipf", seed=778, group=64)


def full_check(spec, path, n_tok=None, tokens=None):
    data = Data(spec, n_tok=n_tok)
    log(f"case {spec.name} group={spec.group} path={path} n_tok={data.x.shape[0]}")
    L = make_layer(B, data, path=PATHS[path])
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    toks = list(range(data.x.shape[0]) if tokens is None else tokens)
    check_outputs(gpu["y"][toks], oracle_y(data, ref, toks), f"{spec.name}/{path}")
    L.close()


def test_group64_blob_size():
    assert B.blob_bytes(6144, 2048, 64) == configs.blob_bytes(6144, 2048, 64) == 20054016


@pytest.mark.parametrize("path", ["gemv", "grouped"])
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_group64_medium_ragged(path, act):
    full_check(MEDIUM64.with_(act=act), path)


@pytest.mark.parametrize("path", ["gemv", "grouped", "auto"])
@pytest.mark.parametrize("hidden,inter,n_tok", [(384, 640, 3), (640, 384, 45), (256, 128, 8)])
def test_group64_shapes(path, hidden, inter, n_tok):
    # 640 = 5 chunks of 128: an odd chunk count per row; 384 leaves the
    # grouped down pass a half-empty last column block.
    spec = MEDIUM64.with_(name=f"g64_h{hidden}_i{inter}_b{n_tok}", hidden=hidden, inter=inter,
                          n_experts=24, top_k=6, n_tok=n_tok)
    full_check(spec, path)


@pytest.mark.parametrize("n_tok", [1, 2, 3, 4])
def test_group64_fused_small_batches(n_tok):
    """The one-launch front (router, selection, union, shared gate/up) and the
    fused down + combine: bit-identical to the three separate calls, and
    against the oracle."""
    data = Data(MEDIUM64, n_tok=n_tok)
    log(f"case fused g64 n_tok={n_tok}")
    L = make_layer(B, data, path=B.PATH_GEMV)
    x = B.activations_to_device(data.x)
    y, idx, w, u = L.layer(x)
    torch.cuda.synchronize()
    assert L.device_errors() == 0
    three = gpu_run(B, L, data, with_logits=False)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), three["y"].view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), three["idx"])
    ref = oracle_route(data)
    check_routing(three, ref, check_logits=False)
    check_outputs(y.cpu().numpy(), oracle_y(data, ref, range(n_tok)), f"fused g64 n_tok={n_tok}")
    L.close()


def test_group64_host_tier_matches_vram():
    """Half the experts in pinned host memory (streamed per call, with and
    without the stream cache): bit-identical to the all-VRAM layer."""
    spec = MEDIUM64.with_(n_tok=16)
    data = Data(spec)
    L = make_layer(B, data)
    all_vram = gpu_run(B, L, data, with_logits=False)
    host = list(range(0, spec.n_experts, 2))
    for e, blob in data.blobs(host).items():
        L.place(e, blob, B.TIER_HOST)
    data.drop_blobs()
    for slots in (0, 6):
        L.set_stream_cache(slots)
        for rep in range(2):
            tiered = gpu_run(B, L, data, with_logits=False)
            log(f"  slots {slots} call {rep}: streamed {L.stream_stats()[0]}")
            for key in ("idx", "weight", "union_ids", "counts", "offsets", "gather", "y"):
                assert np.array_equal(np.asarray(tiered[key]).view(np.uint8),
                                      np.asarray(all_vram[key]).view(np.uint8)), key
    ref = oracle_route(data)
    check_outputs(all_vram["y"], oracle_y(data, ref, range(spec.n_tok)), "g64 host tier")
    L.close()


@pytest.fixture(scope="module")
def full_size_g64():
    """The full-size layer (H 6144, I 2048, 256 experts + shared, top-8) with
    group-64 scales, sized for the 4096-token batch."""
    spec = configs.PREFILL_B4096.with_(name="prefill_b4096_g64", group=64)
    data = Data(spec)
    log("case full-size g64: placing 257 experts")
    L = make_layer(B, data)
    yield spec, data, L
    L.close()


@pytest.mark.parametrize("path", ["auto", "gemv", "grouped"])
def test_group64_full_size_decode(full_size_g64, path):
    spec, _, L = full_size_g64
    data = Data(spec, n_tok=1)
    L.set_path(PATHS[path])
    log(f"case full-size g64 decode B=1 path={path}")
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    check_outputs(gpu["y"], oracle_y(data, ref, [0]), f"g64 decode/{path}")
    if path == "auto":
        y, idx, w, u = L.layer(B.activations_to_device(data.x))
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), gpu["y"].view(np.uint32))


def test_group64_full_size_prefill(full_size_g64):
    spec, data, L = full_size_g64
    L.set_path(B.PATH_AUTO)
    log("case full-size g64 prefill B=4096")
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    tokens = edge_tokens(ref, spec.top_k, extra=[0, 1, 777, 2048, 3001, 4095])
    log(f"  comparing {len(tokens)} tokens")
    check_outputs(gpu["y"][tokens], oracle_y(data, ref, tokens), "g64 prefill_b4096")
