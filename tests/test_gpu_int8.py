"""GPU parity of int8 experts (one two's-complement byte per weight, fp16
group scales; the README's "Scarica il modello" section and the
getting-started page require int8 for the MTP head): the GEMV path and the
one-launch small-batch call, pinned host placement, and the full-size layer,
against the oracle at 8 bits.  Routing and the union bit for bit, outputs
within 2e-3 * max|y_ref|, through the C ABI.  Int8 layers take the GEMV path
for every batch size; asking for the grouped path is an error.
"""
import numpy as np
import pytest

from int4_routed_expert_layer_amd import configs
from moe_case import (Data, check_outputs, check_routing, gpu_run, log, make_layer,
                      oracle_route, oracle_y)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from int4_routed_expert_layer_amd import binding as B  # noqa: E402

MEDIUM8 = configs.Spec("medium_i8_h512_i256_e32_k4_b37", 512, 256, 32, 4, 37, "bf16", True,
                       "zipf", seed=779, bits=8)


def full_check(spec, path=B.PATH_AUTO, n_tok=None):
    data = Data(spec, n_tok=n_tok)
    log(f"case {spec.name} bits={spec.bits} group={spec.group} n_tok={data.x.shape[0]}")
    L = make_layer(B, data, path=path)
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    toks = list(range(data.x.shape[0]))
    check_outputs(gpu["y"][toks], oracle_y(data, ref, toks), spec.name)
    L.close()


def test_int8_blob_size():
    H, I = 6144, 2048
    assert B.blob_bytes(H, I, 64, 8) == configs.blob_bytes(H, I, 64, 8) == 3 * H * I + 3 * H * I // 64 * 2


@pytest.mark.parametrize("group", [32, 64])
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_int8_medium_ragged(group, act):
    full_check(MEDIUM8.with_(act=act, group=group))


@pytest.mark.parametrize("group", [32, 64])
@pytest.mark.parametrize("hidden,inter,n_tok", [(384, 640, 3), (640, 384, 45), (256, 128, 8)])
def test_int8_shapes(group, hidden, inter, n_tok):
    spec = MEDIUM8.with_(name=f"i8_g{group}_h{hidden}_i{inter}_b{n_tok}", hidden=hidden, inter=inter,
                         n_experts=24, top_k=6, n_tok=n_tok, group=group)
    full_check(spec)


def test_int8_rejects_the_grouped_path():
    data = Data(MEDIUM8, n_tok=2)
    L = make_layer(B, data)
    with pytest.raises(B.ColiError) as ei:
        L.set_path(B.PATH_GROUPED)
    assert ei.value.status == B.E_UNSUPPORTED
    L.set_path(B.PATH_GEMV)
    L.close()


@pytest.mark.parametrize("n_tok", [1, 2, 3, 4])
def test_int8_fused_small_batches(n_tok):
    data = Data(MEDIUM8.with_(group=64), n_tok=n_tok)
    log(f"case fused int8 n_tok={n_tok}")
    L = make_layer(B, data)
    x = B.activations_to_device(data.x)
    y, idx, w, u = L.layer(x)
    torch.cuda.synchronize()
    assert L.device_errors() == 0
    three = gpu_run(B, L, data, with_logits=False)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), three["y"].view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), three["idx"])
    ref = oracle_route(data)
    check_routing(three, ref, check_logits=False)
    check_outputs(y.cpu().numpy(), oracle_y(data, ref, range(n_tok)), f"fused int8 n_tok={n_tok}")
    L.close()


def test_int8_host_tier_matches_vram():
    spec = MEDIUM8.with_(n_tok=16, group=64)
    data = Data(spec)
    L = make_layer(B, data)
    all_vram = gpu_run(B, L, data, with_logits=False)
    host = list(range(1, spec.n_experts, 2))
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
    check_outputs(all_vram["y"], oracle_y(data, ref, range(spec.n_tok)), "int8 host tier")
    L.close()


@pytest.fixture(scope="module")
def full_size_i8():
    """The full-size layer (H 6144, I 2048, 256 experts + shared, top-8) with
    int8 weights and group-64 scales, sized for 64 tokens."""
    spec = configs.DECODE_B64.with_(name="decode_b64_i8_g64", bits=8, group=64)
    data = Data(spec)
    log("case full-size int8: placing 257 experts")
    L = make_layer(B, data)
    yield spec, data, L
    L.close()


def test_int8_full_size_decode_b1(full_size_i8):
    spec, _, L = full_size_i8
    data = Data(spec, n_tok=1)
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    check_outputs(gpu["y"], oracle_y(data, ref, [0]), "int8 decode B=1")
    y, idx, w, u = L.layer(B.activations_to_device(data.x))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), gpu["y"].view(np.uint32))


def test_int8_full_size_decode_b64(full_size_i8):
    spec, data, L = full_size_i8
    gpu = gpu_run(B, L, data)
    ref = oracle_route(data)
    check_routing(gpu, ref)
    tokens = list(range(spec.n_tok))          # every token of the batch
    check_outputs(gpu["y"][tokens], oracle_y(data, ref, tokens), "int8 decode B=64")
