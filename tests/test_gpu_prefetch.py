"""Lookahead prefetch (README "Mai aspettare il disco due volte"; the
getting-started page's Overlap step): the next batch's route and union run
first, coli_layer_prefetch_union starts its host-tier experts' copies into
the stream cache, and the forward call then finds them cached.  Results are
bit-identical to the all-VRAM layer; hit counts match the prefetched
experts."""
import numpy as np
import pytest

from int4_routed_expert_layer_amd import configs, inputs
from moe_case import Data, check_outputs, gpu_run, log, make_layer, oracle_route, oracle_y

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from int4_routed_expert_layer_amd import binding as B  # noqa: E402

SPEC = configs.Spec("prefetch_h512_i256_e32_k4_b16", 512, 256, 32, 4, 16, "bf16", True,
                    "zipf", seed=5150)
KEYS = ("idx", "weight", "union_ids", "counts", "offsets", "gather", "y")


def same(a, b):
    for key in KEYS:
        assert np.array_equal(np.asarray(a[key]).view(np.uint8), np.asarray(b[key]).view(np.uint8)), key


@pytest.mark.parametrize("slots", [4, 8, 32])
def test_prefetch_is_bitwise_all_vram(slots):
    data = Data(SPEC, n_tok=3 * SPEC.n_tok)
    L = make_layer(B, data)
    batches = [Data(SPEC, n_tok=SPEC.n_tok) for _ in range(3)]
    for i, b in enumerate(batches):
        b.x = data.x[i * SPEC.n_tok:(i + 1) * SPEC.n_tok]
    resident = [gpu_run(B, L, b, with_logits=False) for b in batches]
    host = [e for e in range(SPEC.n_experts) if e % 3 != 0]
    for e, blob in data.blobs(host).items():
        L.place(e, blob, B.TIER_HOST)
    L.set_stream_cache(slots)
    for i, b in enumerate(batches):
        x = B.activations_to_device(b.x)
        idx, w = L.route(x)
        u = L.union(idx)
        started = L.prefetch_union(u)
        union = u["union_ids"].cpu().numpy()[:int(u["n_union"].cpu()[0])]
        host_in_union = [e for e in union if e in host]
        log(f"  slots {slots} batch {i}: union {len(union)}, host {len(host_in_union)}, prefetched {started}")
        assert started <= min(slots, len(host_in_union))
        y = L.forward(x, idx, w, u)
        torch.cuda.synchronize()
        got = dict(idx=idx.cpu().numpy(), weight=w.cpu().numpy(), y=y.cpu().numpy(),
                   union_ids=union, counts=u["counts"].cpu().numpy(), offsets=u["offsets"].cpu().numpy(),
                   gather=u["gather"].cpu().numpy())
        same(got, resident[i])
        n_streamed, _ = L.stream_stats()
        hits = L.stream_hits()
        assert hits + n_streamed == len(host_in_union)
        assert hits >= started
        assert L.device_errors() == 0
    ref = oracle_route(batches[0])
    check_outputs(resident[0]["y"], oracle_y(batches[0], ref, range(SPEC.n_tok)), "prefetch layer")
    L.close()


def test_prefetch_needs_the_stream_cache():
    data = Data(SPEC)
    L = make_layer(B, data)
    L.place(1, data.blobs([1])[1], B.TIER_HOST)
    x = B.activations_to_device(data.x)
    idx, w = L.route(x)
    u = L.union(idx)
    with pytest.raises(B.ColiError) as ei:
        L.prefetch_union(u)
    assert ei.value.status == B.E_STATE
    L.close()


def test_prefetch_then_replace_is_not_served_stale():
    """An expert prefetched and then re-placed with new contents is read
    from its new blob: placement drops the prefetched copy."""
    data = Data(SPEC)
    L = make_layer(B, data)
    x = B.activations_to_device(data.x)
    idx, w = L.route(x)
    u = L.union(idx)
    union = u["union_ids"].cpu().numpy()[:int(u["n_union"].cpu()[0])]
    e = int(union[0])
    L.place(e, data.blobs([e])[e], B.TIER_HOST)
    L.set_stream_cache(4)
    assert L.prefetch_union(u) == 1
    new = inputs.expert_blob(SPEC, 0, (e + 7) % SPEC.n_experts)
    L.place(e, new, B.TIER_HOST)
    y = L.forward(x, idx, w, u)
    torch.cuda.synchronize()
    data._blobs[e] = new
    ref = oracle_route(data)
    check_outputs(y.cpu().numpy(), oracle_y(data, ref, range(SPEC.n_tok)), "re-placed after prefetch")
    L.close()
