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


def test_lookahead_across_layers_on_a_second_stream():
    """The stack's lookahead: while layer 0 runs on the main stream, layer 1's
    route and union run on a second stream and its host-tier experts are
    prefetched; then layer 1 runs.  Both layers give the bits of their
    all-VRAM twins on every batch."""
    specs = [SPEC.with_(seed=SPEC.seed + i) for i in range(2)]
    datas = [Data(sp, n_tok=3 * SPEC.n_tok) for sp in specs]
    refs = [make_layer(B, d, max_tokens=SPEC.n_tok) for d in datas]
    layers = [make_layer(B, d, max_tokens=SPEC.n_tok) for d in datas]
    for d, L in zip(datas, layers):
        host = [e for e in range(SPEC.n_experts) if e % 2 == 1]
        for e, blob in d.blobs(host).items():
            L.place(e, blob, B.TIER_HOST)
        d.drop_blobs()
        L.set_stream_cache(8)
    ahead = torch.cuda.Stream()
    for b in range(3):
        xs = [B.activations_to_device(d.x[b * SPEC.n_tok:(b + 1) * SPEC.n_tok]) for d in datas]
        want = []
        for L, x in zip(refs, xs):
            y, _, _, _ = L(x)
            want.append(y)
        torch.cuda.synchronize()
        idx0, w0 = layers[0].route(xs[0])
        u0 = layers[0].union(idx0)
        ahead.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(ahead):
            idx1, w1 = layers[1].route(xs[1])
            u1 = layers[1].union(idx1)
            started = layers[1].prefetch_union(u1)
        y0 = layers[0].forward(xs[0], idx0, w0, u0)
        torch.cuda.current_stream().wait_stream(ahead)
        y1 = layers[1].forward(xs[1], idx1, w1, u1)
        torch.cuda.synchronize()
        log(f"  batch {b}: layer 1 prefetched {started}, hits {layers[1].stream_hits()}")
        assert layers[1].stream_hits() >= started
        for got, ref in ((y0, want[0]), (y1, want[1])):
            assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
    for L in refs + layers:
        assert L.device_errors() == 0
        L.close()
