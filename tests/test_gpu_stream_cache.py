"""GPU tests of the stream cache: pinned-host experts kept in VRAM between
tiered calls (least recently used slot replaced).  Every call must give the
bits of the same layer with every expert in VRAM, whatever the cache size
(including the smallest, where copies of one call reuse slots of that call),
and a re-placed expert must never be served from a stale copy."""
import numpy as np
import pytest

from int4_routed_expert_layer_amd import configs, inputs
from moe_case import Data, log, make_layer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from int4_routed_expert_layer_amd import binding as B  # noqa: E402

# Half of 32 experts on the host tier; 8 tokens per call, Zipf routing, so
# popular host-tier experts recur from call to call.
SPEC = configs.Spec("stream_cache_h512_i256_e32_k4_b8", 512, 256, 32, 4, 8, "bf16", True, "zipf",
                    resident_frac=0.5, seed=9090)
CALLS = 5


def run(L, x):
    y, idx, w, u = L.layer(x)
    torch.cuda.synchronize()
    nu = int(u["n_union"].cpu()[0])
    return y.cpu().numpy(), u["union_ids"].cpu().numpy()[:nu]


@pytest.mark.parametrize("slots", [0, 4, 6, 32])
def test_stream_cache_matches_all_vram(slots):
    data = Data(SPEC, n_tok=SPEC.n_tok * CALLS)
    mask = inputs.resident_mask(SPEC, 0)
    tiers = [B.TIER_VRAM if mask[e] else B.TIER_HOST for e in range(SPEC.n_experts)]
    ref = make_layer(B, data, max_tokens=SPEC.n_tok)
    L = make_layer(B, data, tiers=tiers, max_tokens=SPEC.n_tok)
    L.set_stream_cache(slots)
    total_hits = 0
    for c in range(CALLS):
        x = B.activations_to_device(data.x[c * SPEC.n_tok:(c + 1) * SPEC.n_tok])
        log(f"case stream cache slots={slots} call {c}")
        y_ref, _ = run(ref, x)
        y, union = run(L, x)
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))
        n, nbytes = L.stream_stats()
        hits = L.stream_hits()
        host_in_union = int(sum(1 for e in union if not mask[e]))
        assert n + hits == host_in_union
        assert nbytes == n * B.blob_bytes(SPEC.hidden, SPEC.inter)
        if slots == 0 or c == 0:
            assert hits == 0
        total_hits += hits
    if slots >= 16:          # every host-tier expert fits: a repeat is always a hit
        assert total_hits > 0
    assert L.device_errors() == 0
    ref.close()
    L.close()


def test_stream_cache_drops_a_replaced_expert():
    data = Data(SPEC, n_tok=SPEC.n_tok)
    mask = inputs.resident_mask(SPEC, 0)
    tiers = [B.TIER_VRAM if mask[e] else B.TIER_HOST for e in range(SPEC.n_experts)]
    L = make_layer(B, data, tiers=tiers)
    L.set_stream_cache(32)
    x = B.activations_to_device(data.x)
    _, union = run(L, x)
    host = [int(e) for e in union if not mask[e]]
    assert host, "the call must stream at least one host-tier expert"
    e = host[0]
    other = (e + 1) % SPEC.n_experts
    swapped = data.blobs([other])[other]
    L.place(e, swapped, B.TIER_HOST)           # e is cached: its copy is now stale
    y, _ = run(L, x)
    assert L.stream_hits() == len(host) - 1   # every other host expert still hits
    ref = make_layer(B, data)
    ref.place(e, swapped, B.TIER_VRAM)
    y_ref, _ = run(ref, x)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))
    ref.close()
    L.close()


def test_stream_cache_size_is_checked():
    data = Data(SPEC, n_tok=SPEC.n_tok)
    L = B.MoELayer.from_spec(SPEC, max_tokens=SPEC.n_tok)
    for bad in (-1, 1, 3, SPEC.n_experts + 1):
        with pytest.raises(B.ColiError):
            L.set_stream_cache(bad)
    L.set_stream_cache(0)
    L.set_stream_cache(SPEC.n_experts)
    L.set_stream_cache(4)          # shrinking releases the slots past the need
    L.close()


def test_stream_cache_survives_resizing():
    """A large cache, then a small one, then none: every call still gives the
    all-VRAM bits (slots released on shrinking are never used again)."""
    data = Data(SPEC, n_tok=SPEC.n_tok * 3)
    mask = inputs.resident_mask(SPEC, 0)
    tiers = [B.TIER_VRAM if mask[e] else B.TIER_HOST for e in range(SPEC.n_experts)]
    ref = make_layer(B, data, max_tokens=SPEC.n_tok)
    L = make_layer(B, data, tiers=tiers, max_tokens=SPEC.n_tok)
    for c, slots in enumerate((32, 4, 0)):
        L.set_stream_cache(slots)
        x = B.activations_to_device(data.x[c * SPEC.n_tok:(c + 1) * SPEC.n_tok])
        for _ in range(2):
            y_ref, _ = run(ref, x)
            y, _ = run(L, x)
            assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), slots
    assert L.device_errors() == 0
    ref.close()
    L.close()
