"""GPU parity of the routing steps over many shapes, against the oracle.

* top-k: E from 1 to 1024 (one to sixteen keys per lane of the selecting
  wave), k from 1 to 32, with exact logit ties planted between experts;
  logits and ids bit for bit, weights to fp32 rounding.
* top-k at 3 to 128 tokens, where the router and the selection run in one
  launch (the last router workgroup of each four tokens selects them), with
  calls on both sides of that range on one layer, the same shapes and ties.
* union: from a single slab of one chunk to the 64-slab maximum, slabs of
  several chunks, ragged last slabs, E up to 1024 and skewed or uniform
  popularity; every output bit for bit.  Calls of different sizes reuse one
  layer, which exercises the reset of the slab arrival counter.
"""
import numpy as np
import pytest

from int4_routed_expert_layer_amd import configs
from moe_case import Data, log
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from int4_routed_expert_layer_amd import binding as B  # noqa: E402


def random_ids(seed, n_tok, n_experts, k, skew):
    """k distinct ids per token; expert popularity ~ rank**-skew over a
    random popularity order (Gumbel top-k sampling without replacement)."""
    rng = np.random.default_rng(seed)
    logp = -skew * np.log(np.arange(1, n_experts + 1, dtype=np.float64))
    logp = logp[rng.permutation(n_experts)]
    g = rng.gumbel(size=(n_tok, n_experts))
    return np.argsort(-(logp + g), axis=1, kind="stable")[:, :k].astype(np.int32)


def gpu_union(L, ids):
    u = L.union(torch.from_numpy(ids).to("cuda"))
    torch.cuda.synchronize()
    nu = int(u["n_union"].cpu()[0])
    return dict(n_union=nu, union_ids=u["union_ids"].cpu().numpy()[:nu],
                counts=u["counts"].cpu().numpy(), offsets=u["offsets"].cpu().numpy(),
                gather=u["gather"].cpu().numpy()[:ids.size])


def check_union(got, ref):
    assert got["n_union"] == ref["n_union"]
    for key in ("union_ids", "counts", "offsets", "gather"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)


UNION_CASES = [
    # (E, k, token counts called in this order on one layer, skew)
    (1, 1, [700, 1, 700], 0.0),
    (37, 3, [5, 1000, 5], 1.1),
    (256, 8, [1, 31, 32, 33, 64, 2048, 2049, 4096, 8197, 64], 1.1),
    (256, 8, [4096, 255], 0.0),
    (1024, 8, [1000, 8192, 3], 0.8),
    (1024, 32, [3000, 17], 0.5),
]


@pytest.mark.parametrize("E,k,sizes,skew", UNION_CASES)
def test_union_matches_oracle(E, k, sizes, skew):
    L = B.MoELayer(256, 128, E, k, False, max(sizes), "bf16")
    for i, n in enumerate(sizes):
        ids = random_ids(1000 * E + 10 * k + i, n, E, k, skew)
        log(f"case union E={E} k={k} n_tok={n} skew={skew}")
        check_union(gpu_union(L, ids), orc.union(ids, E))
        assert L.device_errors() == 0
    L.close()


TOPK_CASES = [(1, 1), (37, 5), (64, 8), (65, 8), (200, 32), (256, 8), (300, 12), (512, 16),
              (777, 9), (1024, 32), (1024, 1)]


@pytest.mark.parametrize("E,k", TOPK_CASES)
def test_route_matches_oracle(E, k):
    spec = configs.TINY.with_(hidden=256, inter=128, n_experts=E, top_k=k, n_tok=301,
                              has_shared=False, act="f32", routing="gauss")
    data = Data(spec)
    # Exact logit ties between pairs of experts (equal router columns).
    for a in range(0, E - 1, 7):
        data.w[:, a + 1] = data.w[:, a]
    log(f"case route E={E} k={k} n_tok={spec.n_tok}")
    L = B.MoELayer.from_spec(spec)
    L.set_router(data.w, data.b)
    x = B.activations_to_device(data.x)
    logits = L.router_logits(x)
    idx, w = L.route(x)
    torch.cuda.synchronize()
    ref_logits = orc.router_logits(data.x, data.w, data.b)
    ref_idx, ref_w = orc.topk(ref_logits, k)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), ref_logits.view(np.uint32))
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7)
    L.close()


@pytest.mark.parametrize("E,act", [(256, "bf16"), (300, "f32"), (37, "bf16")])
def test_router_logits_large_batch_matches_oracle(E, act):
    """Logits of a large batch (the 8-token x 8-expert tile kernel, ragged
    in both tokens and experts here), bit for bit."""
    spec = configs.TINY.with_(hidden=512, inter=128, n_experts=E, top_k=4, n_tok=1000,
                              has_shared=False, act=act, routing="gauss")
    data = Data(spec)
    log(f"case router E={E} act={act} n_tok={spec.n_tok}")
    L = B.MoELayer.from_spec(spec)
    L.set_router(data.w, data.b)
    x = B.activations_to_device(data.x)
    logits = L.router_logits(x)
    idx, w = L.route(x)
    torch.cuda.synchronize()
    ref_logits = orc.router_logits(data.x, data.w, data.b)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), ref_logits.view(np.uint32))
    ref_idx, _ = orc.topk(ref_logits, spec.top_k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    L.close()


ROUTE_SIZES = [128, 3, 77, 129, 2, 4, 5, 64]   # 3..128: router and selection in one launch


@pytest.mark.parametrize("E,k,act", [(E, k, "f32") for E, k in TOPK_CASES] + [(256, 8, "bf16"), (1000, 20, "bf16")])
def test_route_small_batches_match_oracle(E, k, act):
    n_max = max(ROUTE_SIZES)
    spec = configs.TINY.with_(hidden=256, inter=128, n_experts=E, top_k=k, n_tok=n_max,
                              has_shared=False, act=act, routing="gauss")
    data = Data(spec)
    for a in range(0, E - 1, 7):
        data.w[:, a + 1] = data.w[:, a]
    L = B.MoELayer.from_spec(spec)
    L.set_router(data.w, data.b)
    for i, n in enumerate(ROUTE_SIZES):
        # a different slice of the seeded batch per call, so that counters left
        # by an earlier call would show in the result
        x_np = np.ascontiguousarray(np.roll(data.x, 13 * i, axis=0)[:n])
        log(f"case route-small E={E} k={k} act={act} n_tok={n}")
        idx, w = L.route(B.activations_to_device(x_np))
        torch.cuda.synchronize()
        ref_idx, ref_w = orc.topk(orc.router_logits(x_np, data.w, data.b), k)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx, err_msg=f"n_tok={n}")
        np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7, err_msg=f"n_tok={n}")
    assert L.device_errors() == 0
    L.close()
