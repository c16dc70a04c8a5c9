"""The planted-routing fixture of the tile-count GPU test, checked on the
CPU: under the oracle's router, top-k and union, the planted token sets come
out exactly, so the per-expert counts the GPU test relies on (1, 32, 33, 96,
97, 160, 161, 321 and fillers) are the ones the layer sees."""
import numpy as np

from int4_routed_expert_layer_amd import configs
from moe_case import Data, edge_tokens, oracle_route, planted_inputs, planted_routing

COUNTS = [1, 32, 33, 96, 97, 160, 161, 321, 100, 100, 100, 100, 19]
SPEC = configs.Spec("tiles_h1024_i384_e13_k4_b330", 1024, 384, len(COUNTS), 4, 330, "bf16", True,
                    "gauss", seed=4242)


def test_planted_sets_are_the_oracle_top_k():
    sets = planted_routing(SPEC.n_experts, SPEC.top_k, COUNTS, SPEC.n_tok, seed=11)
    assert all(len(set(r)) == SPEC.top_k for r in sets.tolist())
    data = Data(SPEC)
    data.x, data.w = planted_inputs(SPEC, sets, seed=12)
    ref = oracle_route(data)
    np.testing.assert_array_equal(np.sort(ref["idx"], 1), np.sort(sets, 1))
    np.testing.assert_array_equal(ref["counts"], COUNTS)
    srt = np.sort(ref["logits"], 1)
    assert (srt[:, -SPEC.top_k] - srt[:, -SPEC.top_k - 1]).min() > 2.0


def test_edge_tokens_cover_every_chunk_boundary():
    # Two experts over 6 tokens, top-2, counts 5 and 7 with 160-row chunks
    # replaced by the real constant: rows are offsets 0..4 (expert 0) and
    # 5..11 (expert 1); the first and last row of each expert are chosen.
    ref = dict(gather=np.arange(12), counts=np.array([5, 7]), offsets=np.array([0, 5, 12]))
    assert edge_tokens(ref, 2) == sorted({0 // 2, 4 // 2, 5 // 2, 11 // 2})
    # One expert of 330 rows: chunk boundaries at 160 and 320.
    ref = dict(gather=np.arange(330), counts=np.array([330]), offsets=np.array([0, 330]))
    assert edge_tokens(ref, 1) == [0, 159, 160, 319, 320, 329]
