"""Grouped MFMA path, element by element at every tile count: the router is
planted so that per-expert token counts are 1, 32, 33, 96, 97, 160, 161 and
321 (and filler experts take the rest).  The grouped kernels cut an expert's
rows into chunks of at most 160 rows and run each chunk as one to five 32-row
MFMA tiles, so these counts reach every tile count (1, 1, 2, 3, 4, 5), the
160-row split with a one-row tail (161 -> 160 + 1, 321 -> 160 + 160 + 1) and,
for the 330-token shared expert, 160 + 160 + 10.  Every token's output is
compared with the oracle, at group sizes 32 and 64, on both strategies;
routing and the union bit for bit, through the C ABI.

A chunk whose last 32-row tile would hold 16 rows or fewer ends in a 16-row
tile on v_mfma_f32_16x16x32_f16 instead; a third plant of 200 tokens with
counts 48, 49, 65, 80, 129, 144, 16, 17, 1, 33 and 109 reaches that tail
after one to four full tiles (33, 48, 65, 80, 97-112, 129, 144), its
boundary (48 ends in a 16-row tail, 49 in a full tile) and chunks without
one (16, 17, 1); the 200-token shared expert is 160 + 40 rows (a tail after
one tile).

Calls of at most 64 tokens cut chunks at 32 rows instead (a separate kernel
instance, one 32-row tile per chunk): a second plant of 64 tokens with
counts 1, 31, 32, 33, 62, 64, 17 and 16 reaches chunks of 1, 16, 17, 30, 31
and 32 rows, the splits 33 -> 32 + 1, 62 -> 32 + 30 and 64 -> 32 + 32, and
the 64-row shared expert as two chunks.
"""
import numpy as np
import pytest

from int4_routed_expert_layer_amd import configs
from moe_case import (Data, check_outputs, check_routing, gpu_run, log, make_layer,
                      oracle_route, oracle_y, planted_inputs, planted_routing)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from int4_routed_expert_layer_amd import binding as B  # noqa: E402

# 8 planted counts + 5 fillers = 13 experts; 330 tokens x top-4 = 1320 entries.
COUNTS = [1, 32, 33, 96, 97, 160, 161, 321, 100, 100, 100, 100, 19]
SPEC = configs.Spec("tiles_h1024_i384_e13_k4_b330", 1024, 384, len(COUNTS), 4, 330, "bf16", True,
                    "gauss", seed=4242)


def planted_data(group):
    spec = SPEC.with_(group=group)
    data = Data(spec)
    sets = planted_routing(spec.n_experts, spec.top_k, COUNTS, spec.n_tok, seed=11)
    data.x, data.w = planted_inputs(spec, sets, seed=12)
    return data


@pytest.mark.parametrize("path", ["grouped", "gemv"])
@pytest.mark.parametrize("group", [32, 64])
def test_every_tile_count_and_chunk_split(group, path):
    data = planted_data(group)
    log(f"case planted counts group={group} path={path}")
    ref = oracle_route(data)
    np.testing.assert_array_equal(ref["counts"], COUNTS)     # the plant took
    L = make_layer(B, data, path={"grouped": B.PATH_GROUPED, "gemv": B.PATH_GEMV}[path])
    gpu = gpu_run(B, L, data)
    check_routing(gpu, ref)
    check_outputs(gpu["y"], oracle_y(data, ref, range(SPEC.n_tok)), f"planted g{group}/{path}")
    assert L.device_errors() == 0
    L.close()


# Small calls: 8 experts, top-4, 64 tokens = 256 entries.
SMALL_COUNTS = [1, 31, 32, 33, 62, 64, 17, 16]
SMALL_SPEC = configs.Spec("tiles_small_h1024_i384_e8_k4_b64", 1024, 384, len(SMALL_COUNTS), 4, 64, "bf16", True,
                          "gauss", seed=4343)


@pytest.mark.parametrize("group", [32, 64])
def test_small_call_chunks_of_one_tile(group):
    spec = SMALL_SPEC.with_(group=group)
    data = Data(spec)
    sets = planted_routing(spec.n_experts, spec.top_k, SMALL_COUNTS, spec.n_tok, seed=13)
    data.x, data.w = planted_inputs(spec, sets, seed=14)
    log(f"case small-call planted counts group={group}")
    ref = oracle_route(data)
    np.testing.assert_array_equal(ref["counts"], SMALL_COUNTS)
    L = make_layer(B, data, path=B.PATH_GROUPED)
    gpu = gpu_run(B, L, data)
    check_routing(gpu, ref)
    check_outputs(gpu["y"], oracle_y(data, ref, range(spec.n_tok)), f"small planted g{group}")
    assert L.device_errors() == 0
    L.close()


# Tail tiles: 12 experts, top-4, 200 tokens = 800 entries.
TAIL_COUNTS = [48, 49, 65, 80, 129, 144, 16, 17, 1, 33, 109, 109]
TAIL_SPEC = configs.Spec("tiles_tail_h1024_i384_e12_k4_b200", 1024, 384, len(TAIL_COUNTS), 4, 200, "bf16", True,
                         "gauss", seed=4444)


@pytest.mark.parametrize("group", [32, 64])
def test_tail_tiles_of_sixteen_rows(group):
    spec = TAIL_SPEC.with_(group=group)
    data = Data(spec)
    sets = planted_routing(spec.n_experts, spec.top_k, TAIL_COUNTS, spec.n_tok, seed=15)
    data.x, data.w = planted_inputs(spec, sets, seed=16)
    log(f"case tail-tile planted counts group={group}")
    ref = oracle_route(data)
    np.testing.assert_array_equal(ref["counts"], TAIL_COUNTS)
    L = make_layer(B, data, path=B.PATH_GROUPED)
    gpu = gpu_run(B, L, data)
    check_routing(gpu, ref)
    check_outputs(gpu["y"], oracle_y(data, ref, range(spec.n_tok)), f"tail planted g{group}")
    assert L.device_errors() == 0
    L.close()
