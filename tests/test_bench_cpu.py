"""CPU checks of the benchmark's own arithmetic: the algorithmic bytes and
FLOPs its roofline divides by, for every weight format, against their closed
forms, and the single-GPU contract of its command line."""
import json
import os
import subprocess
import sys

import pytest

import bench
from int4_routed_expert_layer_amd import configs

H, I = 6144, 2048


def panel_bytes(bits, group, rows=16, k=H, mats=2):
    # rows x K weights at `bits` each plus one fp16 scale per `group` columns, per matrix
    return mats * (rows * k * bits // 8 + rows * (k // group) * 2)


@pytest.mark.parametrize("group,bits", [(32, 4), (64, 4), (64, 8)])
def test_decode_b1_gateup_and_down_bytes(group, bits):
    spec = configs.DECODE_B1.with_(group=group, bits=bits)
    nb = bench.algorithmic_bytes(spec, 8, 1)
    # fused small-batch call: the routed gate/up kernel streams the 8 routed experts
    assert nb["gateup"] == 8 * (I // 16) * panel_bytes(bits, group)
    # down streams all 9 (8 routed + shared): 192 panel pairs of 32 rows over I
    assert nb["down"] == 9 * (H // 32) * panel_bytes(bits, group, rows=32, k=I, mats=1)
    assert nb["router"] == H * 256 * 4
    assert nb["total"] == 9 * configs.blob_bytes(H, I, group, bits) + H * 256 * 4 + H * 2 + H * 4


def test_decode_b1_gateup_bytes_are_the_documented_figure():
    assert bench.algorithmic_bytes(configs.DECODE_B1, 8, 1)["gateup"] == 113246208 == 8 * 128 * 110592


def test_prefill_flops():
    spec = configs.PREFILL_B4096
    assert bench.expert_flops(spec, 4096) == 2.0 * (4096 * 8 + 4096) * 3 * H * I


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_record_names_its_sources():
    rec = json.load(open(os.path.join(bench.ROOT, "profiles", "pmc_traffic_gemv_gateup_decode_b1.json")))
    assert rec["source_files"] == bench.KERNEL_SOURCES
    assert rec["algorithmic_bytes_per_launch"] == 113246208
