"""The host-side byte model against the figures the pages print
(tests/golden/pages_traffic.json), and against hand-counted bytes."""
import json
import os

from conv2d_batchnorm_silu_amd import traffic
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_traffic.json")))


def test_conv_bn_silu_trip_count():
    g = GOLD["conv_bn_silu_trips"]
    unf, fus = traffic.chain_trips(g["ops"])
    assert (unf, fus) == (g["unfused_trips"], g["fused_trips"])
    assert abs((unf - fus) / unf - g["removed_fraction"]) < 1e-15


def test_elementwise_chain():
    g = GOLD["elementwise_chain"]
    assert traffic.chain_trips(g["ops"]) == (g["unfused_element_trips_per_N"],
                                             g["fused_element_trips_per_N"])
    unf2, fus2 = traffic.chain_trips(2)
    assert fus2 / unf2 == g["two_op_ratio"]


def test_fp16_intermediate_and_gelu_example():
    g = GOLD["fp16_intermediate"]
    assert traffic.intermediate_bytes(1, g["elem_bytes"]) == (g["store_bytes_per_element"]
                                                              + g["load_bytes_per_element"])
    e = GOLD["gelu_bias_example"]
    # The page's 128 MiB is one materialisation (the store, or the re-read).
    assert traffic.intermediate_bytes(e["fp16_values"], 2) // 2 == e["intermediate_mib"] * 2**20
    r = GOLD["residual_ln_boundary"]
    assert traffic.intermediate_bytes(r["B"] * r["H"], 2) == r["boundary_bytes"]


def test_workload_bytes_hand_counted():
    wl = WORKLOADS["conv1x1_c64_k256"]
    b = traffic.workload_bytes(wl)
    assert b == dict(x=12845056, w=32768, bn=2048, y=51380224)
    assert traffic.fused_bytes(wl) == 64260096
    assert traffic.unfused_bytes(wl) == 64260096 + 4 * 51380224
    assert traffic.split_bytes(wl) == 64260096 + 2 * 51380224
    assert traffic.train_bytes(wl) == 64260096 + 3 * 51380224
    assert traffic.fused_bytes_fp8_out(wl) == 12845056 + 32768 + 2048 + 51380224 // 2
    assert traffic.conv_flops(wl) == 3288334336
    wl = WORKLOADS["stem3x3s2_k16"]
    assert traffic.fused_bytes(wl) == 19267584 + 864 + 128 + 25690112
    assert traffic.conv_flops(WORKLOADS["conv7x7_c64_k64"]) == 20141047808
    assert traffic.conv_flops(WORKLOADS["conv3x3_c128_k128"]) == 7398752256
    assert traffic.fused_bytes(WORKLOADS["tiny_f32_3x3"]) == 3072 + 864 + 64 + 8192
