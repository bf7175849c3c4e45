"""The seeded input generators: determinism, per-head independence, shapes,
bf16 rounding and the locality structure the coarse stage relies on."""
import numpy as np

import oracle
from block_sparse_video_major_amd import workloads as wl


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9, 3.0e38], np.float32)
    b = wl.f32_to_bf16_bits(x)
    back = wl.bf16_bits_to_f32(b)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert back.tolist()[:4] == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]
    assert back[4] == 1.0
    assert np.all(wl.f32_to_bf16_bits(back) == b)


def test_generation_is_deterministic_and_per_head():
    w = wl.SMALL
    a = wl.make_inputs(w)
    b = wl.make_inputs(w, heads=[2])
    assert a["q"].shape == (1, 4, 2048, 64) and a["q"].dtype == np.uint16
    assert np.array_equal(a["q"][:, 2:3], b["q"])
    assert np.array_equal(a["v"][:, 2:3], b["v"])
    assert not np.array_equal(a["q"][:, 0], a["q"][:, 1])


def test_tiny_is_plain_fp32_normal():
    x = wl.make_inputs(wl.TINY)
    assert x["q"].dtype == np.float32 and x["q"].shape == (1, 1, 256, 64)
    assert abs(float(x["q"].std()) - 1.0) < 0.05


def test_locality_field_makes_near_cubes_score_higher():
    w = wl.SMALL
    x = {n: wl.as_float64(a) for n, a in wl.make_inputs(w).items()}
    r = oracle.vsa_forward(x["q"], x["k"], x["v"], (w.T, w.H, w.W), w.cube, w.top_k)
    # the diagonal (self cube) should usually be among the selected cubes
    lut = r["kv_block_idx"]
    hits = np.mean([i in lut[0, h, i] for h in range(w.heads) for i in range(w.n_cubes)])
    assert hits > 0.9


def test_workload_sizes():
    assert wl.WAN.n_tokens == 32768 and wl.WAN.n_cubes == 512
    assert abs(wl.WAN.sparsity - 0.6992) < 1e-3
    assert wl.LARGE.n_tokens == 122880 and wl.LARGE.n_cubes == 1920
    assert wl.WAN.selected_flops() == 4 * 12 * 32768 * 64 * 154 * 128


def test_wan_workload_matches_the_pages_benchmark_configuration():
    """The 32K-token workload is the configuration the pages print for their
    headline benchmark (tests/golden/vsa_rocm_benchmark_config.json, each
    value with its section)."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "vsa_rocm_benchmark_config.json")))["values"]
    w = wl.WAN
    assert [w.batch, w.heads, w.n_tokens, w.head_dim] == g["qkv_shape"]["value"]
    assert list(w.cube) == g["cube"]["value"]
    assert w.cube[0] * w.cube[1] * w.cube[2] == g["tokens_per_cube"]["value"]
    # Top-K 154 of 512 cubes is the nearest whole count to 70% sparsity
    target = 1.0 - g["headline_sparsity"]["value"]
    assert abs(w.top_k / w.n_cubes - target) <= 0.5 / w.n_cubes
    # N^2 is "about one billion" (within a factor of 1.1)
    assert 1.0 <= w.n_tokens ** 2 / g["attention_ops_per_layer"]["value"] < 1.1
