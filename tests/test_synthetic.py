"""The synthetic workloads carry the statistics the pages print (tests/golden/page_values.json)
and are deterministic."""
import json
import os

import numpy as np
import pytest

from synthetic import LINEAR_CONFIGS, bf16_bits_to_f32, f64_to_bf16_bits, make_kv, make_linear

PV = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def test_bf16_formatting_is_round_to_nearest_even():
    import torch

    x = np.random.default_rng(0).standard_normal(10000) * 100
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(f64_to_bf16_bits(x), ref.view(np.uint16))
    np.testing.assert_array_equal(bf16_bits_to_f32(ref.view(np.uint16)),
                                  torch.from_numpy(ref).view(torch.bfloat16).float().numpy())


def test_deterministic_and_seed_sensitive():
    a = make_linear(1)
    b = make_linear(1)
    c = make_linear(1, seed=1)
    assert np.array_equal(a["X"], b["X"]) and np.array_equal(a["W"], b["W"])
    assert not np.array_equal(a["X"], c["X"])
    k1, k2 = make_kv(tokens=16), make_kv(tokens=16)
    assert np.array_equal(k1["K"], k2["K"]) and not np.array_equal(k1["K"], k1["V"])


def test_tiny_config_outliers():
    d = make_linear(1)
    X = bf16_bits_to_f32(d["X"]).astype(np.float64)
    assert X.shape == (64, 256) and d["W"].shape == (256, 256)
    ch = d["outlier_channels"]
    assert ch.size == 4
    amax = np.abs(X).max(0)
    others = np.delete(amax, ch)
    assert amax[ch].min() > 20 * np.median(others)


@pytest.mark.parametrize("cid", [2, 3])
def test_attention_and_ffn_up_outlier_model(cid):
    d = make_linear(cid, M=512)
    cfg = LINEAR_CONFIGS[cid]
    ch = d["outlier_channels"]
    assert ch.size == round(0.01 * cfg.K) == 31
    X = bf16_bits_to_f32(d["X"]).astype(np.float64)
    std = X.std(0)
    assert (std[ch] > 15).all() and (np.delete(std, ch) < 1.2).all()


def test_attention_weight_has_rank8_spike_of_norm_10():
    d = make_linear(2, M=8)
    W = bf16_bits_to_f32(d["W"]).astype(np.float64)
    s = np.linalg.svd(W, compute_uv=False)
    # spike singular values ~10 on top of a bulk with edge ~ (1 + sqrt(K/N)) = 2
    assert (s[:8] > 9.0).all() and (s[:8] < 12.5).all() and s[8] < 2.5


def test_ffn_down_max_over_median_and_heavy_tails():
    d = make_linear(4)
    X = bf16_bits_to_f32(d["X"])
    a = np.abs(X)
    ratio = float(a.max() / np.median(a))
    target = PV["ffn_down_max_over_median"]["value"]
    assert abs(ratio / target - 1) < 0.02, ratio
    assert d["outlier_channels"].size == round(0.005 * 12288) == 61
    body = np.delete(X[:1024].astype(np.float64), d["outlier_channels"], axis=1).ravel()
    kurt = np.mean((body - body.mean()) ** 4) / np.var(body) ** 2
    assert kurt > 3.0 + 2.0  # Laplace: 6; well above a Gaussian's 3


def test_kv_cache_skew_and_channel_cv():
    d = make_kv()
    assert d["K"].shape == (10240, 32, 128)
    for name in ("K", "V"):
        x = bf16_bits_to_f32(d[name].reshape(10240, -1)).astype(np.float64)
        mu, sd = x.mean(0), x.std(0)
        skew = np.mean(((x - mu) / sd) ** 3, axis=0)
        assert abs(skew.mean() - PV["kv_skewness"]["value"]) < 0.02, skew.mean()
        cv = sd.std() / sd.mean()
        assert cv > PV["kv_channel_cv_min"]["value"], cv
