"""Host-side checks of the seeded input generator (CPU only)."""
import json
import os

import numpy as np
import torch

from mixture_experts_layer_32_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 0.0,
                                  np.float32(3.4e38)], np.float32)])
    ours = inputs.round_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    bits = inputs.bf16_bits(ours)
    assert np.array_equal(inputs.bf16_bits_to_f32(bits).view(np.uint32), ours.view(np.uint32))


def test_generator_is_deterministic_and_keyed_per_expert():
    cfg = inputs.CONFIGS["tiny"].with_(T=64)
    a = inputs.make_layer(cfg)
    b = inputs.make_layer(cfg)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
    wg3, wu3, wd3 = inputs.expert_weights(cfg, 3)
    assert np.array_equal(wg3, a["wg"][3]) and np.array_equal(wd3, a["wd"][3])
    share = inputs.make_weights(cfg.with_(E_local=2, e0=5))
    assert np.array_equal(share[1][1], a["wu"][6])


def test_distributions_and_encodings():
    cfg, L = inputs.custom_layer(T=2048, H=512, F=256, E=16, k=4, dtype="bf16")
    assert abs(L["x"].std() - 1.0) < 0.02
    assert abs(L["wg"].std() * np.sqrt(512) - 1.0) < 0.02
    assert abs(L["wd"].std() * np.sqrt(256) - 1.0) < 0.02
    assert abs(L["logits"].std() - 0.02 * np.sqrt(512)) < 0.03
    for n in ("x", "dy", "wg", "wu", "wd"):
        inputs.bf16_bits(L[n])            # raises unless bf16-exact
    assert L["logits"].dtype == np.float32


def test_zipf_prior_skews_loads():
    cfg, L = inputs.custom_layer(T=4096, H=256, F=128, E=32, k=4, zipf_s=1.1)
    top = np.argsort(-L["logits"], axis=1, kind="stable")[:, :4]
    counts = np.bincount(top.ravel(), minlength=32)
    assert counts[0] > 5 * counts[16:].mean()


def test_pages_layer_timings_are_self_consistent(repo_root):
    g = json.load(open(os.path.join(repo_root, "tests", "golden", "pages_layer_timings.json")))
    s = g["qwen3_30b_a3b"]
    (f0, f1), (b0, b1) = s["fwd_ms"], s["bwd_ms"]
    assert abs(f0 / f1 - s["fwd_speedup"]) < 0.05          # printed ratios are from unrounded times
    assert abs(b0 / b1 - s["bwd_speedup"]) < 0.01
    assert abs((2 * f0 + b0) / (2 * f1 + b1) - s["full_layer_speedup"]) < 0.02
    L = g["qwen3_235b_a22b"]
    (B0, B1), (T0, T1) = L["bwd_ms"], L["full_layer_ms"]
    assert abs(B0 / B1 - L["bwd_speedup"]) < 0.01
    assert abs(T0 / T1 - L["full_layer_speedup"]) < 0.01
    assert abs(((T0 - B0) / 2) / ((T1 - B1) / 2) - L["fwd_speedup"]) < 0.01
