"""The seeded input generator: determinism, prefix consistency, bf16 rounding (CPU only)."""
import numpy as np
import torch

from synthetic import (get_config, draw_beams, unpacked_node_tensors, round_to_bf16, kv_cache,
                       lm_weight, base_seed)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-5, 5, 100000),
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65504.0, 3.3895e38], np.float32)])
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_beams_are_deterministic_and_per_request():
    cfg = get_config("gqa")
    a = draw_beams(cfg, 17)
    b = draw_beams(cfg, 17)
    np.testing.assert_array_equal(a, b)
    c = draw_beams(cfg.with_(B=5), 17)          # request b does not depend on the batch size
    np.testing.assert_array_equal(a[:5], c)
    assert not np.array_equal(draw_beams(cfg, 18), a)
    assert a.min() >= 0 and a.max() < cfg.V


def test_geometric_share_ratios_span_the_sweep():
    from oracle import pack_beams
    ratios = []
    for name in ("dedup_p0.1", "dedup_p0.5", "dedup_p0.9"):
        cfg = get_config(name).with_(B=8)
        r = pack_beams(draw_beams(cfg, base_seed(cfg)))["length"].mean() / cfg.P_max
        ratios.append(r)
    assert ratios[0] > 0.95 and 0.8 < ratios[1] < 0.95 and 0.25 < ratios[2] < 0.5


def test_node_tensors_depend_only_on_prefix():
    cfg = get_config("llama_mha").with_(B=2, Hq=2, Hkv=2, D=8)
    beams = draw_beams(cfg, 3)
    t = unpacked_node_tensors(cfg, 3, beams)
    for b in range(cfg.B):
        for w in range(cfg.W):
            for w2 in range(cfg.W):
                for l in range(cfg.L):
                    same = (beams[b, w, :l + 1] == beams[b, w2, :l + 1]).all()
                    for key in ("q", "k", "v", "hidden"):
                        eq = np.array_equal(t[key][b, w, l], t[key][b, w2, l])
                        assert eq == same
    sub = unpacked_node_tensors(cfg, 3, beams, requests=[1])
    np.testing.assert_array_equal(sub["q"][0], t["q"][1])


def test_value_distributions():
    cfg = get_config("llama_mha").with_(V=512, S=256)
    w = lm_weight(cfg, 1)
    assert w.shape == (512, cfg.hidden) and abs(w.std() - 0.02) < 1e-3
    np.testing.assert_array_equal(round_to_bf16(w), w)
    k, v = kv_cache(cfg, 1, 0)
    assert k.shape == (cfg.Hkv, cfg.S, cfg.D) and abs(k.std() - 1) < 0.01 and abs(v.mean()) < 0.01
    f32 = get_config("tiny_f32")
    k32, _ = kv_cache(f32, 1, 0)
    assert k32.dtype == np.float32 and not np.array_equal(round_to_bf16(k32), k32)
