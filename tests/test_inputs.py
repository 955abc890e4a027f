"""The seeded input generator: determinism and bf16 rounding (checked against
torch's float32 -> bfloat16 conversion, which rounds to nearest even)."""
import numpy as np
import torch

import tc_inputs


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, -2.5, 3.0039062, 1.00390625, 1.01171875, 0.0, -0.0], np.float32)])
    ours = tc_inputs.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    bits = tc_inputs.bf16_bits(ours)
    assert np.array_equal(bits, torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_generator_is_deterministic_and_shaped():
    a = tc_inputs.prefill_inputs(2, T=128)
    b = tc_inputs.prefill_inputs(2, T=128)
    for key in ["q", "k", "v", "lam", "eta", "gate"]:
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (8, 8, 128, 64)
    assert np.all((a["lam"] > 0.88) & (a["lam"] < 0.9934))
    assert np.all((a["eta"] > 0.047) & (a["eta"] < 0.5))
    c = tc_inputs.prefill_inputs(1)
    assert c["q"].dtype == np.float32 and c["q"].shape == (1, 1, 64, 16)
    assert c["lam"][0] == np.float32(0.9) and c["eta"][0] == np.float32(0.5) and c["gate"][0] == 0


def test_plants_repeat_keys_more_than_window_apart():
    d = tc_inputs.prefill_inputs(3, T=4096, H=2)
    W = 1024
    pl = d["plants"]
    assert len(pl) == 2 * round(0.05 * 4096)
    for b, h, i, j in pl[:200]:
        assert j > i + W
        assert np.array_equal(d["k"][b, h, i], d["k"][b, h, j])
