"""The seeded input generator: determinism, per-head regeneration, laws."""
import numpy as np

import synthetic as syn


def test_bf16_rounding_is_exact_and_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3, 65504.0], np.float32)
    r = syn.round_bf16(x)
    # representable in bf16: low 16 bits are zero
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties to even -> 1.0
    assert r[1] == np.float32(1.0)
    assert syn.round_bf16(r).tobytes() == r.tobytes()
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(t, r)


def test_heads_regenerate_independently():
    case = syn.CFG3.with_(B=2, H=3, T=128)
    full = syn.chunk_inputs(case)
    part = syn.chunk_inputs(case, heads=[(1, 2), (0, 1)])
    for key in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(full[key][1, 2], part[key][0])
        assert np.array_equal(full[key][0, 1], part[key][1])


def test_laws():
    case = syn.CFG3.with_(B=1, H=2, T=512)
    x = syn.chunk_inputs(case)
    n = np.linalg.norm(x["k"].astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)               # unit norm up to bf16 rounding
    assert np.all((x["beta"] > 0) & (x["beta"] < 1))
    assert np.all(x["g"] < 0)
    assert abs(np.mean(x["g"]) + 0.806) < 0.05        # E[softplus(N(0,1))] ~ 0.806
    c2 = syn.chunk_inputs(syn.CFG2.with_(B=1, H=1, T=2048))
    assert np.all(c2["q"] > 0) and c2["g"] is None and c2["beta"] is None
    c4 = syn.chunk_inputs(syn.CFG4.with_(T=64, H=1))
    assert c4["g"].shape == (1, 1, 64, 128)


def test_decode_tokens_deterministic():
    case = syn.CFG5.__class__("t", 4, 2, 16, 16, 3)
    a = syn.decode_tokens(case, 1)
    b = syn.decode_tokens(case, 1)
    c = syn.decode_tokens(case, 2)
    assert np.array_equal(a["q"], b["q"]) and not np.array_equal(a["q"], c["q"])
    s = syn.decode_state(case)
    assert s.shape == (4, 2, 16, 16) and abs(float(s.std()) - 0.02) < 0.003
