"""The seeded input generators: rounding, determinism, prefix consistency."""
import numpy as np

from fixed_cost_drafter_amd import workload as WLM


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 4.5,
                  1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    got = WLM.bf16_bits_to_f32(WLM.f32_to_bf16_bits(x)).tolist()
    # 1+2^-8 is halfway between 1 and 1+2^-7: ties to even -> 1.0
    # 1+3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 1+2^-6
    assert got == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 4.5, 1.0 + 2 ** -7]


def test_prefix_is_deterministic_and_prefix_consistent():
    wl = WLM.WORKLOADS["tiny_f32"].with_(dtype="bf16", C=3, Hkv=2, d=16, L0=50)
    K1, V1 = WLM.prefix(wl, threads=1)
    K2, V2 = WLM.prefix(wl, threads=4)
    np.testing.assert_array_equal(K1, K2)
    np.testing.assert_array_equal(V1, V2)
    Ks, Vs = WLM.prefix(wl, L0=20, threads=2)
    np.testing.assert_array_equal(Ks, K1[:, :20])
    np.testing.assert_array_equal(Vs, V1[:, :20])
    Kl, _ = WLM.prefix(wl, L0=20, threads=2, rows_alloc=64)
    assert Kl.shape == (3, 64, 2, 16)
    np.testing.assert_array_equal(Kl[:, :20], K1[:, :20])


def test_logits_plant_a_unique_lowest_index_maximum():
    wl = WLM.WORKLOADS["tiny_f32"].with_(dtype="bf16", C=8, B=6, V=300)
    x, g = WLM.logits_entry(wl, 0)
    xf = WLM.bf16_bits_to_f32(x)
    for c in range(wl.C):
        for i in range(wl.B + 1):
            row = xf[c, i]
            assert row[g[c, i]] == WLM.LOGIT_TOP
            assert np.all(row[: g[c, i]] < WLM.LOGIT_TOP)
    assert (xf == WLM.LOGIT_TOP).sum() > wl.C * (wl.B + 1)   # some planted ties exist


def test_draft_tokens_match_at_the_stated_rate():
    wl = WLM.WORKLOADS["tiny_f32"].with_(C=200, B=8, V=50, p_match=0.8)
    _, g = WLM.logits_entry(wl, 0)
    rnd = WLM.round_inputs(wl, 0, g)
    rate = (rnd["draft"] == g[:, : wl.B]).mean()
    assert abs(rate - 0.8) < 0.04
    assert rnd["draft"].min() >= 0 and rnd["draft"].max() < wl.V


def test_lambda_rule_and_state_bytes():
    wl = WLM.WORKLOADS["q3_8b_32k"]
    lam = WLM.lambdas(wl)
    assert lam[0] == 0.0 and lam[1] == 0.5 and lam[16] == 0.0 and lam[15] == 1 - 2 ** -15
    assert np.isneginf(WLM.log_lambda(wl)[0])
    # ring 4 MiB + fp32 summary ~1 MiB + bf16 slots 0.5 MiB per sequence
    assert 5.4 * 2 ** 20 < WLM.state_bytes(wl) < 5.6 * 2 ** 20


def test_named_workloads_come_from_their_config_files(tmp_path):
    """The five workloads are the JSON files under configs/; a file of one's
    own loads the same way, and unknown fields are refused."""
    import json
    import os
    from fixed_cost_drafter_amd import workload as WLM
    assert sorted(WLM.WORKLOADS) == sorted(WLM.CONFIG_NAMES)
    for name in WLM.CONFIG_NAMES:
        path = os.path.join(WLM.CONFIG_DIR, name + ".json")
        assert WLM.load_workload(path) == WLM.WORKLOADS[name]
        assert WLM.resolve_workload(name) is WLM.WORKLOADS[name]
    h = WLM.WORKLOADS["q3_8b_128k"]
    assert (h.C, h.Hq, h.Hkv, h.d, h.L0, h.W, h.S, h.B, h.V) == (16, 32, 8, 128, 131072, 1024, 128, 16, 151936)
    own = dict(name="own", dtype="bf16", C=2, Hq=8, Hkv=2, d=128, L0=300, W=64, S=64, B=5, V=2000,
               rounds=3, p_match=0.8, seed=5, lambdas=[1.0] * 64, about="a test shape")
    p = tmp_path / "own.json"
    p.write_text(json.dumps(own))
    wl = WLM.resolve_workload(str(p))
    assert wl.C == 2 and wl.lambdas == tuple([1.0] * 64) and wl.logits_pool == 0
    own["Q"] = 1
    p.write_text(json.dumps(own))
    import pytest
    with pytest.raises(ValueError):
        WLM.load_workload(str(p))
    with pytest.raises(KeyError):
        WLM.resolve_workload("no_such_workload")
