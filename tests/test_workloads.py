"""The seeded input generator: determinism, exact ignore counts, label law."""
import numpy as np

import workloads as wk


def test_deterministic_and_seed_sensitive():
    wl = wk.custom(300, 40, 700, ignore_frac=0.05, label_dist="zipf", seed=7)
    a, b = wk.draw(wl), wk.draw(wl)
    assert a.digest() == b.digest()
    c = wk.draw(wk.custom(300, 40, 700, ignore_frac=0.05, label_dist="zipf", seed=8))
    assert c.digest() != a.digest()


def test_slab_parallel_fill_is_thread_count_independent(monkeypatch):
    wl = wk.custom(9000, 16, 10, seed=3)
    a = wk.draw(wl)
    monkeypatch.setattr(wk, "_threads", lambda: 1)
    b = wk.draw(wl)
    assert a.digest() == b.digest()


def test_exact_ignore_counts_of_named_workloads():
    want = {1: 0, 2: 205, 3: 164, 4: 492, 5: 328}
    for k, n in want.items():
        assert wk.WORKLOADS[k].n_ignored == n


def test_labels_and_bf16_rounding():
    wl = wk.custom(2000, 24, 5000, ignore_frac=0.1, label_dist="zipf", zipf_s=1.1, seed=11)
    inp = wk.draw(wl)
    y = inp.labels
    assert y.dtype == np.int32
    assert (y == -100).sum() == 200
    v = y[y != -100]
    assert v.min() >= 0 and v.max() < 5000
    # bf16 values round-trip exactly and the RNE rounding is within half an ulp
    assert np.array_equal(wk.bf16_bits_to_f32(inp.X_bits), inp.X)
    raw = np.float32(1.0) + np.float32(2.0 ** -8)  # exactly halfway between bf16 1 and 1+2^-7
    assert wk.bf16_bits_to_f32(wk.round_to_bf16_bits(np.array([raw])))[0] == 1.0  # ties to even
    raw = np.float32(1.0) + np.float32(3 * 2.0 ** -8)  # halfway between 1+2^-7 and 1+2^-6
    assert wk.bf16_bits_to_f32(wk.round_to_bf16_bits(np.array([raw])))[0] == np.float32(1 + 2.0 ** -6)


def test_zipf_head_mass():
    # The most frequent label of Zipf(s) on V ranks has probability
    # 1 / sum_k k^-s: 0.1333 for s = 1.1, V = 128256.
    g = np.random.default_rng(0)
    r = wk._zipf_ranks(g, 200_000, 128256, 1.1)
    frac = (r == 0).mean()
    assert abs(frac - 0.13334) < 4 * np.sqrt(0.1333 * 0.8667 / 200_000)


def test_draw_logits_deterministic_labels_and_scale():
    # the logits of the loss-on-logits path: seeded, the same labels as draw(),
    # N(0, (w_sigma sqrt H)^2) -- the spread of x.w for unit x and W of sd w_sigma
    wl = wk.custom(600, 256, 3001, "bf16", 0.02, "zipf", 1.1, 0.05, 0.0, seed=21)
    a, b = wk.draw_logits(wl), wk.draw_logits(wl)
    assert a.digest() == b.digest()
    assert np.array_equal(a.labels, wk.draw(wl).labels)
    assert np.array_equal(wk.bf16_bits_to_f32(a.Z_bits), a.Z)
    sd = 0.02 * np.sqrt(256)
    assert abs(a.Z.std() / sd - 1.0) < 0.01 and abs(a.Z.mean()) < 0.01 * sd
    f = wk.draw_logits(wk.custom(600, 256, 3001, "fp32", 0.02, seed=21))
    assert f.Z_bits is None and f.Z.dtype == np.float32
