"""The seeded input generator: determinism and the stated distributions."""
import numpy as np

from w4_gemv_greedy_amd import synth


def test_deterministic_and_distinct():
    a = synth.weights(64, 1024, workload=1, matrix=synth.O_PROJ, layer=2)
    b = synth.weights(64, 1024, workload=1, matrix=synth.O_PROJ, layer=2)
    c = synth.weights(64, 1024, workload=1, matrix=synth.O_PROJ, layer=3)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    assert not np.array_equal(a[0], c[0])


def test_weight_distributions():
    wq, sc, bi = synth.weights(2048, 1024, workload=1)
    assert wq.shape == (2048, 128) and wq.dtype == np.uint32
    assert sc.shape == bi.shape == (2048, 16) and sc.dtype == np.uint16
    codes = np.stack([(wq >> np.uint32(4 * j)) & np.uint32(15) for j in range(8)])
    hist = np.bincount(codes.ravel(), minlength=16) / codes.size
    assert np.all(np.abs(hist - 1 / 16) < 0.002)
    s = synth.bf16_bits_to_f32(sc)
    assert np.all(np.abs(s) >= 0.0019) and np.all(np.abs(s) <= 0.0201)
    assert 0.45 < np.mean(s > 0) < 0.55
    b = synth.bf16_bits_to_f32(bi)
    eps = b + 8 * s
    assert abs(float(np.mean(eps))) < 1e-4 and 0.8e-3 < float(np.std(eps)) < 1.3e-3


def test_activation_distribution():
    x = synth.bf16_bits_to_f32(synth.activations(4, 8192, workload=2))
    assert abs(float(x.mean())) < 0.05 and 0.95 < float(x.std()) < 1.05


def test_bf16_rounding():
    v = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, 1e-40], np.float32)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v))
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == np.float32(1.015625) and got[3] == -2.5
    assert np.isfinite(got[4]) and got[5] >= 0


def test_planted_logits():
    x, notes = synth.planted_logits(5000)
    assert x.shape == (8, 5000) and len(notes) == 8
    assert np.isnan(x[2]).sum() == 1 and np.isposinf(x[3]).sum() == 1 and np.isneginf(x[4]).sum() == 1
