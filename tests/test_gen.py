"""Synthetic workload generator: shapes, determinism, subset consistency."""

import numpy as np

from gen import SPECS, make_config, make_custom, to_bf16_bits, bf16_bits_to_f32


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38], dtype=np.float32)
    back = bf16_bits_to_f32(to_bf16_bits(x))
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa (1.0) wins;
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even (1+2^-6) wins
    assert list(back[:4]) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0]
    assert back[4] == -2.5


def test_tiny_config_shapes_and_determinism():
    a = make_config(0)
    b = make_config(0)
    assert a.U.shape == (4, 5, 1024) and a.target.shape == (4, 6, 1024)
    assert a.W1.shape == (1024, 32) and a.W2.shape == (32, 1024) and a.w.shape == (96,)
    assert a.uniforms.shape == (4, 6, 2) and np.all(a.uniforms < 1) and np.all(a.uniforms >= 0)
    for f in ("U", "target", "W1", "W2", "w", "hidden", "anchor", "uniforms"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.sps[0] == 0 and abs(a.sps[64] - 500.0) < 1e-12


def test_subset_rows_equal_full_rows():
    full = make_config(0)
    sub = make_config(0, requests=[2, 3])
    np.testing.assert_array_equal(sub.U, full.U[2:4])
    np.testing.assert_array_equal(sub.target, full.target[2:4])
    np.testing.assert_array_equal(sub.uniforms, full.uniforms[2:4])


def test_large_config_subset_structure():
    w = make_config(4, requests=range(3))
    assert w.U.dtype == np.uint16 and w.U.shape == (3, 7, 151936)
    spec = SPECS[4]
    full_T = make_config(4, requests=range(spec.B), with_target=False).temperature
    assert int((full_T == 0).sum()) == 51
    u = bf16_bits_to_f32(w.U[0, 0])
    # three peaks of +8..+12 over a N(0, 1.5) background
    assert (u > 7.0).sum() >= 3 and abs(u.std() - 1.5) < 0.05


def test_rnn_weights_shapes_and_streams():
    from gen.workloads import rnn_weights
    a = rnn_weights(32, 64, "f32", seed=0)
    b = rnn_weights(32, 64, "f32", seed=0)
    c = rnn_weights(32, 64, "bf16", seed=0)
    assert a["Wr"].shape == (96, 128) and a["br"].shape == (96,)
    np.testing.assert_array_equal(a["Wr"], b["Wr"])
    assert c["Wr"].dtype == np.uint16
    # each column block adds O(1) to the pre-activations
    assert 0.1 < float(np.std(a["Wr"][:, :32])) * np.sqrt(32) < 10
    assert 0.1 < float(np.std(a["Wr"][:, 64:])) * np.sqrt(64) < 10
    # the RNN draw leaves the other components' draws unchanged
    w0 = make_custom(2, 3, 64, 32, 16, "f32", "gaussian", seed=0)
    w1 = make_custom(2, 3, 64, 32, 16, "f32", "gaussian", seed=0)
    np.testing.assert_array_equal(w0.W2, w1.W2)
