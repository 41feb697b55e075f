"""The seeded input generator (shared by both sides of every parity check)."""
import numpy as np

import sdm_inputs as si


def test_deterministic_and_thread_independent():
    wl = si.WORKLOADS[2].with_(B=2)
    a = si.generate(wl, T=1500, threads=1)
    b = si.generate(wl, T=1500, threads=6)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_truncation_is_a_prefix():
    wl = si.WORKLOADS[1].with_(B=2)
    a = si.generate(wl, T=1100)
    b = si.generate(wl, T=700)
    for k in ("qp", "v", "alpha", "beta"):
        np.testing.assert_array_equal(a[k][:, :700], b[k])
    np.testing.assert_array_equal(a["M0"], b["M0"])


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0, -0.0],
                 dtype=np.float32)
    bits = si.f32_to_bf16_bits(x)
    back = si.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    np.testing.assert_array_equal(back, np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0, -0.0],
                                                 dtype=np.float32))
    assert np.signbit(back[-1])


def test_key_reuse_structure():
    wl = si.WORKLOADS[4]
    d = si.generate(wl.with_(d_v=8, sqrtN=16), T=20000)
    src = d["src"][0]
    frac = (src != np.arange(src.size)).mean()
    assert 0.08 < frac < 0.12
    assert (src <= np.arange(src.size)).all()
    np.testing.assert_array_equal(d["kp"][0], d["kp"][0][src])
    # q' is never reused
    assert (d["qp"][0, 1:] != d["qp"][0, :-1]).any(axis=(1, 2)).all()


def test_distributions():
    wl = si.WORKLOADS[1].with_(B=2, H=4)
    d = si.generate(wl, T=2048)
    assert abs(d["kp"].mean()) < 0.01 and abs(d["kp"].std() - 1) < 0.01
    assert abs(d["M0"].std() - 0.02) < 1e-3
    assert ((d["alpha"] > 0) & (d["alpha"] <= 1)).all()
    assert ((d["beta"] > 0) & (d["beta"] < 1)).all()
    assert abs(np.median(d["beta"]) - 0.5) < 0.02
