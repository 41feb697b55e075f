"""CPU pins of the float64 oracle (no GPU).

Each test ties the oracle to something other than itself: hand-worked
fixtures (tests/golden), an independent brute-force sort over all N scores,
closed forms of the recurrence, or exact algebraic invariants.
"""
import numpy as np
import pytest

import oracle
import sdm_inputs as si
from oracle import brute


# ---------------------------------------------------------------- selection

def test_golden_topk(golden):
    for c in golden("topk_outer_sum.txt"):
        S, K = int(c["sqrtN"][0]), int(c["K"][0])
        x = np.array(c["x"], dtype=np.float32)
        idx, w = oracle.select(x, S, K)
        assert idx.tolist() == [int(v) for v in c["idx"]], c["name"]
        np.testing.assert_allclose(w, c["w"], rtol=0, atol=1e-15, err_msg=c["name"])
        bi, bw = brute.topk(x, S, K)
        assert bi.tolist() == idx.tolist(), c["name"]


def test_pkm_identity_tiny_all_headtokens():
    wl = si.WORKLOADS[0]
    d = si.generate(wl)
    for key, K in (("kp", wl.W), ("qp", wl.R)):
        idx, w = oracle.select(d[key], wl.sqrtN, K)
        bi, bw = brute.topk_rows(d[key], wl.sqrtN, K)
        np.testing.assert_array_equal(idx, bi)
        np.testing.assert_allclose(w, bw, rtol=1e-14, atol=0)


@pytest.mark.parametrize("seed", range(6))
def test_pkm_identity_massive_ties(seed):
    """Small-integer inputs: most scores tie, so the index tie-break decides."""
    rng = np.random.default_rng(seed)
    for _ in range(40):
        S = int(rng.integers(1, 13))
        K = int(rng.integers(1, S + 1))
        x = rng.integers(-2, 3, size=(3, 2 * S)).astype(np.float32)
        if rng.random() < 0.3:
            x[:] = np.where(rng.random(x.shape) < 0.5, -0.0, 0.0)
        idx, w = oracle.select(x, S, K)
        bi, bw = brute.topk_rows(x, S, K)
        np.testing.assert_array_equal(idx, bi, err_msg=f"S={S} K={K} x={x}")
        np.testing.assert_allclose(w, bw, rtol=1e-14, atol=0)


def test_pkm_identity_bf16_ties():
    """bf16 inputs: exact ties straddle the K boundary in many vectors."""
    rng = np.random.default_rng(7)
    S, K = 64, 64
    x = si.f32_to_bf16_bits(rng.standard_normal((48, 2 * S)).astype(np.float32))
    idx, w = oracle.select(x, S, K)
    bi, bw = brute.topk_rows(x, S, K)
    np.testing.assert_array_equal(idx, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-14, atol=0)


def test_pkm_identity_extreme_magnitudes():
    """Sums of values ~2^40 apart: a float64 sum alone would round them."""
    rng = np.random.default_rng(11)
    S, K = 8, 6
    big = rng.choice([1.0, -1.0], size=(64, 2 * S)) * 2.0 ** 20
    tiny = rng.standard_normal((64, 2 * S)) * 2.0 ** -40
    x = np.where(rng.random((64, 2 * S)) < 0.5, big, big + tiny).astype(np.float32)
    x[:, :S] = np.where(rng.random((64, S)) < 0.5, x[:, :S], tiny[:, :S].astype(np.float32))
    idx, _ = oracle.select(x, S, K)
    bi, _ = brute.topk_rows(x, S, K)
    np.testing.assert_array_equal(idx, bi)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_pkm_identity_workload_samples(cfg):
    """Sampled head-tokens of every workload shape (same input recipe)."""
    wl = si.WORKLOADS[cfg]
    d = si.generate(wl.with_(B=1), T=8)
    rows = 8 if cfg == 4 else 16
    for key, K in (("kp", wl.W), ("qp", wl.R)):
        x = d[key].reshape(-1, 2 * wl.sqrtN)[:rows]
        idx, w = oracle.select(x, wl.sqrtN, K)
        bi, bw = brute.topk_rows(x, wl.sqrtN, K)
        np.testing.assert_array_equal(idx, bi)
        np.testing.assert_allclose(w, bw, rtol=1e-13, atol=0)


def test_weights_are_a_distribution():
    wl = si.WORKLOADS[1]
    d = si.generate(wl.with_(B=1), T=16)
    idx, w = oracle.select(d["kp"], wl.sqrtN, wl.W)
    assert (w > 0).all()
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (np.diff(w, axis=-1) <= 0).all()  # listed by descending score
    # slots are distinct and inside [0, N)
    s = np.sort(idx, axis=-1)
    assert (np.diff(s, axis=-1) > 0).all() and s.min() >= 0 and s.max() < wl.N


# ---------------------------------------------------------------- recurrence

def _run(inp, S, W, R, **kw):
    return oracle.forward(inp, S, W, R, **kw)


def test_golden_recurrence(golden):
    (c,) = golden("recurrence_small.txt")
    S, D, T = int(c["sqrtN"][0]), int(c["d_v"][0]), int(c["T"][0])
    inp = dict(
        kp=np.array(c["kp"], np.float32).reshape(1, T, 1, 2 * S),
        qp=np.array(c["qp"], np.float32).reshape(1, T, 1, 2 * S),
        v=np.array(c["v"], np.float32).reshape(1, T, 1, D),
        alpha=np.array(c["alpha"], np.float32).reshape(1, T, 1),
        beta=np.array(c["beta"], np.float32).reshape(1, T, 1),
        M0=np.array(c["M0"], np.float32).reshape(1, S * S, D))
    o = _run(inp, S, 1, 1)
    assert o["Iw"].reshape(-1).tolist() == [int(v) for v in c["Iw"]]
    assert o["Ir"].reshape(-1).tolist() == [int(v) for v in c["Ir"]]
    assert (o["kw"] == 1.0).all() and (o["qw"] == 1.0).all()
    np.testing.assert_array_equal(o["y"].reshape(-1), c["y"])
    np.testing.assert_array_equal(o["M"].reshape(-1), c["M"])


def _tiny(seed=0, B=2, T=24, H=2, S=6, D=5, W=3, R=3):
    wl = si.Workload("t", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype="f32",
                     reuse=0.0, seed=seed)
    return wl, si.generate(wl)


def test_unselected_rows_bit_unchanged():
    """Rows never selected for writing keep M_0 bit for bit (sparse write)."""
    wl, d = _tiny(seed=3, S=8)
    # concentrate the keys so that only a few slots are ever written
    d["kp"][..., :wl.sqrtN] = -8.0
    d["kp"][..., :2] = 8.0
    o = _run(d, wl.sqrtN, wl.W, wl.R)
    for b in range(wl.B):
        for h in range(wl.H):
            written = np.unique(o["Iw"][b, :, h])
            never = np.setdiff1d(np.arange(wl.N), written)
            assert never.size > 0
            np.testing.assert_array_equal(o["M"][b, h, never], d["M0"][h, never].astype(np.float64))


def test_beta_zero_is_pure_decay():
    """beta = 0: a selected row only decays, M_T[i] = prod(alpha) * M_0[i]."""
    wl, d = _tiny(seed=4)
    d["beta"][:] = 0.0
    o = _run(d, wl.sqrtN, wl.W, wl.R)
    Iw, _ = brute.topk_rows(d["kp"], wl.sqrtN, wl.W)  # independent selection
    np.testing.assert_array_equal(Iw, o["Iw"])
    for b in range(wl.B):
        for h in range(wl.H):
            f = np.ones(wl.N)
            for t in range(wl.T):
                f[Iw[b, t, h]] *= float(d["alpha"][b, t, h])
            ref = f[:, None] * d["M0"][h].astype(np.float64)
            np.testing.assert_allclose(o["M"][b, h], ref, rtol=1e-14, atol=0)


def test_alpha_one_beta_one_overwrites_row():
    """alpha = beta = 1 and W = 1 (k = 1): a written row becomes v_t exactly."""
    wl, d = _tiny(seed=5, W=1)
    d["alpha"][:] = 1.0
    d["beta"][:] = 1.0
    o = _run(d, wl.sqrtN, 1, wl.R)
    assert (o["kw"] == 1.0).all()
    for b in range(wl.B):
        for h in range(wl.H):
            last = {}
            for t in range(wl.T):
                last[int(o["Iw"][b, t, h, 0])] = t
            for s, t in last.items():
                np.testing.assert_array_equal(o["M"][b, h, s], d["v"][b, t, h].astype(np.float64))


def test_repeated_writes_closed_form():
    """One shared k' for every token: a fixed write set with fixed weights k.

    Then M_T[i] = (prod_t a_t) M_0[i] + sum_t c_t (prod_{l>t} a_l) v_t with
    a_t = alpha_t (1 - beta_t k) and c_t = beta_t k, the unrolled affine map.
    """
    wl, d = _tiny(seed=6, T=40, W=4)
    d["kp"][:] = d["kp"][:, :1]
    o = _run(d, wl.sqrtN, wl.W, wl.R)
    for b in range(wl.B):
        for h in range(wl.H):
            for w in range(wl.W):
                s = int(o["Iw"][b, 0, h, w])
                k = float(o["kw"][b, 0, h, w])
                al = d["alpha"][b, :, h].astype(np.float64)
                be = d["beta"][b, :, h].astype(np.float64)
                a = al * (1.0 - be * k)
                c = be * k
                ref = np.prod(a) * d["M0"][h, s].astype(np.float64)
                for t in range(wl.T):
                    ref = ref + c[t] * np.prod(a[t + 1:]) * d["v"][b, t, h].astype(np.float64)
                np.testing.assert_allclose(o["M"][b, h, s], ref, rtol=1e-12, atol=1e-15)


def test_one_hot_read_returns_row():
    """R = 1 (q = 1): y_t is the post-write row M_t[slot], bit for bit."""
    wl, d = _tiny(seed=8, T=10, R=1)
    for t in range(wl.T):
        sub = {k: (v[:, :t + 1] if k not in ("M0", "src") else v) for k, v in d.items()}
        o = _run(sub, wl.sqrtN, wl.W, 1)
        for b in range(wl.B):
            for h in range(wl.H):
                s = int(o["Ir"][b, t, h, 0])
                np.testing.assert_array_equal(o["y"][b, t, h], o["M"][b, h, s])


def test_dominant_read_weight_underflows_others():
    """A score gap above 800 makes the other read weights exactly 0."""
    wl, d = _tiny(seed=9, T=6, R=4)
    S = wl.sqrtN
    d["qp"][:] = 0.0
    d["qp"][..., 0] = 900.0          # q'_1[0]
    d["qp"][..., S + 1:] = -900.0    # q'_2[j > 0]
    o = _run(d, S, wl.W, 4)
    assert (o["Ir"][..., 0] == 0).all()
    assert (o["qw"][..., 0] == 1.0).all() and (o["qw"][..., 1:] == 0.0).all()
    np.testing.assert_array_equal(o["y"][:, -1], o["M"][:, :, 0])


def test_scaling_by_two_is_exact():
    """The recurrence is linear in (M_0, v): doubling both doubles y and M exactly."""
    wl, d = _tiny(seed=10)
    o1 = _run(d, wl.sqrtN, wl.W, wl.R)
    d2 = dict(d, M0=d["M0"] * 2, v=d["v"] * 2)
    o2 = _run(d2, wl.sqrtN, wl.W, wl.R)
    np.testing.assert_array_equal(o2["y"], 2 * o1["y"])
    np.testing.assert_array_equal(o2["M"], 2 * o1["M"])


def test_column_window_matches_full_run():
    """Columns never interact, so a column window reproduces the full run."""
    wl, d = _tiny(seed=12, D=19)
    full = _run(d, wl.sqrtN, wl.W, wl.R)
    part = _run(d, wl.sqrtN, wl.W, wl.R, c0=5, c1=14)
    np.testing.assert_array_equal(part["y"], full["y"][..., 5:14])
    np.testing.assert_array_equal(part["M"], full["M"][..., 5:14])


def test_bf16_inputs_are_widened_exactly():
    wl, d = _tiny(seed=13)
    bf = {k: (si.f32_to_bf16_bits(d[k]) if k in ("kp", "qp", "v") else d[k]) for k in d}
    wid = {k: (si.bf16_bits_to_f32(bf[k]) if k in ("kp", "qp", "v") else d[k]) for k in d}
    a = _run(bf, wl.sqrtN, wl.W, wl.R)
    b = _run(wid, wl.sqrtN, wl.W, wl.R)
    for k in ("Iw", "Ir", "kw", "qw", "y", "M"):
        np.testing.assert_array_equal(a[k], b[k])


def test_thread_count_does_not_change_results():
    wl, d = _tiny(seed=14, D=21)
    a = oracle.forward(d, wl.sqrtN, wl.W, wl.R, threads=1)
    b = oracle.forward(d, wl.sqrtN, wl.W, wl.R, threads=5)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_bad_arguments_rejected():
    x = np.zeros((2, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.select(x, 4, 5)  # K > sqrtN
    with pytest.raises(ValueError):
        oracle.select(x, 3, 2)  # wrong length


# ------------------------------------------------- state size (closed form)

@pytest.mark.parametrize("cfg,d_model", [(1, 2048), (2, 2048), (3, 4096), (4, 2048)])
def test_state_size_equation(cfg, d_model):
    """Eq. (6) of the explainer (§3.3): (d_qk^tot)^2 d_v^tot / (4 H^2) = H N d_v,
    with d_qk^tot = d/2 and d_v^tot = d (isoFLOP rule, §3.2)."""
    wl = si.WORKLOADS[cfg]
    dqk, dv = d_model // 2, d_model
    assert dqk % (2 * wl.H) == 0
    assert wl.sqrtN == dqk // (2 * wl.H) and wl.d_v == dv // wl.H
    assert dqk * dqk * dv // (4 * wl.H * wl.H) == wl.H * wl.N * wl.d_v


# ------------------------------------------------------ bfloat16 state (reading)

def test_round_bf16_matches_torch_conversion():
    """The oracle's bfloat16 rounding (nearest, ties to even) agrees with
    torch's float32 -> bfloat16 conversion on float32 inputs: random values
    over many binades, exact halfway cases with even and odd neighbours,
    subnormals and signed zeros."""
    import torch
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-40, 40, 20000))).astype(np.float32)
    bits = rng.integers(0, 2**31 - 1, 4000, dtype=np.int64).astype(np.uint32)
    ties = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)              # exactly halfway
    sub = (rng.integers(1, 2**23, 2000, dtype=np.int64).astype(np.uint32)).view(np.float32)
    special = np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 3.0078125, 0.1, 65504.0], np.float32)
    for arr in (x, ties[np.isfinite(ties)], sub, -sub, special):
        want = torch.from_numpy(arr.copy()).to(torch.bfloat16).to(torch.float64).numpy()
        got = oracle.round_bf16(arr.astype(np.float64))
        np.testing.assert_array_equal(got, want)


def test_golden_recurrence_bf16_state(golden):
    (c,) = golden("recurrence_bf16_state.txt")
    S, D, T = int(c["sqrtN"][0]), int(c["d_v"][0]), int(c["T"][0])
    inp = dict(
        kp=np.array(c["kp"], np.float32).reshape(1, T, 1, 2 * S),
        qp=np.array(c["qp"], np.float32).reshape(1, T, 1, 2 * S),
        v=np.array(c["v"], np.float32).reshape(1, T, 1, D),
        alpha=np.array(c["alpha"], np.float32).reshape(1, T, 1),
        beta=np.array(c["beta"], np.float32).reshape(1, T, 1),
        M0=np.array(c["M0"], np.float32).reshape(1, S * S, D))
    o = oracle.forward(inp, S, 1, 1, state="bf16")
    np.testing.assert_array_equal(o["y"].reshape(-1), c["y"])
    np.testing.assert_array_equal(o["M"].reshape(-1), c["M"])
    # the float64 state keeps the low bits the bfloat16 state drops
    o64 = oracle.forward(inp, S, 1, 1)
    assert o64["y"].reshape(-1)[0] != c["y"][0]


def test_bf16_state_unwritten_rows_are_rounded_m0():
    wl, d = _tiny(seed=31, S=8)
    d["kp"][..., :wl.sqrtN] = -8.0
    d["kp"][..., :2] = 8.0
    o = oracle.forward(d, wl.sqrtN, wl.W, wl.R, state="bf16")
    for b in range(wl.B):
        for h in range(wl.H):
            never = np.setdiff1d(np.arange(wl.N), np.unique(o["Iw"][b, :, h]))
            assert never.size > 0
            np.testing.assert_array_equal(o["M"][b, h, never],
                                          oracle.round_bf16(d["M0"][h, never].astype(np.float64)))


def test_bf16_state_overwrite_gate():
    """alpha = beta = 1 with W = 1 (weight 1): the written row becomes
    bfloat16(v_t) exactly."""
    wl, d = _tiny(seed=32, W=1, R=1)
    d["alpha"][:] = 1.0
    d["beta"][:] = 1.0
    o = oracle.forward(d, wl.sqrtN, 1, 1, state="bf16")
    for b in range(wl.B):
        for h in range(wl.H):
            last = {}
            for t in range(wl.T):
                last[int(o["Iw"][b, t, h, 0])] = t
            for s, t in last.items():
                np.testing.assert_array_equal(
                    o["M"][b, h, s], oracle.round_bf16(d["v"][b, t, h].astype(np.float64)))


def test_bf16_state_error_bound():
    """Each stored value carries at most half a bfloat16 spacing (2^-9
    relative) of fresh rounding, and writes are contractions, so the
    bfloat16-state result stays within (writes + 1) * 2^-8 * max|M| of the
    float64-state result (a loose bound: 2^-8 covers the rounding of M_0)."""
    wl, d = _tiny(seed=33, T=40, S=6, W=3, R=3)
    o16 = oracle.forward(d, wl.sqrtN, wl.W, wl.R, state="bf16")
    o64 = oracle.forward(d, wl.sqrtN, wl.W, wl.R)
    scale = max(np.abs(o64["M"]).max(), np.abs(d["v"]).max())
    writes = wl.T  # at most one write per token per slot
    assert np.abs(o16["M"] - o64["M"]).max() <= (writes + 1) * 2.0**-8 * scale
    assert np.abs(o16["y"] - o64["y"]).max() <= (writes + 1) * 2.0**-8 * scale
    assert np.abs(o16["M"] - o64["M"]).max() > 0  # the rounding is really applied


# ------------------------------------------------- scaled E4M3 state (reading)

def _e4m3_values():
    """Every finite non-negative value of the E4M3 format, ascending (from
    torch's decoding of the 256 codes)."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    v = codes.to(torch.float64).numpy()
    return np.unique(v[np.isfinite(v) & (v >= 0)])


@pytest.mark.parametrize("s", [0, -4, 5])
def test_round_fp8_matches_torch_conversion(s):
    """The oracle's E4M3 rounding of x at scale 2^s (nearest, ties to even)
    agrees with torch's float32 -> float8_e4m3fn conversion of x * 2^-s,
    scaled back, wherever torch stays finite (|x * 2^-s| <= 464): random
    values over the whole range, every value halfway between two
    neighbours, the subnormals, signed zeros."""
    import torch
    rng = np.random.default_rng(11 + s)
    a = (rng.standard_normal(30000) * np.exp2(rng.integers(-14, 9, 30000))).astype(np.float32)
    vals = _e4m3_values()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[1:] + vals[:-1]) / 2)  # exact
    sub = np.arange(0, 9, dtype=np.float32) * np.float32(2.0**-9)
    special = np.array([0.0, -0.0, 448.0, 464.0, -464.0, 0.1, 1.0625, 1.1875], np.float32)
    for arr in (a, mids, -mids, sub, special):
        arr = arr[np.abs(arr) <= 464]
        want = torch.from_numpy(arr.copy()).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        got = oracle.round_fp8(arr.astype(np.float64) * 2.0**s, s) * 2.0**-s
        np.testing.assert_array_equal(got, want)
    # ties go to the neighbour with an even last mantissa bit: both ways occur
    up = oracle.round_fp8(mids.astype(np.float64), 0) > mids
    assert up.any() and (~up).any()


def test_round_fp8_saturates():
    """Beyond the largest magnitude the reading saturates (a state must stay
    finite); torch's conversion gives NaN there."""
    x = np.array([464.0001, 480.0, 500.0, 1e6, 1e30])
    for s in (0, -4, 3):
        np.testing.assert_array_equal(oracle.round_fp8(x * 2.0**s, s), 448.0 * 2.0**s)
        np.testing.assert_array_equal(oracle.round_fp8(-x * 2.0**s, s), -448.0 * 2.0**s)


def test_golden_recurrence_fp8_state(golden):
    (c,) = golden("recurrence_fp8_state.txt")
    S, D, T = int(c["sqrtN"][0]), int(c["d_v"][0]), int(c["T"][0])
    sc = int(c["scale_log2"][0])
    inp = dict(
        kp=np.array(c["kp"], np.float32).reshape(1, T, 1, 2 * S),
        qp=np.array(c["qp"], np.float32).reshape(1, T, 1, 2 * S),
        v=np.array(c["v"], np.float32).reshape(1, T, 1, D),
        alpha=np.array(c["alpha"], np.float32).reshape(1, T, 1),
        beta=np.array(c["beta"], np.float32).reshape(1, T, 1),
        M0=np.array(c["M0"], np.float32).reshape(1, S * S, D))
    o = oracle.forward(inp, S, 1, 1, state="fp8", scale_log2=sc)
    np.testing.assert_array_equal(o["y"].reshape(-1), c["y"])
    np.testing.assert_array_equal(o["M"].reshape(-1), c["M"])
    # another scale gives other values (the scale really applies)
    o2 = oracle.forward(inp, S, 1, 1, state="fp8", scale_log2=0)
    assert not np.array_equal(o2["y"], o["y"])


def test_fp8_state_unwritten_rows_and_overwrite_gate():
    """Rows never written hold M_0 rounded to the scaled format; with
    alpha = beta = 1 and W = 1 a written row becomes round(v_t)."""
    wl, d = _tiny(seed=34, S=8)
    d["kp"][..., :wl.sqrtN] = -8.0
    d["kp"][..., :2] = 8.0
    o = oracle.forward(d, wl.sqrtN, wl.W, wl.R, state="fp8", scale_log2=-5)
    for b in range(wl.B):
        for h in range(wl.H):
            never = np.setdiff1d(np.arange(wl.N), np.unique(o["Iw"][b, :, h]))
            assert never.size > 0
            np.testing.assert_array_equal(
                o["M"][b, h, never], oracle.round_fp8(d["M0"][h, never].astype(np.float64), -5))
    wl, d = _tiny(seed=35, W=1, R=1)
    d["alpha"][:] = 1.0
    d["beta"][:] = 1.0
    o = oracle.forward(d, wl.sqrtN, 1, 1, state="fp8", scale_log2=-3)
    for b in range(wl.B):
        for h in range(wl.H):
            last = {int(o["Iw"][b, t, h, 0]): t for t in range(wl.T)}
            for sl, t in last.items():
                np.testing.assert_array_equal(
                    o["M"][b, h, sl], oracle.round_fp8(d["v"][b, t, h].astype(np.float64), -3))


def test_fp8_state_error_bound():
    """Each stored value carries at most half an E4M3 spacing (2^-4 relative
    in the normal range, 2^-10 * 2^s absolute below it) of fresh rounding,
    and writes are contractions, so the state stays within (writes + 1) *
    (2^-4 * max|M| + 2^(s-10)) of the float64 state."""
    wl, d = _tiny(seed=36, T=40, S=6, W=3, R=3)
    s = -4
    o8 = oracle.forward(d, wl.sqrtN, wl.W, wl.R, state="fp8", scale_log2=s)
    o64 = oracle.forward(d, wl.sqrtN, wl.W, wl.R)
    scale = max(np.abs(o64["M"]).max(), np.abs(d["v"]).max())
    bound = (wl.T + 1) * (2.0**-4 * scale + 2.0**(s - 10))
    assert np.abs(o8["M"] - o64["M"]).max() <= bound
    assert np.abs(o8["y"] - o64["y"]).max() <= bound
    assert np.abs(o8["M"] - o64["M"]).max() > 0


# ------------------------------------------------------------------ backward

def _loss(inp, S, W, R, Ry, RM):
    o = oracle.forward(inp, S, W, R)
    return float((o["y"] * Ry).sum() + (o["M"] * RM).sum()), o


@pytest.mark.parametrize("case", [
    dict(B=1, T=6, H=1, S=4, D=3, W=2, R=2, dtype="f32", seed=51),
    dict(B=2, T=9, H=2, S=5, D=4, W=3, R=2, dtype="f32", seed=52),
    dict(B=1, T=12, H=1, S=3, D=5, W=3, R=3, dtype="f32", seed=53),  # every slot rewritten often
    dict(B=2, T=7, H=1, S=4, D=4, W=2, R=3, dtype="bf16", seed=54),
])
def test_backward_matches_finite_differences(case):
    """Every gradient of the oracle's backward (with the selections held
    fixed) against central differences of the forward, for the loss
    L = sum(y * Ry) + sum(M_T * RM) with random Ry, RM."""
    c = dict(case)
    wl = si.Workload("fd", B=c["B"], T=c["T"], H=c["H"], sqrtN=c["S"], d_v=c["D"], W=c["W"],
                     R=c["R"], dtype=c["dtype"], reuse=0.2, seed=c["seed"])
    d = si.generate(wl)
    # gates away from 0 and 1 so that +-h stays a valid gate; M_0 of order 1
    d["alpha"][:] = np.clip(d["alpha"], 0.2, 0.95)
    d["beta"][:] = np.clip(d["beta"], 0.05, 0.95)
    d["M0"][:] = (d["M0"] * 40).astype(np.float32)
    rng = np.random.default_rng(c["seed"])
    Ry = rng.standard_normal((wl.B, wl.T, wl.H, wl.d_v))
    RM = rng.standard_normal((wl.B, wl.H, wl.N, wl.d_v))
    L0, o0 = _loss(d, wl.sqrtN, wl.W, wl.R, Ry, RM)
    g = oracle.backward(d, wl.sqrtN, wl.W, wl.R, Ry, RM)
    names = {"kp": "dkp", "qp": "dqp", "v": "dv", "alpha": "dalpha", "beta": "dbeta",
             "M0": "dM0"}
    checked = 0
    for name, gname in names.items():
        x = d[name]
        flat = x.reshape(-1)
        for idx in rng.choice(flat.size, size=min(12, flat.size), replace=False):
            if x.dtype == np.uint16:  # bf16 inputs: step to the neighbouring bf16 values
                old = flat[idx]
                bf = lambda bits: float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])
                if bf(old) == 0.0 or (int(old) & 0x7FFF) in (0, 0x7FFF):
                    continue  # stay away from zero and the top of the range
                flat[idx] = old + 1; xp = bf(flat[idx]); Lp, op = _loss(d, wl.sqrtN, wl.W, wl.R, Ry, RM)
                flat[idx] = old - 1; xm = bf(flat[idx]); Lm, om = _loss(d, wl.sqrtN, wl.W, wl.R, Ry, RM)
                flat[idx] = old
            else:
                old = flat[idx]
                h = np.float32(2.0 ** -9 * max(1.0, abs(float(old))))
                flat[idx] = old + h; xp = float(flat[idx]); Lp, op = _loss(d, wl.sqrtN, wl.W, wl.R, Ry, RM)
                flat[idx] = old - h; xm = float(flat[idx]); Lm, om = _loss(d, wl.sqrtN, wl.W, wl.R, Ry, RM)
                flat[idx] = old
            if name in ("kp", "qp"):  # the selection must not move
                if not all((op[k] == o0[k]).all() and (om[k] == o0[k]).all() for k in ("Iw", "Ir")):
                    continue
            fd = (Lp - Lm) / (xp - xm)
            an = float(g[gname].reshape(-1)[idx])
            assert abs(fd - an) <= 2e-3 * (1.0 + abs(an)), (name, idx, fd, an)
            checked += 1
    assert checked >= 40


def test_backward_linear_pieces_are_exact():
    """Closed forms the backward must reproduce: with dMT only (dy = 0), the
    gradient reaching M_0 through never-written rows is dMT itself, summed
    over sequences; and beta = 0 makes v, beta-free paths vanish: dv = 0."""
    wl, d = _tiny(seed=55, S=8)
    d["kp"][..., :wl.sqrtN] = -8.0
    d["kp"][..., :2] = 8.0
    rng = np.random.default_rng(55)
    RM = rng.standard_normal((wl.B, wl.H, wl.N, wl.d_v))
    o = oracle.forward(d, wl.sqrtN, wl.W, wl.R)
    g = oracle.backward(d, wl.sqrtN, wl.W, wl.R, np.zeros((wl.B, wl.T, wl.H, wl.d_v)), RM)
    for h in range(wl.H):
        never = np.setdiff1d(np.arange(wl.N), np.unique(o["Iw"][:, :, h]))
        assert never.size > 0
        np.testing.assert_allclose(g["dM0"][h, never], RM[:, h, never].sum(0), rtol=1e-15)
    d2 = dict(d)
    d2["beta"] = np.zeros_like(d["beta"])
    g2 = oracle.backward(d2, wl.sqrtN, wl.W, wl.R, rng.standard_normal((wl.B, wl.T, wl.H, wl.d_v)), RM)
    assert (g2["dv"] == 0).all()
