"""GPU backward of the core (sdm_backward) against the float64 oracle's
backward (itself pinned by finite differences on the CPU)."""
import numpy as np
import pytest
import torch

import oracle
import sdm_inputs as si
import sparse_memory_linear_select_amd as sdm
from gpu_util import Timer, log, make_core, upload

pytestmark = pytest.mark.gpu

# max |gpu - ref| <= GTOL * (1 + |ref|) elementwise.  The GPU accumulates in
# float32 what the oracle accumulates in float64: the adjoint of a row sums
# q*dy over every later read of the slot (contracted by each write), and the
# weight gradients are dot products over d_v columns followed by the softmax
# backward w (dw - <w, dw>), whose cancellation turns the float32 rounding of
# dw (~ sqrt(d_v) * 2^-24 * |G| |row|, |G| ~ a few units here) into an
# absolute error of ~1e-6.  Observed at most 1.7e-6 (the 1.4B-style layer).
GTOL = 1e-4
NAMES = ("dkp", "dqp", "dv", "dalpha", "dbeta", "dMinit", "dM0")


def _grads(wl, d, seed, with_dMT=True):
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((wl.B, wl.T, wl.H, wl.d_v)).astype(np.float32)
    dMT = rng.standard_normal((wl.B, wl.H, wl.N, wl.d_v)).astype(np.float32) if with_dMT else None
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    g = core.backward(*args, torch.from_numpy(dy).cuda(),
                      dMT=None if dMT is None else torch.from_numpy(dMT).cuda())
    torch.cuda.synchronize()
    ref = oracle.backward(d, wl.sqrtN, wl.W, wl.R, dy.astype(np.float64),
                          None if dMT is None else dMT.astype(np.float64))
    ref["dMinit"] = None
    return core, dd, args, g, dy, dMT, ref


def _compare(g, ref, names=NAMES):
    worst = {}
    for n in names:
        if ref.get(n) is None:
            continue
        got = g[n].cpu().numpy().astype(np.float64)
        r = ref[n]
        assert np.isfinite(got).all(), n
        err = float((np.abs(got - r) / (1.0 + np.abs(r))).max()) if r.size else 0.0
        worst[n] = err
        assert err <= GTOL, f"{n}: max |err|/(1+|ref|) = {err:.3e}"
    log("  max rel err " + "  ".join(f"{k} {v:.1e}" for k, v in worst.items()))


SHAPES = [
    # (B, T, H, sqrtN, d_v, W, R, dtype, reuse)
    (1, 64, 1, 16, 32, 4, 4, "f32", 0.0),
    (1, 1, 1, 1, 4, 1, 1, "f32", 0.0),          # N = 1, single token
    (2, 200, 2, 16, 48, 16, 16, "f32", 0.0),    # 13 epochs
    (1, 257, 2, 64, 64, 32, 32, "f32", 0.3),    # key reuse
    (2, 91, 1, 32, 36, 32, 20, "bf16", 0.5),    # bf16 inputs, W != R, ragged slice
    (3, 50, 1, 9, 8, 9, 9, "f32", 0.0),         # every token writes 9 of 81 slots
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:7]) for s in SHAPES])
def test_backward_shapes(shape):
    B, T, H, S, D, W, R, dt, reuse = shape
    wl = si.Workload("bwd", B=B, T=T, H=H, sqrtN=S, d_v=D, W=W, R=R, dtype=dt, reuse=reuse,
                     seed=900 + T)
    log(f"backward: B={B} T={T} H={H} S={S} d_v={D} W={W} R={R} {dt}")
    d = si.generate(wl)
    core, dd, args, g, dy, dMT, ref = _grads(wl, d, seed=T)
    # dMinit summed over sequences is dM0; per sequence it is the oracle's
    # dM0 of that sequence alone
    assert torch.allclose(g["dMinit"].sum(0), g["dM0"], rtol=1e-6, atol=1e-6)
    _compare(g, ref)


def test_backward_without_dMT_and_per_sequence_initial_state():
    """dMT = None means zero; dMinit of each sequence equals the oracle's dM0
    of that sequence run alone."""
    wl = si.Workload("bwd2", B=2, T=120, H=2, sqrtN=16, d_v=32, W=8, R=8, dtype="f32",
                     reuse=0.0, seed=77)
    d = si.generate(wl)
    core, dd, args, g, dy, dMT, ref = _grads(wl, d, seed=5, with_dMT=False)
    _compare(g, ref)
    for b in range(wl.B):
        sub = {k: (v[b:b + 1] if k != "M0" else v) for k, v in d.items() if k != "src"}
        rb = oracle.backward(sub, wl.sqrtN, wl.W, wl.R, dy[b:b + 1].astype(np.float64))
        got = g["dMinit"][b].cpu().numpy().astype(np.float64)
        assert (np.abs(got - rb["dM0"]) / (1 + np.abs(rb["dM0"]))).max() <= GTOL


def test_backward_from_a_continued_state():
    """Minit: the forward starts from a given state (a continuation).  Split a
    sequence in two: the backward of the second half from the state the first
    half left, chained into the backward of the first half (its dMT = the
    second half's dMinit), gives the gradients of the whole sequence."""
    wl = si.Workload("bwd3", B=1, T=150, H=2, sqrtN=16, d_v=32, W=8, R=8, dtype="f32",
                     reuse=0.0, seed=78)
    d = si.generate(wl)
    rng = np.random.default_rng(6)
    dy = torch.from_numpy(rng.standard_normal((wl.B, wl.T, wl.H, wl.d_v)).astype(np.float32)).cuda()
    dMT = torch.from_numpy(rng.standard_normal((wl.B, wl.H, wl.N, wl.d_v)).astype(np.float32)).cuda()
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    whole = core.backward(*args, dy, dMT=dMT)
    k = 70
    first = [a[:, :k].contiguous() for a in args]
    second = [a[:, k:].contiguous() for a in args]
    _, Mk = core.forward(*first)
    g2 = core.backward(*second, dy[:, k:].contiguous(), dMT=dMT, Minit=Mk)
    g1 = core.backward(*first, dy[:, :k].contiguous(), dMT=g2["dMinit"])
    torch.cuda.synchronize()
    for n in ("dkp", "dqp", "dv", "dalpha", "dbeta"):
        cat = torch.cat([g1[n], g2[n]], 1)
        assert torch.allclose(cat, whole[n], rtol=1e-4, atol=1e-4), n
    assert torch.allclose(g1["dMinit"], whole["dMinit"], rtol=1e-4, atol=1e-4)


def test_backward_is_deterministic():
    wl = si.Workload("bwd4", B=2, T=300, H=2, sqrtN=32, d_v=64, W=16, R=16, dtype="f32",
                     reuse=0.2, seed=79)
    d = si.generate(wl)
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    dy = torch.randn((wl.B, wl.T, wl.H, wl.d_v), device="cuda")
    g1 = core.backward(*args, dy)
    g2 = core.backward(*args, dy)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n


def test_backward_full_workload():
    """The 1.4B-style layer at full size, every gradient against the oracle."""
    wl = si.WORKLOADS[1]
    with Timer("generate"):
        d = si.generate(wl)
    with Timer("gpu + oracle backward"):
        core, dd, args, g, dy, dMT, ref = _grads(wl, d, seed=11)
        _compare(g, ref)


def _dy_dMT(wl, seed):
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((wl.B, wl.T, wl.H, wl.d_v)).astype(np.float32)
    dMT = rng.standard_normal((wl.B, wl.H, wl.N, wl.d_v)).astype(np.float32)
    return dy, dMT


def test_backward_chunk_counts_agree_bitwise():
    """The backward takes the tokens in chunks of whole epochs (the tape holds
    one chunk; each chunk's forward runs again from its start state).  The
    least-memory workspace (several chunks) and the whole-sequence workspace
    (one chunk) give the same gradients bit for bit, and both match the
    oracle."""
    wl = si.Workload("bwd chunks", B=2, T=1200, H=2, sqrtN=16, d_v=32, W=8, R=8, dtype="f32",
                     reuse=0.2, seed=81)
    d = si.generate(wl)
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R)
    n_min = core.backward_workspace_size(wl.B, wl.T, sdm.F32, 0)
    n_one = core.backward_workspace_size(wl.B, wl.T, sdm.F32, 1)
    log(f"backward workspace: least {n_min} B, one chunk {n_one} B")
    assert n_min < n_one
    dy, dMT = _dy_dMT(wl, 12)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    dyg, dMTg = torch.from_numpy(dy).cuda(), torch.from_numpy(dMT).cuda()
    g_min = core.backward(*args, dyg, dMT=dMTg, chunks=0)
    g_one = core.backward(*args, dyg, dMT=dMTg, chunks=1)
    torch.cuda.synchronize()
    for n in g_min:
        assert torch.equal(g_min[n], g_one[n]), n
    ref = oracle.backward(d, wl.sqrtN, wl.W, wl.R, dy.astype(np.float64), dMT.astype(np.float64))
    ref["dMinit"] = None
    _compare(g_min, ref)


def test_backward_8b_style_shape_in_chunks():
    """The 8B-style layer's head shape (sqrtN = 256, d_v = 1024, W = R = 64;
    epochs of 1024 tokens, whose reads take the sampled link search in the
    forward) over 4 epochs, in the least memory (two chunks), against the
    oracle."""
    wl = si.Workload("bwd 8B-style", B=1, T=4096, H=2, sqrtN=256, d_v=1024, W=64, R=64,
                     dtype="f32", reuse=0.1, seed=82)
    log(f"backward: B={wl.B} T={wl.T} H={wl.H} S={wl.sqrtN} d_v={wl.d_v} W={wl.W} R={wl.R}")
    with Timer("generate"):
        d = si.generate(wl)
    with Timer("gpu + oracle backward"):
        core, dd, args, g, dy, dMT, ref = _grads(wl, d, seed=13)
        assert core.backward_workspace_size(wl.B, wl.T, sdm.F32, 0) < \
            core.backward_workspace_size(wl.B, wl.T, sdm.F32, 1)
        _compare(g, ref)


def test_backward_long_context_epochs_in_chunks():
    """The long-context slot count (sqrtN = 512, W = R = 64: epochs of 4096
    tokens) over three epochs, bf16 inputs and key reuse, on 64 columns
    (columns never interact, so the state's width does not change the
    schedule).  The backward in three chunks of one epoch and in one chunk
    gives the same gradients bit for bit, and both match the oracle."""
    wl = si.Workload("bwd long epochs", B=1, T=9000, H=1, sqrtN=512, d_v=64, W=64, R=64,
                     dtype="bf16", reuse=0.1, seed=84)
    log(f"backward: B={wl.B} T={wl.T} H={wl.H} S={wl.sqrtN} d_v={wl.d_v} bf16, 1 and 3 chunks")
    with Timer("generate"):
        d = si.generate(wl)
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R)
    # (here E*W = N: one epoch of the tape is the size of one chunk-start
    # state, so three chunks take as much memory as one)
    dy, dMT = _dy_dMT(wl, 15)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    dyg, dMTg = torch.from_numpy(dy).cuda(), torch.from_numpy(dMT).cuda()
    g3 = core.backward(*args, dyg, dMT=dMTg, chunks=3)
    g1 = core.backward(*args, dyg, dMT=dMTg, chunks=1)
    torch.cuda.synchronize()
    for n in g3:
        assert torch.equal(g3[n], g1[n]), n
    with Timer("oracle backward"):
        ref = oracle.backward(d, wl.sqrtN, wl.W, wl.R, dy.astype(np.float64),
                              dMT.astype(np.float64))
    ref["dMinit"] = None
    _compare(g3, ref)


def test_backward_long_context_shape_chained_calls():
    """The long-context head shape (sqrtN = 512, d_v = 2048, W = R = 64, bf16
    inputs, key reuse) run as three calls that continue the state (the
    chunking a caller does across calls): forwards to get each call's start
    state, then the backwards in reverse, each fed the next one's dMinit as
    dMT.  The concatenated gradients match the oracle's backward of the whole
    sequence."""
    wl = si.Workload("bwd long", B=1, T=600, H=1, sqrtN=512, d_v=2048, W=64, R=64,
                     dtype="bf16", reuse=0.1, seed=83)
    log(f"backward: B={wl.B} T={wl.T} H={wl.H} S={wl.sqrtN} d_v={wl.d_v} bf16, 3 calls")
    d = si.generate(wl)
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R)
    dy, dMT = _dy_dMT(wl, 14)
    dyg, dMTg = torch.from_numpy(dy).cuda(), torch.from_numpy(dMT).cuda()
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    cuts = [0, 200, 400, 600]
    part = lambda x, i: x[:, cuts[i]:cuts[i + 1]].contiguous()
    starts = [None]
    M = None
    for i in range(2):  # start states of calls 1 and 2
        _, M = core.forward(*[part(a, i) for a in args], M=None if M is None else M.clone(),
                            cont=M is not None)
        starts.append(M.clone())
    grads = [None] * 3
    upstream = dMTg
    for i in (2, 1, 0):
        grads[i] = core.backward(*[part(a, i) for a in args], part(dyg, i), dMT=upstream,
                                 Minit=starts[i])
        upstream = grads[i]["dMinit"]
    torch.cuda.synchronize()
    got = {n: torch.cat([grads[i][n] for i in range(3)], 1) for n in
           ("dkp", "dqp", "dv", "dalpha", "dbeta")}
    got["dM0"] = grads[0]["dMinit"][0]
    with Timer("oracle backward"):
        ref = oracle.backward(d, wl.sqrtN, wl.W, wl.R, dy.astype(np.float64),
                              dMT.astype(np.float64))
    _compare(got, ref, names=("dkp", "dqp", "dv", "dalpha", "dbeta", "dM0"))


def test_backward_rejects_bf16_state():
    wl = si.Workload("bwd5", B=1, T=8, H=1, sqrtN=8, d_v=8, W=4, R=4, dtype="f32", reuse=0.0,
                     seed=80)
    d = si.generate(wl)
    dd = upload(d)
    core = make_core(dd, wl.W, wl.R, torch.bfloat16)
    args = [dd[n] for n in ("kp", "qp", "v", "alpha", "beta")]
    with pytest.raises(sdm.SDMError) as e:
        core.backward(*args, torch.zeros((1, 8, 1, 8), device="cuda"))
    assert e.value.status == 2
