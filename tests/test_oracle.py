"""Pins of the CPU fp64 oracle to things other than itself (no GPU needed).

Each test fixes the oracle against what the pages and the mathematics fix:
brute force at 30+ digits, closed forms, exact special cases and invariants.
Together they are chosen so that a plausible slip in the oracle -- a dropped
term, a wrong sign, Delta taken from the wrong step, B and C swapped, the gate
applied before the skip, a transposed index -- fails at least one of them
(``test_planted_mistakes_are_caught`` plants such slips in a Python copy of the
oracle loop and checks that these same pins reject them).
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import scipy.signal
import torch

import gen
import oracle


def _np(x):
    return None if x is None else x.detach().float().numpy().astype(np.float64)


def run(x, **kw):
    return oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x.get("D"), x.get("z"),
                       x.get("dt_bias"), x.get("softplus", True), **kw)


# ---------------------------------------------------------------------------
# P1: brute force.  The recurrence unrolled with the decay-product form
# dh_t/dh_s = prod_{r=s+1..t} Abar_r = exp(A * sum_{r=s+1..t} Delta_r)
# ("Mamba close reading", jsqmd.com, §6.1):
#   h_t[n] = sum_{s<=t} exp(A[d,n] * (S_t - S_s)) * Delta_s * B_s[n] * u_s,
# with S the running sum of Delta, evaluated in mpmath at 30 digits.
# ---------------------------------------------------------------------------
def brute_force(x, dps=30):
    mpmath.mp.dps = dps
    u, dl, z = _np(x["u"]), _np(x["delta"]), _np(x.get("z"))
    Bm, Cm, A = _np(x["B"]), _np(x["C"]), _np(x["A"])
    D = _np(x.get("D"))
    bias = _np(x.get("dt_bias"))
    sp = x.get("softplus", True)
    Bt, Dm, L = u.shape
    N = A.shape[1]
    y = np.zeros((Bt, Dm, L))
    last = np.zeros((Bt, Dm, N))
    for b in range(Bt):
        for d in range(Dm):
            dts = []
            for t in range(L):
                v = mpmath.mpf(dl[b, d, t]) + (mpmath.mpf(bias[d]) if bias is not None else 0)
                dts.append(mpmath.log(1 + mpmath.exp(v)) if sp else v)
            S = [mpmath.mpf(0)]
            for t in range(L):
                S.append(S[-1] + dts[t])   # S[t+1] = Delta_0 + ... + Delta_t
            for t in range(L):
                acc = mpmath.mpf(0)
                for n in range(N):
                    a = mpmath.mpf(A[d, n])
                    h = mpmath.fsum(mpmath.exp(a * (S[t + 1] - S[s + 1])) * dts[s] * mpmath.mpf(Bm[b, n, s])
                                    * mpmath.mpf(u[b, d, s]) for s in range(t + 1))
                    acc += mpmath.mpf(Cm[b, n, t]) * h
                    if t == L - 1:
                        last[b, d, n] = float(h)
                yt = acc + (mpmath.mpf(D[d]) * mpmath.mpf(u[b, d, t]) if D is not None else 0)
                if z is not None:
                    zz = mpmath.mpf(z[b, d, t])
                    yt *= zz / (1 + mpmath.exp(-zz))
                y[b, d, t] = float(yt)
    return y, last


def test_p1_brute_force_workload0():
    x = gen.scan_inputs(0)
    # 4 of the 16 channels keep the CPU suite fast; all indexing paths are exercised.
    sub = dict(x)
    for k in ("u", "delta", "z"):
        sub[k] = x[k][:, :4].contiguous()
    sub["A"], sub["D"], sub["dt_bias"] = x["A"][:4].contiguous(), x["D"][:4], x["dt_bias"][:4]
    y, last = run(sub)
    yb, lb = brute_force(sub)
    assert oracle.rel_err(y, yb) < 1e-13
    assert oracle.rel_err(last, lb) < 1e-13


@pytest.mark.parametrize("opts", [
    dict(),
    dict(with_D=False),
    dict(with_z=False),
    dict(with_bias=False),
    dict(softplus=False, delta_scale=0.5),
    dict(a_mode="random"),
])
def test_p1_brute_force_random_tiny(opts):
    o = dict(opts)
    sp = o.pop("softplus", True)
    x = gen.random_scan_inputs(2, 3, 3, 9, "f32", seed=1, softplus=sp, **o)
    if not sp:  # keep Delta > 0 without softplus
        x["delta"] = x["delta"].abs() + 0.01
    y, last = run(x)
    yb, lb = brute_force(x)
    assert oracle.rel_err(y, yb) < 1e-13
    assert oracle.rel_err(last, lb) < 1e-13


def test_p1_brute_force_bf16_inputs():
    x = gen.random_scan_inputs(1, 2, 4, 12, "bf16", seed=3)
    y, last = run(x)
    yb, lb = brute_force(x)  # brute force reads the same bf16 values, widened exactly
    assert oracle.rel_err(y, yb) < 1e-13
    assert oracle.rel_err(last, lb) < 1e-13


# ---------------------------------------------------------------------------
# P2: LTI closed form.  With Delta, B and C constant in t the system is time
# invariant and equals a causal convolution y = K * u (+ D u, gated) with
# K_k = sum_n C_n exp(k Delta A_n) Delta B_n (LTI = convolution: the
# tech.kj168168.com essay §二.1; mlqm.cn tutorial §3.3).
# ---------------------------------------------------------------------------
def lti_inputs(Bt, Dm, N, L, seed):
    g = np.random.default_rng(seed)
    u = g.standard_normal((Bt, Dm, L)).astype(np.float32)
    z = g.standard_normal((Bt, Dm, L)).astype(np.float32)
    dconst = (0.1 * g.standard_normal((Bt, Dm, 1))).astype(np.float32)
    delta = np.repeat(dconst, L, axis=2)
    Bc = g.standard_normal((Bt, N, 1)).astype(np.float32)
    Cc = g.standard_normal((Bt, N, 1)).astype(np.float32)
    x = dict(u=torch.from_numpy(u), z=torch.from_numpy(z), delta=torch.from_numpy(np.ascontiguousarray(delta)),
             B=torch.from_numpy(np.ascontiguousarray(np.repeat(Bc, L, axis=2))),
             C=torch.from_numpy(np.ascontiguousarray(np.repeat(Cc, L, axis=2))),
             A=torch.from_numpy(-np.exp(g.standard_normal((Dm, N))).astype(np.float32)),
             D=torch.from_numpy(g.standard_normal(Dm).astype(np.float32)),
             dt_bias=torch.from_numpy(np.log(np.expm1(np.exp(g.uniform(np.log(1e-3), np.log(1e-1), Dm))))
                                      .astype(np.float32)), softplus=True)
    return x


def test_p2_lti_convolution():
    x = lti_inputs(2, 3, 5, 80, seed=7)
    y, _ = run(x)
    u, z, A = _np(x["u"]), _np(x["z"]), _np(x["A"])
    Bc, Cc = _np(x["B"])[:, :, 0], _np(x["C"])[:, :, 0]
    dt = np.logaddexp(0.0, _np(x["delta"])[:, :, 0] + _np(x["dt_bias"])[None, :])  # softplus, fp64
    D = _np(x["D"])
    L = u.shape[2]
    k = np.arange(L)
    for b in range(u.shape[0]):
        for d in range(u.shape[1]):
            K = (Cc[b][None, :] * np.exp(k[:, None] * dt[b, d] * A[d][None, :]) * dt[b, d] * Bc[b][None, :]).sum(1)
            conv = np.array([np.dot(K[:t + 1], u[b, d, t::-1]) for t in range(L)])
            ref = (conv + D[d] * u[b, d]) * (z[b, d] / (1 + np.exp(-z[b, d])))
            assert oracle.rel_err(y[b, d], ref) < 1e-12


def test_p2_lti_lfilter_single_state():
    # N = 1, no D, no z: h is a first-order IIR filter of Delta*B*u
    x = lti_inputs(1, 2, 1, 200, seed=11)
    x["D"], x["z"] = None, None
    y, last = run(x)
    u, A = _np(x["u"]), _np(x["A"])
    Bc, Cc = _np(x["B"])[0, 0, 0], _np(x["C"])[0, 0, 0]
    dt = np.logaddexp(0.0, _np(x["delta"])[0, :, 0] + _np(x["dt_bias"]))
    for d in range(2):
        abar = np.exp(dt[d] * A[d, 0])
        h = scipy.signal.lfilter([dt[d] * Bc], [1.0, -abar], u[0, d])
        assert oracle.rel_err(y[0, d], Cc * h) < 1e-12
        assert abs(last[0, d, 0] - h[-1]) <= 1e-12 * abs(h).max()


# ---------------------------------------------------------------------------
# P3: Delta -> 0 leaves the state unchanged (small step = keep the state:
# junchaoiu.github.io summary, 方法 step 1; mlqm.cn tutorial §5.2).  Exact.
# ---------------------------------------------------------------------------
def test_p3_zero_step_keeps_state():
    x = gen.random_scan_inputs(2, 5, 4, 33, "f32", seed=4, softplus=False)
    x["delta"] = torch.zeros_like(x["delta"])
    x["dt_bias"] = None
    y, last = run(x)
    assert np.all(last == 0.0)
    u, z, D = _np(x["u"]), _np(x["z"]), _np(x["D"])
    ref = (D[None, :, None] * u) * (z / (1 + np.exp(-z)))
    assert oracle.rel_err(y, ref) < 1e-15
    # decode: bit-identical state
    s0 = torch.randn(2, 5, 4, dtype=torch.float64)
    st = gen.random_scan_inputs(2, 5, 4, 1, "f32", seed=5)
    yd, s1 = oracle.step(s0, st["u"][..., 0], torch.full((2, 5), -1e30), st["A"], st["B"][..., 0],
                         st["C"][..., 0], st["D"], st["z"][..., 0], None)
    # softplus(-1e30) = 0 exactly in fp64 -> Abar = 1, input term 0
    assert np.array_equal(s1, s0.numpy())


# ---------------------------------------------------------------------------
# P4: Delta -> infinity overwrites the state (large step = write the current
# token: mlqm.cn tutorial §5.2): y_t = Delta u_t sum_n C_t B_t + D u_t (gated).
# ---------------------------------------------------------------------------
def test_p4_large_step_is_memoryless():
    x = gen.random_scan_inputs(2, 3, 4, 20, "f32", seed=6, softplus=False)
    x["delta"] = torch.full_like(x["delta"], 60.0)
    x["dt_bias"] = None
    y, last = run(x)
    u, z, D = _np(x["u"]), _np(x["z"]), _np(x["D"])
    Bm, Cm = _np(x["B"]), _np(x["C"])
    cb = (Cm * Bm).sum(1)  # [B, L]
    ref = (60.0 * u * cb[:, None, :] + D[None, :, None] * u) * (z / (1 + np.exp(-z)))
    assert oracle.rel_err(y, ref) < 1e-15
    ref_last = 60.0 * Bm[:, None, :, -1] * u[:, :, -1:]
    assert oracle.rel_err(last, ref_last) < 1e-15


# ---------------------------------------------------------------------------
# P5: chunked two-level scan == sequential.  The recurrence is an associative
# scan over (a, b) pairs with (a1,b1) (+) (a2,b2) = (a1 a2, a2 b1 + b2)
# (tech.kj168168.com essay §二.3; "Mamba close reading" §2.2 and §7; mlqm.cn
# tutorial §6).  Chunk-local scans, a scan over chunk aggregates, then the
# carry-in fix-up -- in fp64 numpy -- must equal the sequential oracle.
# ---------------------------------------------------------------------------
def combine(p, q):
    return p[0] * q[0], q[0] * p[1] + q[1]


def chunked_scan(x, chunk):
    u, dl, z = _np(x["u"]), _np(x["delta"]), _np(x["z"])
    Bm, Cm, A, D, bias = _np(x["B"]), _np(x["C"]), _np(x["A"]), _np(x["D"]), _np(x["dt_bias"])
    dt = np.logaddexp(0.0, dl + bias[None, :, None])            # [B, D, L]
    a = np.exp(dt[..., None] * A[None, :, None, :])              # [B, D, L, N]
    bb = (dt * u)[..., None] * np.transpose(Bm, (0, 2, 1))[:, None]  # [B, D, L, N]
    Bt, Dm, L, N = a.shape
    h = np.empty_like(a)
    carry = (np.ones((Bt, Dm, N)), np.zeros((Bt, Dm, N)))        # identity element
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        # local inclusive prefix within the chunk
        pref = []
        acc = (a[:, :, c0], bb[:, :, c0])
        pref.append(acc)
        for t in range(c0 + 1, c1):
            acc = combine(acc, (a[:, :, t], bb[:, :, t]))
            pref.append(acc)
        for i, t in enumerate(range(c0, c1)):
            h[:, :, t] = combine(carry, pref[i])[1]
        carry = combine(carry, pref[-1])
    y = (h * np.transpose(Cm, (0, 2, 1))[:, None]).sum(-1) + D[None, :, None] * u
    y *= z / (1 + np.exp(-z))
    return y, h[:, :, -1]


@pytest.mark.parametrize("chunk", [1, 3, 7, 64, 128, 300])
def test_p5_chunked_equals_sequential(chunk):
    x = gen.random_scan_inputs(2, 3, 4, 300, "f32", seed=8)
    y, last = run(x)
    yc, lc = chunked_scan(x, chunk)
    assert oracle.rel_err(y, yc) < 1e-12
    assert oracle.rel_err(last, lc) < 1e-12


# ---------------------------------------------------------------------------
# P6: the combine operator is associative (exactly, in rationals).
# ---------------------------------------------------------------------------
def test_p6_combine_is_associative_exactly():
    g = np.random.default_rng(0)
    for _ in range(200):
        p, q, r = [(Fraction(int(g.integers(-50, 50)), int(g.integers(1, 20))),
                    Fraction(int(g.integers(-50, 50)), int(g.integers(1, 20)))) for _ in range(3)]
        assert combine(combine(p, q), r) == combine(p, combine(q, r))


# ---------------------------------------------------------------------------
# P7: step response.  Constant u, Delta, B, C from h_{-1} = 0 is a finite
# geometric series: h_t = Delta B u (1 - Abar^{t+1}) / (1 - Abar).
# ---------------------------------------------------------------------------
def test_p7_step_response():
    L, N = 50, 3
    u = torch.full((1, 2, L), 0.75)
    delta = torch.full((1, 2, L), 0.25)
    B = torch.tensor([0.5, -1.25, 2.0]).reshape(1, N, 1).repeat(1, 1, L).contiguous()
    C = torch.tensor([1.5, 0.25, -0.5]).reshape(1, N, 1).repeat(1, 1, L).contiguous()
    A = torch.tensor([[-1.0, -2.0, -0.5], [-3.0, -0.25, -1.5]])
    x = dict(u=u, delta=delta, A=A, B=B, C=C, D=None, z=None, dt_bias=None, softplus=False)
    y, last = run(x)
    t = np.arange(L)
    dt = 0.25
    for d in range(2):
        abar = np.exp(dt * A[d].double().numpy())
        h = dt * B[0, :, 0].double().numpy()[None] * 0.75 * (1 - abar[None] ** (t[:, None] + 1)) / (1 - abar[None])
        assert oracle.rel_err(y[0, d], h @ C[0, :, 0].double().numpy()) < 1e-13
        assert oracle.rel_err(last[0, d], h[-1]) < 1e-13


# ---------------------------------------------------------------------------
# P8: linearity in u for fixed Delta, B, C, z (the D*u skip included).
# Dyadic inputs keep 3*u1 - 2*u2 exact in fp32.
# ---------------------------------------------------------------------------
def test_p8_linearity_in_u():
    x = gen.random_scan_inputs(2, 4, 4, 40, "f32", seed=9)
    g = np.random.default_rng(1)
    u1 = torch.from_numpy((g.integers(-512, 512, x["u"].shape) / 256).astype(np.float32))
    u2 = torch.from_numpy((g.integers(-512, 512, x["u"].shape) / 256).astype(np.float32))
    ya, _ = run({**x, "u": u1})
    yb, _ = run({**x, "u": u2})
    yc, _ = run({**x, "u": 3 * u1 - 2 * u2})
    assert oracle.rel_err(yc, 3 * ya - 2 * yb) < 1e-12


# ---------------------------------------------------------------------------
# P9: causality -- a change at t0 leaves every y_t, t < t0, bit-identical.
# ---------------------------------------------------------------------------
def test_p9_causality():
    x = gen.random_scan_inputs(1, 3, 4, 64, "f32", seed=10)
    y, _ = run(x)
    t0 = 37
    x2 = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    for k in ("u", "delta", "z", "B", "C"):
        x2[k][..., t0:] += 1.0
    y2, _ = run(x2)
    assert np.array_equal(y[..., :t0], y2[..., :t0])
    assert not np.array_equal(y[..., t0:], y2[..., t0:])


# ---------------------------------------------------------------------------
# P10: equivariance -- permuting batch rows (with B, C) or channels (with
# A, D, dt_bias) permutes the outputs exactly.
# ---------------------------------------------------------------------------
def test_p10_permutation_equivariance():
    x = gen.random_scan_inputs(3, 5, 4, 30, "f32", seed=12)
    y, last = run(x)
    pb = torch.tensor([2, 0, 1])
    pd = torch.tensor([3, 1, 4, 0, 2])
    xb = dict(x)
    for k in ("u", "delta", "z", "B", "C"):
        xb[k] = x[k][pb].contiguous()
    yb, lb = run(xb)
    assert np.array_equal(yb, y[pb.numpy()]) and np.array_equal(lb, last[pb.numpy()])
    xd = dict(x)
    for k in ("u", "delta", "z"):
        xd[k] = x[k][:, pd].contiguous()
    xd["A"], xd["D"], xd["dt_bias"] = x["A"][pd].contiguous(), x["D"][pd], x["dt_bias"][pd]
    yd, ld = run(xd)
    assert np.array_equal(yd, y[:, pd.numpy()]) and np.array_equal(ld, last[:, pd.numpy()])


# ---------------------------------------------------------------------------
# P11: prefill -> decode hand-off.  scan(L) gives the state; k decode steps on
# the next inputs reproduce scan(L + k) ("AI inference series (14)",
# wiblog.cn: prefill writes the final state, decode updates it in place).
# Also: a scan resumed from a state equals the scan of the whole sequence.
# ---------------------------------------------------------------------------
def test_p11_prefill_then_decode():
    L, k = 40, 6
    x = gen.random_scan_inputs(2, 3, 4, L + k, "bf16", seed=13)
    y_all, last_all = run(x)
    pre = dict(x)
    for key in ("u", "delta", "z", "B", "C"):
        pre[key] = x[key][..., :L].contiguous()
    _, state = run(pre)
    for t in range(L, L + k):
        yt, state = oracle.step(state, x["u"][..., t].contiguous(), x["delta"][..., t].contiguous(), x["A"],
                                x["B"][..., t].contiguous(), x["C"][..., t].contiguous(), x["D"],
                                x["z"][..., t].contiguous(), x["dt_bias"])
        assert oracle.rel_err(yt, y_all[..., t]) < 1e-12
    assert oracle.rel_err(state, last_all) < 1e-12
    post = dict(x)
    for key in ("u", "delta", "z", "B", "C"):
        post[key] = x[key][..., L:].contiguous()
    _, pre_state = run(pre)
    y2, last2 = run(post, h0=pre_state)
    assert oracle.rel_err(y2, y_all[..., L:]) < 1e-12
    assert oracle.rel_err(last2, last_all) < 1e-12


def test_p11_channel_subset_matches_full():
    x = gen.random_scan_inputs(2, 5, 4, 25, "f32", seed=14)
    y, last = run(x)
    chans = [7, 0, 9, 3]
    ys, ls = run(x, chans=chans)
    assert np.array_equal(ys, y.reshape(10, 25)[chans]) and np.array_equal(ls, last.reshape(10, 4)[chans])


# ---------------------------------------------------------------------------
# P12: stability -- A = -exp(A_log) < 0 and Delta > 0 give 0 < Abar < 1 and
# |h| <= max|Delta B u| / (1 - max Abar) ("Mamba close reading" §4.1).
# ---------------------------------------------------------------------------
def test_p12_stability_bound():
    x = gen.random_scan_inputs(1, 4, 4, 500, "f32", seed=15)
    _, last = run(x)
    dt = np.logaddexp(0.0, _np(x["delta"]) + _np(x["dt_bias"])[None, :, None])
    A = _np(x["A"])
    abar = np.exp(dt[..., None] * A[None, :, None, :])
    assert np.all(abar > 0) and np.all(abar < 1)
    bmax = np.abs(dt * _np(x["u"])).max(-1)[..., None] * np.abs(_np(x["B"])).max(-1)[:, None, :]
    bound = bmax / (1 - abar.max(2))
    assert np.all(np.abs(last) <= bound)


def test_empty_sequence():
    x = gen.random_scan_inputs(1, 2, 4, 0, "f32", seed=0)
    y, last = run(x)
    assert y.shape == (1, 2, 0) and np.all(last == 0)


def test_thread_count_does_not_change_result():
    x = gen.random_scan_inputs(2, 8, 4, 50, "bf16", seed=16)
    y1, l1 = run(x, threads=1)
    y4, l4 = run(x, threads=4)
    assert np.array_equal(y1, y4) and np.array_equal(l1, l4)


# ---------------------------------------------------------------------------
# Planted mistakes: a Python transcription of the oracle loop with one slip
# each must fail the pins above (brute force / closed forms).  This shows the
# pins can catch the plausible mistakes, not only that the oracle passes them.
# ---------------------------------------------------------------------------
def python_scan(x, slip=None):
    u, dl, z = _np(x["u"]), _np(x["delta"]), _np(x["z"])
    Bm, Cm, A, D, bias = _np(x["B"]), _np(x["C"]), _np(x["A"]), _np(x["D"]), _np(x["dt_bias"])
    Bt, Dm, L = u.shape
    N = A.shape[1]
    y = np.zeros((Bt, Dm, L))
    for b in range(Bt):
        for d in range(Dm):
            h = np.zeros(N)
            for t in range(L):
                xx = dl[b, d, t] + bias[d]
                dt = np.logaddexp(0.0, xx)
                tb = t - 1 if (slip == "delta_prev_step" and t > 0) else t
                dtb = np.logaddexp(0.0, dl[b, d, tb] + bias[d])
                abar = np.exp(dt * A[d]) if slip != "sign_A" else np.exp(-dt * A[d])
                Bv, Cv = (Cm[b, :, t], Bm[b, :, t]) if slip == "swap_BC" else (Bm[b, :, t], Cm[b, :, t])
                inp = dtb * Bv * u[b, d, t] if slip != "drop_delta_in_input" else Bv * u[b, d, t]
                h = abar * h + inp
                acc = Cv @ h
                zz = z[b, d, t]
                g = zz / (1 + np.exp(-zz))
                if slip == "gate_before_skip":
                    y[b, d, t] = acc * g + D[d] * u[b, d, t]
                elif slip == "drop_skip":
                    y[b, d, t] = acc * g
                else:
                    y[b, d, t] = (acc + D[d] * u[b, d, t]) * g
    return y


@pytest.mark.parametrize("slip", [None, "delta_prev_step", "sign_A", "swap_BC", "drop_delta_in_input",
                                  "gate_before_skip", "drop_skip"])
def test_planted_mistakes_are_caught(slip):
    x = gen.random_scan_inputs(1, 2, 3, 8, "f32", seed=2)
    yb, _ = brute_force(x)
    err = oracle.rel_err(python_scan(x, slip), yb)
    if slip is None:
        assert err < 1e-12
    else:
        assert err > 1e-6, f"pin did not catch planted slip {slip}"


def test_golden_workload0_regression():
    """Stored oracle outputs of the tiny workload (tests/golden/make_golden.py)."""
    import os
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_golden
    lines = open(make_golden.OUT).read().splitlines()
    x = gen.scan_inputs(0)
    assert lines[1] == "input_sha256 " + make_golden.input_digest(x)
    ys = np.array([float(l.split()[1]) for l in lines if l.startswith("y ")])
    ls = np.array([float(l.split()[1]) for l in lines if l.startswith("last ")])
    y, last = run(x)
    assert np.array_equal(y.ravel(), ys) and np.array_equal(last.ravel(), ls)
