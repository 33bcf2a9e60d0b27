"""Pins of the fp64 causal-conv1d oracle (no GPU needed).

The convolution ahead of the selective SSM in the Mamba block (a causal depthwise
1-D convolution, then SiLU) is fixed here against things other than the oracle
itself: numpy's convolution routine, scipy's logistic function, exact special
filters (identity, pure delay), splitting a sequence and carrying the state,
step-by-step decode, linearity and causality.  A plain Python copy of the window
loop with a planted slip (the filter read forwards, the window one step late, the
state taken newest first) must fail the same pins.
"""
import numpy as np
import pytest
import scipy.special
import torch

import gen
import oracle


def inputs(batch, dim, L, K, dtype="f32", seed=0, bias=True, state=False):
    g = np.random.default_rng(seed)
    x = gen.to_dtype(g.standard_normal((batch, dim, L), dtype=np.float32), dtype)
    w = torch.from_numpy(g.standard_normal((dim, K), dtype=np.float32) * 0.5)
    b = torch.from_numpy(g.standard_normal(dim, dtype=np.float32) * 0.1) if bias else None
    st = torch.from_numpy(g.standard_normal((batch, dim, K - 1), dtype=np.float32)) if state else None
    return x, w, b, st


def np64(t):
    return t.detach().float().numpy().astype(np.float64)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_matches_numpy_convolve(K):
    x, w, b, _ = inputs(2, 5, 40, K, seed=K)
    out, _ = oracle.conv1d(x, w, b, silu=False)
    xx, ww, bb = np64(x), np64(w), np64(b)
    for i in range(2):
        for d in range(5):
            # out_t = sum_k w[k] x[t-(K-1)+k]: a convolution with the filter reversed
            ref = np.convolve(xx[i, d], ww[d][::-1])[:40] + bb[d]
            assert np.max(np.abs(out[i, d] - ref)) <= 1e-13


def test_silu_matches_logistic():
    x, w, b, st = inputs(2, 6, 33, 4, seed=3, state=True)
    lin, _ = oracle.conv1d(x, w, b, silu=False, state=st)
    act, _ = oracle.conv1d(x, w, b, silu=True, state=st)
    assert np.max(np.abs(act - lin * scipy.special.expit(lin))) <= 1e-14


@pytest.mark.parametrize("K", [2, 4])
def test_identity_and_delay_filters_are_exact(K):
    x, _, _, st = inputs(1, 3, 17, K, seed=5, state=True)
    ident = torch.zeros(3, K)
    ident[:, K - 1] = 1.0
    out, so = oracle.conv1d(x, ident, None, silu=False, state=st)
    assert np.array_equal(out, np64(x))
    delay = torch.zeros(3, K)
    delay[:, 0] = 1.0
    out, _ = oracle.conv1d(x, delay, None, silu=False, state=st)
    full = np.concatenate([np64(st), np64(x)], axis=-1)  # inputs at steps -(K-1) .. L-1
    assert np.array_equal(out, full[..., :17])
    # the state out is the last K-1 inputs
    assert np.array_equal(so, np64(x)[..., 17 - (K - 1):])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_sequence_carries_state_exactly(dtype):
    x, w, b, st = inputs(2, 4, 50, 4, dtype=dtype, seed=7, state=True)
    whole, s_whole = oracle.conv1d(x, w, b, state=st)
    o1, s1 = oracle.conv1d(x[..., :21].contiguous(), w, b, state=st)
    o2, s2 = oracle.conv1d(x[..., 21:].contiguous(), w, b, state=torch.from_numpy(s1))
    assert np.array_equal(np.concatenate([o1, o2], axis=-1), whole)
    assert np.array_equal(s2, s_whole)


def test_decode_steps_equal_whole_sequence():
    x, w, b, st = inputs(3, 5, 12, 4, seed=9, state=True)
    whole, s_whole = oracle.conv1d(x, w, b, state=st)
    s = st
    for t in range(12):
        o, s_np = oracle.conv1d(x[..., t:t + 1].contiguous(), w, b, state=s)
        assert np.array_equal(o[..., 0], whole[..., t])
        s = torch.from_numpy(s_np)
    assert np.array_equal(s.numpy(), s_whole)


def test_short_sequence_state_mixes_old_state_and_inputs():
    x, w, b, st = inputs(1, 2, 2, 4, seed=11, state=True)  # L = 2 < K - 1 = 3
    _, so = oracle.conv1d(x, w, b, state=st)
    expect = np.concatenate([np64(st)[..., 2:], np64(x)], axis=-1)
    assert np.array_equal(so, expect)


def test_linearity_and_causality():
    x1, w, _, _ = inputs(1, 3, 30, 4, seed=13)
    x2, _, _, _ = inputs(1, 3, 30, 4, seed=14)
    # eighths: 0.5 * x1 - 2 * x2 is then exact in fp32, so the inputs carry no rounding
    x1, x2 = torch.round(x1 * 8) / 8, torch.round(x2 * 8) / 8
    o1, _ = oracle.conv1d(x1, w, None, silu=False)
    o2, _ = oracle.conv1d(x2, w, None, silu=False)
    o3, _ = oracle.conv1d(0.5 * x1 - 2.0 * x2, w, None, silu=False)
    assert np.max(np.abs(o3 - (0.5 * o1 - 2.0 * o2))) <= 1e-12
    x3 = x1.clone()
    x3[..., 20:] += 5.0
    o4, _ = oracle.conv1d(x3, w, None, silu=True)
    o5, _ = oracle.conv1d(x1, w, None, silu=True)
    assert np.array_equal(o4[..., :20], o5[..., :20]) and not np.array_equal(o4[..., 20:], o5[..., 20:])


def test_bf16_inputs_widen_exactly():
    x, w, b, _ = inputs(1, 4, 25, 3, dtype="bf16", seed=15)
    a, _ = oracle.conv1d(x, w, b)
    c, _ = oracle.conv1d(x.float(), w, b)
    assert np.array_equal(a, c)


# A Python copy of the window loop with one planted slip each: the pins above must reject it.
def python_conv(x, w, b, st, slip):
    X, W = np64(x), np64(w)
    B = np64(b) if b is not None else np.zeros(W.shape[0])
    S = np64(st)
    batch, dim, L = X.shape
    K = W.shape[1]
    out = np.zeros_like(X)
    for i in range(batch):
        for d in range(dim):
            hist = S[i, d][::-1] if slip == "state-newest-first" else S[i, d]
            full = np.concatenate([hist, X[i, d]])
            for t in range(L):
                win = full[t + (1 if slip == "window-late" else 0): t + K + (1 if slip == "window-late" else 0)]
                if slip == "window-late" and len(win) < K:
                    win = np.concatenate([win, np.zeros(K - len(win))])
                ww = W[d][::-1] if slip == "filter-forwards" else W[d]
                out[i, d, t] = B[d] + np.dot(ww, win)
    return out


@pytest.mark.parametrize("slip", ["none", "filter-forwards", "window-late", "state-newest-first"])
def test_planted_mistakes_are_caught(slip):
    x, w, b, st = inputs(1, 3, 20, 4, seed=17, state=True)
    ref, _ = oracle.conv1d(x, w, b, silu=False, state=st)
    got = python_conv(x, w, b, st, slip)
    err = np.max(np.abs(got - ref))
    if slip == "none":
        assert err <= 1e-12
    else:
        assert err > 1e-3, f"planted slip {slip} not caught"
