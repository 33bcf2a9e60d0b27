"""Pins of the SSD (Mamba-2, scalar decay per head) oracle, no GPU needed.

oracle.ssd runs the sequential recurrence with the per-head decay and step size
broadcast to the head's channels.  It is pinned here against the other side of the
duality the pages describe (mlqm.cn tutorial §8; AI inference series (14), the part on
how Mamba-2 reorganises the SSM into matrix computation: the selective scan equals a
multiplication by a lower-triangular semiseparable matrix): the
explicit matrix M[t, s] = (C_t . B_s) exp(A (cs_t - cs_s)) Delta_s, built with numpy
in fp64 and applied with a matmul; against the chunked evaluation the GPU kernels use
(intra-chunk masked matrix product, chunk states, state passing), at several chunk
lengths; and against the closed form for A = 0.  Planted slips in the chunked
evaluation must fail the same comparison.
"""
import numpy as np
import pytest
import torch

import gen
import oracle


def f64(t):
    return None if t is None else t.detach().float().numpy().astype(np.float64)


def steps(x, h):
    raw = f64(x["dt"])[:, h] + (0.0 if x["dt_bias"] is None else float(x["dt_bias"][h]))
    return np.logaddexp(0.0, raw) if x["softplus"] else raw


def gate(x, y, b, sl):
    X = f64(x["x"])[b, sl]
    if x["D"] is not None:
        y = y + f64(x["D"])[sl, None] * X
    if x["z"] is not None:
        zz = f64(x["z"])[b, sl]
        y = y * zz / (1.0 + np.exp(-zz))
    return y


def dense(x):
    """y = M x per (batch row, head) with the semiseparable matrix written out."""
    X, Bm, Cm, A = f64(x["x"]), f64(x["B"]), f64(x["C"]), f64(x["A"])
    batch, dim, L = X.shape
    P = x["headdim"]
    y = np.zeros_like(X)
    last = np.zeros((batch, dim, Bm.shape[1]))
    t_ge_s = np.tril(np.ones((L, L), dtype=bool))
    for b in range(batch):
        G = Cm[b].T @ Bm[b]                                   # G[t, s] = C_t . B_s
        for h in range(A.shape[0]):
            dl = steps(x, h)[b]
            cs = np.cumsum(dl)
            expo = np.where(t_ge_s, A[h] * (cs[:, None] - cs[None, :]), -np.inf)
            M = G * np.exp(expo) * dl[None, :]
            sl = slice(h * P, (h + 1) * P)
            y[b, sl] = gate(x, X[b, sl] @ M.T, b, sl)
            w = np.exp(A[h] * (cs[-1] - cs)) * dl                # weight of step s in the final state
            last[b, sl] = (X[b, sl] * w[None, :]) @ Bm[b].T     # [P, N]
    return y, last


def chunked(x, Q, slip=None):
    """The chunked evaluation: intra-chunk masked product, state passing between chunks."""
    X, Bm, Cm, A = f64(x["x"]), f64(x["B"]), f64(x["C"]), f64(x["A"])
    batch, dim, L = X.shape
    P, N = x["headdim"], Bm.shape[1]
    y = np.zeros_like(X)
    last = np.zeros((batch, dim, N))
    for b in range(batch):
        for h in range(A.shape[0]):
            dl = steps(x, h)[b]
            sl = slice(h * P, (h + 1) * P)
            H = np.zeros((N, P))
            for c0 in range(0, L, Q):
                c1 = min(c0 + Q, L)
                q = c1 - c0
                d = dl[c0:c1]
                cs = np.cumsum(d)
                if slip == "exclusive-decay":
                    cs = cs - d
                Bc, Cc, Xc = Bm[b][:, c0:c1], Cm[b][:, c0:c1], X[b, sl, c0:c1]
                lower = np.tril(np.ones((q, q), dtype=bool))
                expo = np.where(lower, A[h] * (cs[:, None] - cs[None, :]), -np.inf)
                M = (Cc.T @ Bc) * np.exp(expo) * d[None, :]
                Y = M @ Xc.T                                       # [q, P]
                if slip != "no-carry-in":
                    Y = Y + np.exp(A[h] * cs)[:, None] * (Cc.T @ H)
                w = np.exp(A[h] * (cs[-1] - cs)) * d
                decay = 1.0 if slip == "state-not-decayed" else np.exp(A[h] * cs[-1])
                H = decay * H + (Bc * w[None, :]) @ Xc.T          # [N, P]
                y[b, sl, c0:c1] = Y.T
            y[b, sl] = gate(x, y[b, sl], b, sl)
            last[b, sl] = H.T
    return y, last


def ref(x):
    return oracle.ssd(x["x"], x["dt"], x["A"], x["B"], x["C"], x["D"], x["z"], x["dt_bias"], x["softplus"],
                      headdim=x["headdim"])


def close(a, b, tol=1e-11):
    return np.max(np.abs(a - b)) <= tol * max(1.0, np.max(np.abs(b)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("opts", [{}, {"with_z": False, "with_D": False}, {"softplus": False, "with_bias": False}])
def test_equals_explicit_semiseparable_matrix(dtype, opts):
    x = gen.ssd_inputs(2, 3, 4, 5, 37, dtype, seed=1, **opts)
    if not x["softplus"]:
        x["dt"] = torch.abs(x["dt"])  # a nonnegative raw step keeps every decay factor <= 1
    y, last = ref(x)
    yd, ld = dense(x)
    assert close(y, yd) and close(last, ld)


@pytest.mark.parametrize("Q", [1, 5, 16, 64, 100])
def test_chunked_evaluation_equals_recurrence(Q):
    x = gen.ssd_inputs(1, 2, 8, 16, 100, "bf16", seed=2)
    y, last = ref(x)
    yc, lc = chunked(x, Q)
    assert close(y, yc) and close(last, lc)


def test_no_decay_is_a_running_sum():
    # A = 0: h_t = sum_{s<=t} Delta_s B_s x_s, so y_t = C_t . (cumulative sum), gated
    x = gen.ssd_inputs(1, 2, 3, 4, 30, "f32", seed=3, with_z=False, with_D=False)
    x["A"] = torch.zeros_like(x["A"])
    y, _ = ref(x)
    X, Bm, Cm = f64(x["x"]), f64(x["B"]), f64(x["C"])
    for h in range(2):
        dl = steps(x, h)[0]
        sl = slice(3 * h, 3 * h + 3)
        S = np.cumsum(dl[None, None, :] * Bm[0][:, None, :] * X[0, sl][None, :, :], axis=-1)  # [N, P, L]
        expect = np.einsum("nt,npt->pt", Cm[0], S)
        assert close(y[0, sl], expect)


@pytest.mark.parametrize("slip", ["exclusive-decay", "no-carry-in", "state-not-decayed"])
def test_planted_slips_are_caught(slip):
    x = gen.ssd_inputs(1, 2, 4, 8, 70, "f32", seed=4)
    y, last = ref(x)
    yc, lc = chunked(x, 16, slip=slip)
    assert not (close(y, yc, 1e-6) and close(last, lc, 1e-6)), slip
