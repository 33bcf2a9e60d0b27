"""Pins of the fp64 backward oracle (no GPU needed).

The gradients of L = sum(dy * y) that oracle.scan_bwd returns are fixed against
(1) central finite differences of the pinned forward oracle, entry by entry, for
every input; (2) torch.autograd through an independent float64 forward written
with tensor operations; (3) exact special cases and invariants (dy = 0, no input
path, linearity in dy, thread count).  Planted slips in a copy of the adjoint
loop (the adjoint carried without its transition, the step size of the wrong
step) must fail the same pins.
"""
import numpy as np
import pytest
import torch

import gen
import oracle


def small(seed=0, batch=1, dim=3, N=4, L=12, dtype="f32", **kw):
    x = gen.random_scan_inputs(batch, dim, N, L, dtype, seed=seed, **kw)
    g = np.random.default_rng(100 + seed)
    dy = gen.to_dtype(g.standard_normal((batch, dim, L), dtype=np.float32), dtype)
    h0 = torch.from_numpy(g.standard_normal((batch, dim, N), dtype=np.float32) * 0.5)
    return x, dy, h0


def fwd_loss(x, dy, h0):
    y, _ = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x.get("D"), x.get("z"), x.get("dt_bias"),
                       x.get("softplus", True), h0=h0)
    return float(np.sum(y * dy.double().numpy()))


def bwd(x, dy, h0, **kw):
    return oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x.get("D"), x.get("z"), x.get("dt_bias"),
                           x.get("softplus", True), h0=h0, dy=dy, **kw)


# ---------------------------------------------------------------- finite differences
H = 2.0 ** -10  # exact in fp32 for the |values| < 2 perturbed here


def perturbed(x, h0, key, idx, step):
    x2 = dict(x)
    if key == "h0":
        t = h0.clone()
        t.view(-1)[idx] += step
        return x2, t
    t = x[key].clone()
    t.view(-1)[idx] += step
    x2[key] = t
    return x2, h0


GRAD_OF = {"u": "du", "delta": "ddelta", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "D": "dD",
           "dt_bias": "ddt_bias", "h0": "dh0"}


@pytest.mark.parametrize("key", list(GRAD_OF))
def test_gradients_match_central_differences(key):
    x, dy, h0 = small(seed=3)
    g = bwd(x, dy, h0)[GRAD_OF[key]]
    flat = g.reshape(-1)
    scale = max(1e-3, float(np.max(np.abs(flat))))
    rng = np.random.default_rng(7)
    for idx in rng.choice(flat.size, size=min(6, flat.size), replace=False):
        xp, hp = perturbed(x, h0, key, int(idx), H)
        xm, hm = perturbed(x, h0, key, int(idx), -H)
        fd = (fwd_loss(xp, dy, hp) - fwd_loss(xm, dy, hm)) / (2 * H)
        assert abs(fd - flat[idx]) <= 2e-4 * scale, (key, idx, fd, flat[idx])


# ---------------------------------------------------------------- autograd of a separate forward
def torch_forward(x, h0):
    """The forward recurrence with float64 tensor operations (one step per iteration, all
    channels at once), differentiable by torch.autograd."""
    u, dl, z = (x[k].double() for k in ("u", "delta", "z"))
    A, B, C = x["A"].double(), x["B"].double(), x["C"].double()
    D, bias = x["D"].double(), x["dt_bias"].double()
    h = h0.double()
    ys = []
    for t in range(u.shape[-1]):
        dt = torch.nn.functional.softplus(dl[..., t] + bias)                 # [B, D]
        h = torch.exp(dt[..., None] * A) * h + (dt * u[..., t])[..., None] * B[:, None, :, t]
        s = (C[:, None, :, t] * h).sum(-1) + D * u[..., t]
        ys.append(s * torch.nn.functional.silu(z[..., t]))
    return torch.stack(ys, dim=-1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gradients_match_autograd(dtype):
    x, dy, h0 = small(seed=5, batch=2, dim=5, N=4, L=20, dtype=dtype)
    leaves = {k: x[k].double().clone().requires_grad_(True) for k in ("u", "delta", "z", "A", "B", "C", "D",
                                                                      "dt_bias")}
    h0l = h0.double().clone().requires_grad_(True)
    y = torch_forward(leaves, h0l)
    loss = (y * dy.double()).sum()
    grads = torch.autograd.grad(loss, [*leaves.values(), h0l])
    got = bwd(x, dy, h0)
    for (k, _), ga in zip(list(leaves.items()) + [("h0", None)], grads):
        ref = ga.numpy()
        err = np.max(np.abs(got[GRAD_OF[k]] - ref)) / max(1e-12, np.max(np.abs(ref)))
        assert err <= 1e-10, (k, err)


# ---------------------------------------------------------------- special cases and invariants
def test_zero_upstream_gives_zero_gradients():
    x, dy, h0 = small(seed=8)
    g = bwd(x, torch.zeros_like(dy), h0)
    for k, v in g.items():
        assert v is None or not np.any(v), k


def test_without_input_path_only_the_skip_remains():
    # B = 0 and h0 = 0 keep every state at 0: y = D u silu(z); dC = dA = ddelta = 0 (the
    # adjoint itself, and so dh0, is not zero: C still reads the state)
    x, dy, h0 = small(seed=9)
    x["B"] = torch.zeros_like(x["B"])
    g = bwd(x, dy, torch.zeros_like(h0))
    u, z, D = (x[k].double().numpy() for k in ("u", "z", "D"))
    sil = z / (1 + np.exp(-z))
    ds = dy.double().numpy() * sil
    assert not np.any(g["dC"]) and not np.any(g["dA"]) and not np.any(g["ddelta"])
    assert np.any(g["dh0"])
    assert np.max(np.abs(g["du"] - ds * D[None, :, None])) <= 1e-14
    assert np.max(np.abs(g["dD"] - (ds * u).sum(axis=(0, 2)))) <= 1e-13


def test_linear_in_upstream_gradient():
    x, dy, h0 = small(seed=10)
    # eighths: 0.5 * dy - 2 * dy2 is exact in fp32, so the combined upstream carries no rounding
    dy = torch.round(dy * 8) / 8
    dy2 = torch.flip(dy, dims=[-1]).contiguous()
    g1, g2 = bwd(x, dy, h0), bwd(x, dy2, h0)
    g3 = bwd(x, (0.5 * dy - 2.0 * dy2).contiguous(), h0)
    for k in g1:
        if g1[k] is None:
            continue
        ref = 0.5 * g1[k] - 2.0 * g2[k]
        assert np.max(np.abs(g3[k] - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref))), k


def test_thread_count_does_not_change_gradients():
    x, dy, h0 = small(seed=11, batch=3, dim=7, N=8, L=40)
    a, b = bwd(x, dy, h0, threads=1), bwd(x, dy, h0, threads=5)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


# ---------------------------------------------------------------- planted slips
def python_bwd_du(x, dy, h0, slip):
    """du by the adjoint, in plain Python, with one planted slip."""
    u, dl, z = (x[k].double().numpy() for k in ("u", "delta", "z"))
    A, B, C = (x[k].double().numpy() for k in ("A", "B", "C"))
    D, bias = x["D"].double().numpy(), x["dt_bias"].double().numpy()
    dyv = dy.double().numpy()
    batch, dim, L = u.shape
    N = A.shape[1]
    du = np.zeros_like(u)
    for b in range(batch):
        for d in range(dim):
            dt = np.log1p(np.exp(dl[b, d] + bias[d]))
            lam = np.zeros(N)
            for t in range(L - 1, -1, -1):
                g = z[b, d, t] / (1 + np.exp(-z[b, d, t]))
                ds = dyv[b, d, t] * g
                lam = ds * C[b, :, t] + lam
                step = dt[t - 1] if (slip == "wrong-step" and t > 0) else dt[t]
                du[b, d, t] = ds * D[d] + np.sum(lam * step * B[b, :, t])
                if slip != "no-transition":
                    lam = lam * np.exp(dt[t] * A[d])
    return du


@pytest.mark.parametrize("slip", ["none", "no-transition", "wrong-step"])
def test_planted_slips_are_caught(slip):
    x, dy, h0 = small(seed=12)
    ref = bwd(x, dy, h0)["du"]
    got = python_bwd_du(x, dy, h0, slip)
    err = np.max(np.abs(got - ref))
    if slip == "none":
        assert err <= 1e-12
    else:
        assert err > 1e-6, f"slip {slip} not caught"
