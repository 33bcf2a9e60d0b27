"""Pins of the SSD backward oracle (no GPU needed).

oracle.ssd_bwd gives the gradients of L = sum(dy * y) for the SSD forward oracle.ssd (Mamba-2
form: one decay rate and one step size per head; mlqm.cn tutorial §8).  They are fixed here
against central finite differences of oracle.ssd itself, entry by entry, for every input: the
per-head step sizes dt, the per-head decay A and dt_bias, whose gradients gather the whole head's
channels (and for A every state), and the per-channel x, z, D, B, C and initial state.  A planted
slip (the head sums taken over the wrong axis) must fail the same pin.
"""
import numpy as np
import pytest
import torch

import gen
import oracle

H = 2.0 ** -10  # exact in fp32 for the |values| < 2 perturbed here


def small(seed=0, heads=2, headdim=3, N=4, L=10):
    x = gen.ssd_inputs(1, heads, headdim, N, L, "f32", seed=seed)
    g = np.random.default_rng(300 + seed)
    dy = gen.to_dtype(g.standard_normal((1, heads * headdim, L), dtype=np.float32), "f32")
    h0 = torch.from_numpy(g.standard_normal((1, heads * headdim, N), dtype=np.float32) * 0.5)
    return x, dy, h0


def loss(x, dy, h0):
    y, _ = oracle.ssd(x["x"], x["dt"], x["A"], x["B"], x["C"], x["D"], x["z"], x["dt_bias"], x["softplus"],
                      headdim=x["headdim"], h0=h0)
    return float(np.sum(y * dy.double().numpy()))


def grads(x, dy, h0):
    return oracle.ssd_bwd(x["x"], x["dt"], x["A"], x["B"], x["C"], x["D"], x["z"], x["dt_bias"], x["softplus"],
                          headdim=x["headdim"], h0=h0, dy=dy)


GRAD_OF = {"x": "dx", "dt": "ddt", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "D": "dD", "dt_bias": "ddt_bias",
           "h0": "dh0"}


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


def central(x, dy, h0, key, idx):
    xp, hp = perturbed(x, h0, key, idx, H)
    xm, hm = perturbed(x, h0, key, idx, -H)
    return (loss(xp, dy, hp) - loss(xm, dy, hm)) / (2 * H)


@pytest.mark.parametrize("key", list(GRAD_OF))
def test_ssd_gradients_match_central_differences(key):
    x, dy, h0 = small(seed=5)
    g = grads(x, dy, h0)[GRAD_OF[key]]
    flat = np.asarray(g).reshape(-1)
    scale = max(1e-3, float(np.max(np.abs(flat))))
    rng = np.random.default_rng(11)
    for idx in rng.choice(flat.size, size=min(6, flat.size), replace=False):
        fd = central(x, dy, h0, key, int(idx))
        assert abs(fd - flat[idx]) <= 2e-4 * scale, (key, idx, fd, flat[idx])


def test_ssd_gradients_without_softplus_bias_or_gate():
    x = gen.ssd_inputs(1, 2, 2, 3, 8, "f32", seed=6, with_D=False, with_z=False, with_bias=False, softplus=False)
    x["dt"] = (x["dt"].abs() * 0.5 + 0.05).contiguous()  # positive steps without softplus
    g = np.random.default_rng(6)
    dy = gen.to_dtype(g.standard_normal((1, 4, 8), dtype=np.float32), "f32")
    out = grads(x, dy, None)
    assert out["dz"] is None and out["dD"] is None and out["ddt_bias"] is None
    for key in ("dt", "A", "x"):
        flat = np.asarray(out[GRAD_OF[key]]).reshape(-1)
        scale = max(1e-3, float(np.max(np.abs(flat))))
        for idx in range(min(4, flat.size)):
            assert abs(central(x, dy, None, key, idx) - flat[idx]) <= 2e-4 * scale, (key, idx)


def test_planted_head_sum_slip_fails_the_pin():
    """Summing the channel gradients of dt over the wrong axis (the state axis of dA's layout
    instead of the head's channels) gives numbers the finite differences reject."""
    x, dy, h0 = small(seed=7)
    heads, P = x["heads"], x["headdim"]
    g = oracle.scan_bwd(x["x"], x["dt"].repeat_interleave(P, dim=1).contiguous(),
                        x["A"].repeat_interleave(P)[:, None].expand(heads * P, x["dstate"]).contiguous(),
                        x["B"], x["C"], x["D"], x["z"], x["dt_bias"].repeat_interleave(P), x["softplus"], h0=h0, dy=dy)
    wrong = g["ddelta"].reshape(1, P, heads, -1).sum(axis=1)  # channels regrouped across heads
    fd = central(x, dy, h0, "dt", 1)
    right = grads(x, dy, h0)["ddt"].reshape(-1)[1]
    assert abs(fd - right) <= 2e-4 * max(1e-3, abs(right))
    assert abs(fd - wrong.reshape(-1)[1]) > 1e-3 * max(1e-3, abs(right))
