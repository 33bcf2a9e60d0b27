"""Seeded generator: determinism, shapes, dtypes and distributions (no GPU)."""
import hashlib

import numpy as np
import pytest
import torch

import gen


def _digest(x):
    h = hashlib.sha256()
    for k in sorted(x):
        v = x[k]
        if isinstance(v, torch.Tensor):
            h.update(k.encode())
            h.update(v.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    assert _digest(gen.scan_inputs(0)) == _digest(gen.scan_inputs(0))
    assert _digest(gen.scan_inputs(0)) != _digest(gen.scan_inputs(0, seed=1))
    a = gen.decode_step_inputs(4, 3)
    b = gen.decode_step_inputs(4, 3)
    assert all(torch.equal(a[k], b[k]) for k in a)
    assert not torch.equal(a["u"], gen.decode_step_inputs(4, 4)["u"])


@pytest.mark.parametrize("w", [0, 1])
def test_scan_shapes_and_dtypes(w):
    wl = gen.WORKLOADS[w]
    x = gen.scan_inputs(w)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    for k in ("u", "delta", "z"):
        assert x[k].shape == (wl.batch, wl.dim, wl.seqlen) and x[k].dtype == dt and x[k].is_contiguous()
    for k in ("B", "C"):
        assert x[k].shape == (wl.batch, wl.dstate, wl.seqlen) and x[k].dtype == dt
    assert x["A"].shape == (wl.dim, wl.dstate) and x["A"].dtype == torch.float32
    assert x["D"].shape == (wl.dim,) and x["dt_bias"].shape == (wl.dim,)


def test_distributions():
    x = gen.scan_inputs(1)
    A = x["A"].numpy()
    assert np.array_equal(A, -np.broadcast_to(np.arange(1, 17, dtype=np.float32), A.shape))
    bias = x["dt_bias"].double().numpy()
    dt0 = np.log1p(np.exp(bias))       # softplus(dt_bias) is the drawn step
    assert dt0.min() >= 1e-3 * (1 - 1e-5) and dt0.max() <= 1e-1 * (1 + 1e-5)
    dt = np.log1p(np.exp(x["delta"][0].float().double().numpy() + bias[:, None]))
    assert 2e-4 < dt.min() and dt.max() < 0.3
    D = x["D"].numpy()
    assert abs(D.mean() - 1) < 0.02 and abs(D.std() - 0.1) < 0.02
    u = x["u"].float().numpy()
    assert abs(u.mean()) < 0.01 and abs(u.std() - 1) < 0.01
    d = x["delta"].float().numpy()
    assert abs(d.std() - 0.1) < 0.002
    assert torch.all(gen.scan_inputs(0)["D"] == 1)


def test_bf16_rounding_is_rne():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    r = gen.to_dtype(v, "bf16").float().numpy()
    # ties go to even mantissa; above-tie rounds up
    assert r.tolist() == [1.0, 1.0 + 4 * 2 ** -8, 1.0 + 2 ** -7]


def test_token_workload_u_is_projection():
    # small stand-in for workload 3's recipe (u = P[token]): each column of u is one of 4 rows of P
    w = gen.Workload(99, "tok", 1, 8, 4, 512, "f32", u_tokens=True)
    x = gen.scan_inputs(w, seed=3)
    cols = x["u"][0].T.numpy()   # [L, D]
    uniq = np.unique(cols, axis=0)
    assert uniq.shape[0] == 4


def test_decode_inputs():
    p = gen.decode_params(4)
    s = gen.decode_state(4)
    st = gen.decode_step_inputs(4, 0)
    assert s.shape == (256, 5120, 16) and s.dtype == torch.float32
    assert st["u"].shape == (256, 5120) and st["u"].dtype == torch.bfloat16
    assert st["B"].shape == (256, 16)
    assert p["A"].shape == (5120, 16)


def test_device_inputs_are_seeded_and_shaped():
    # the on-device recipe, here drawn on the CPU device: same seed, same bytes; the stated scales
    a = gen.device_scan_inputs(2, 3, 4, 4096, seed=5, device="cpu")
    b = gen.device_scan_inputs(2, 3, 4, 4096, seed=5, device="cpu")
    for k in ("u", "delta", "z", "B", "C"):
        assert a[k].dtype == torch.bfloat16 and torch.equal(a[k], b[k]), k
    assert a["u"].shape == (2, 3, 4096) and a["B"].shape == (2, 4, 4096)
    assert abs(a["delta"].float().std().item() - 0.1) < 0.01 and abs(a["u"].float().std().item() - 1.0) < 0.05
    assert torch.equal(a["A"], gen.scan_inputs(0)["A"][:3, :4])
