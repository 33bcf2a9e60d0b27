"""GPU parity of the SSD backward (ssd_scan_bwd) against the fp64 oracle.ssd_bwd.

Every gradient the C ABI returns is compared element by element with oracle.ssd_bwd (itself
pinned against central differences of the SSD forward oracle), on small shapes (several heads,
odd head sizes, fp32 and bf16, with and without the gate, D, dt_bias and softplus, an initial
state, a ragged sequence) and on the full 2.8B-shaped layer as 80 heads of 64 channels.
Tolerances as for the backward scan: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs, on the metric
of oracle.rel_err.  The per-head gradients (ddt, dA, ddt_bias) are sums over a head's channels
taken in a fixed order, so the results are reproducible bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import gen
import oracle
import selective_scan_02_amd as ssm

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
KEYS = ("dx", "ddt", "dz", "dA", "dB", "dC", "dD", "ddt_bias", "dh0")


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().double().numpy()


def inputs(b, H, P, N, L, dt, seed, **kw):
    x = gen.ssd_inputs(b, H, P, N, L, dt, seed=seed, **kw)
    g = np.random.default_rng(700 + seed)
    x["dy"] = gen.to_dtype(g.standard_normal((b, H * P, L), dtype=np.float32), dt)
    x["h0"] = None
    return x


def gpu(x):
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    g = ssm.ssd_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["z"], c["dt_bias"], c["softplus"],
                    dy=c["dy"], initial_state=c["h0"], headdim=x["headdim"])
    torch.cuda.synchronize()
    g["dh0"] = g.pop("dinitial_state")
    return g


def ref(x):
    return oracle.ssd_bwd(x["x"], x["dt"], x["A"], x["B"], x["C"], x["D"], x["z"], x["dt_bias"], x["softplus"],
                          headdim=x["headdim"], h0=x["h0"], dy=x["dy"])


def compare(got, want, tol):
    worst = {}
    for k in KEYS:
        if want[k] is None:
            assert got[k] is None or k in ("dD", "ddt_bias"), k
            continue
        worst[k] = oracle.rel_err(f64(got[k]), want[k])
    note("  " + " ".join(f"{k}={v:.1e}" for k, v in worst.items()))
    for k, v in worst.items():
        assert v <= tol, (k, v)


# (batch, heads, headdim, dstate, seqlen, dtype, options)
CASES = [
    (2, 4, 64, 16, 256, "bf16", {}),
    (1, 3, 32, 16, 200, "f32", {"h0": True}),
    (2, 5, 7, 4, 99, "f32", {"h0": True}),                                        # odd head size, ragged L
    (1, 2, 16, 8, 64, "bf16", {"with_z": False, "with_D": False}),
    (1, 3, 8, 16, 48, "f32", {"with_bias": False, "softplus": False}),
    (2, 6, 128, 32, 136, "bf16", {}),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}x{c[3]}x{c[4]}-{c[5]}")
def test_ssd_bwd_matches_oracle(case):
    b, H, P, N, L, dt, opt = case
    opt = dict(opt)
    use_h0 = opt.pop("h0", False)
    note(f"ssd bwd B={b} H={H} P={P} N={N} L={L} {dt} h0={use_h0} {opt}")
    x = inputs(b, H, P, N, L, dt, seed=L + P, **opt)
    if not x["softplus"]:
        x["dt"] = gen.to_dtype(np.abs(x["dt"].float().numpy()) * 0.5 + 0.05, dt)  # positive steps
    if use_h0:
        g = np.random.default_rng(L)
        x["h0"] = torch.from_numpy(g.standard_normal((b, H * P, N), dtype=np.float32))
    compare(gpu(x), ref(x), TOL[dt])


def test_ssd_bwd_full_2p8b_layer():
    b, H, P, N, L = 4, 80, 64, 16, 2048
    note("ssd bwd, the 2.8B-shaped layer as 80 heads of 64 channels, every output against the oracle")
    x = inputs(b, H, P, N, L, "bf16", seed=1)
    compare(gpu(x), ref(x), TOL["bf16"])


def test_ssd_bwd_is_deterministic():
    x = inputs(2, 8, 64, 16, 512, "bf16", seed=3)
    note("ssd bwd run twice, bitwise")
    a, c = gpu(x), gpu(x)
    for k in KEYS:
        if a[k] is not None:
            assert torch.equal(a[k], c[k]), k


def test_ssd_bwd_empty_sequence():
    x = inputs(2, 3, 16, 8, 0, "f32", seed=4)
    note("ssd bwd L = 0")
    g = gpu(x)
    for k in ("dA", "dD", "ddt_bias", "dh0"):
        assert torch.count_nonzero(g[k]) == 0, k
    assert g["dx"].numel() == 0 and g["ddt"].numel() == 0
