"""GPU parity of the Mamba-2 SSD scan (ssd_scan_fwd, matrix cores) against the fp64 oracle.

oracle.ssd is the sequential recurrence with the per-head decay and step broadcast to
the head's channels (pinned in test_oracle_ssd.py).  Every output is compared element by
element on small shapes (ragged last chunk, one to three heads, dstate 16/32/64, with and
without gate, skip, bias, softplus and initial state; heads of 32, 64 and 128 channels) and on
the 2.8B-shaped layer as 80 heads of 64 channels.  The matrix-core products take bf16 operands, so the bound is the
bf16 one (2e-2, metric of oracle.rel_err) for y and for the final state.
"""
import sys

import numpy as np
import pytest
import torch

import gen
import oracle
import selective_scan_02_amd as ssm

pytestmark = pytest.mark.gpu

TOL = 2e-2


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    ssm.load()
    yield
    torch.cuda.synchronize()


def f64(t):
    return t.detach().float().cpu().double().numpy()


def run(x, h0=None, in_place=False):
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    hg = None if h0 is None else h0.cuda()
    y, last = ssm.ssd_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["z"], c["dt_bias"], x["softplus"],
                          initial_state=hg, last_state=hg if in_place else None, headdim=x["headdim"])
    torch.cuda.synchronize()
    ry, rl = oracle.ssd(x["x"], x["dt"], x["A"], x["B"], x["C"], x["D"], x["z"], x["dt_bias"], x["softplus"],
                        headdim=x["headdim"], h0=h0)
    return oracle.rel_err(f64(y), ry), oracle.rel_err(f64(last), rl)


CASES = [
    (1, 1, 16, 64, {}),
    (2, 3, 16, 200, {}),                                  # ragged last chunk (8 steps)
    (1, 2, 32, 1000, {"with_z": False}),
    (2, 1, 64, 136, {"with_D": False, "with_bias": False}),
    (1, 2, 16, 8, {}),
    (3, 2, 16, 520, {"softplus": False, "with_bias": False}),
    (1, 4, 64, 2048, {}),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}h{c[1]}n{c[2]}L{c[3]}")
def test_ssd_matches_oracle(case):
    b, h, n, L, opt = case
    note(f"ssd B={b} H={h} N={n} L={L} {opt}")
    x = gen.ssd_inputs(b, h, 64, n, L, "bf16", seed=L + n, **opt)
    if not x["softplus"]:
        x["dt"] = torch.abs(x["dt"])
    ey, el = run(x)
    note(f"  y {ey:.2e}  last_state {el:.2e}")
    assert ey <= TOL and el <= TOL


# heads of 32 and 128 channels (the kernels are templates over the head size)
HEAD_CASES = [
    (32, 1, 2, 16, 200, {}),                                # ragged last chunk
    (32, 2, 3, 32, 1032, {"with_z": False}),
    (32, 1, 1, 64, 136, {"with_D": False, "with_bias": False}),
    (128, 1, 2, 16, 520, {}),
    (128, 2, 1, 32, 1000, {"softplus": False, "with_bias": False}),
    (128, 1, 3, 16, 8, {}),
]


@pytest.mark.parametrize("case", HEAD_CASES, ids=lambda c: f"P{c[0]}b{c[1]}h{c[2]}n{c[3]}L{c[4]}")
def test_ssd_other_head_sizes_match_oracle(case):
    P, b, h, n, L, opt = case
    note(f"ssd P={P} B={b} H={h} N={n} L={L} {opt}")
    x = gen.ssd_inputs(b, h, P, n, L, "bf16", seed=L + n + P, **opt)
    if not x["softplus"]:
        x["dt"] = torch.abs(x["dt"])
    ey, el = run(x)
    note(f"  y {ey:.2e}  last_state {el:.2e}")
    assert ey <= TOL and el <= TOL


def test_ssd_head_128_from_initial_state():
    x = gen.ssd_inputs(1, 2, 128, 32, 264, "bf16", seed=9)
    h0 = torch.from_numpy(np.random.default_rng(9).standard_normal((1, 256, 32), dtype=np.float32))
    note("ssd P=128 resumed from a state")
    ey, el = run(x, h0=h0)
    note(f"  y {ey:.2e}  last_state {el:.2e}")
    assert ey <= TOL and el <= TOL


def test_ssd_from_initial_state_in_place():
    x = gen.ssd_inputs(2, 2, 64, 16, 300 - 300 % 8, "bf16", seed=5)
    h0 = torch.from_numpy(np.random.default_rng(5).standard_normal((2, 128, 16), dtype=np.float32))
    note("ssd resumed from a state, advanced in place")
    ey, el = run(x, h0=h0, in_place=True)
    note(f"  y {ey:.2e}  last_state {el:.2e}")
    assert ey <= TOL and el <= TOL


def test_ssd_full_2p8b_layer():
    s = gen.SSD_LAYER
    x = gen.ssd_inputs(s["batch"], s["heads"], s["headdim"], s["dstate"], s["seqlen"], s["dtype"], seed=2)
    note("ssd 2.8B-shaped layer (80 heads x 64 channels, N=16, L=2048), every output")
    ey, el = run(x)
    note(f"  y {ey:.2e}  last_state {el:.2e}")
    assert ey <= TOL and el <= TOL


def test_ssd_empty_sequence():
    x = gen.ssd_inputs(1, 2, 64, 16, 0, "bf16", seed=1)
    h0 = torch.ones(1, 128, 16)
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    _, last = ssm.ssd_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["z"], c["dt_bias"],
                          initial_state=h0.cuda())
    torch.cuda.synchronize()
    assert torch.equal(last.cpu(), h0)
