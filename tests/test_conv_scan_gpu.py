"""GPU parity of the causal conv1d + SiLU fused ahead of the scan (selective_scan_fwd_conv).

Reference: the fp64 oracle's convolution (oracle.conv1d) followed by its scan (oracle.scan) --
the block's step before the scan, then the scan (Mamba summary, 方法 third step; mlqm.cn
tutorial §7.1).  The oracle's scan reads its inputs as fp32 or bf16 bytes of one dtype, so the
composed reference widens x's companions (delta, z, B, C) exactly to fp32 and rounds the fp64
convolution output u to fp32 (relative error 2^-24, far below the tolerances), and further to bf16
for bf16 rows, as the convolution kernel of their route stores it.  The call runs the
fused kernels for fp32 rows (u kept in fp32, never stored) and, for bf16 rows, the convolution
kernel into scratch and then the scan (the faster route there; u rounded to bf16 in between), so:
  * y and last_state match that reference within 1e-4 (fp32 I/O) or 2e-2 (bf16 I/O);
  * the convolution state out is exact (it is a copy of inputs);
  * with fp32 I/O the fused call equals causal_conv1d_fwd followed by the scan bit for bit
    (same fp32 arithmetic in the same order; the separate route stores u in fp32 too).
Every launch plan is covered: intervals, one pass and the two-pass split, with the fused kernels
(fp32, dstate 16) and with the two-kernel route (bf16, other dstates, rows that are not whole
16-byte pieces).
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


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().double().numpy()


def conv_inputs(b, d, n, L, dt, K, seed, bias=True, state=True, h0=False):
    x = gen.random_scan_inputs(b, d, n, L, dt, seed=seed)
    g = np.random.default_rng(seed + 1)
    x["cw"] = torch.from_numpy((g.standard_normal((d, K)) * 0.5).astype(np.float32))
    x["cb"] = torch.from_numpy((g.standard_normal(d) * 0.1).astype(np.float32)) if bias else None
    x["cst"] = torch.from_numpy(g.standard_normal((b, d, K - 1)).astype(np.float32)) if state and K > 1 else None
    x["h0"] = torch.from_numpy(g.standard_normal((b, d, n)).astype(np.float32)) if h0 else None
    return x


def cuda(t):
    return None if t is None else t.cuda()


def gpu_fused(x):
    y, last, cso = ssm.scan_fwd_conv(cuda(x["u"]), cuda(x["cw"]), cuda(x["delta"]), cuda(x["A"]), cuda(x["B"]),
                                     cuda(x["C"]), cuda(x["D"]), cuda(x["z"]), cuda(x["dt_bias"]),
                                     conv_bias=cuda(x["cb"]), conv_state=cuda(x["cst"]),
                                     initial_state=cuda(x["h0"]))
    torch.cuda.synchronize()
    return y, last, cso


def reference(x, chans=None):
    """oracle.conv1d then oracle.scan (on the sampled channels when given)."""
    u, st = x["u"], x["cst"]
    b, d, L = u.shape
    if chans is None:
        u64, so = oracle.conv1d(u, x["cw"], x["cb"], True, st)
        u32 = torch.from_numpy(u64.astype(np.float32))
    else:
        rows = np.asarray(chans)
        ds = rows % d
        xs = u.reshape(b * d, L)[rows].reshape(1, len(rows), L)
        sts = None if st is None else st.reshape(b * d, -1)[rows].reshape(1, len(rows), -1)
        u64, so = oracle.conv1d(xs, x["cw"][ds], None if x["cb"] is None else x["cb"][ds], True, sts)
        u32 = torch.zeros((b * d, L), dtype=torch.float32)
        u32[rows] = torch.from_numpy(u64.reshape(len(rows), L).astype(np.float32))
        u32 = u32.reshape(b, d, L)
        so = so.reshape(len(rows), -1)
    if x["dtype"] == "bf16":
        # bf16 rows take the convolution kernel, which writes u in the rows' dtype, then the scan
        u32 = u32.to(torch.bfloat16).float()
    f = lambda t: None if t is None else t.float()
    h0 = x["h0"]
    if h0 is not None and chans is not None:
        h0 = h0.reshape(b * d, -1)[np.asarray(chans)]
    yr, lr = oracle.scan(u32, f(x["delta"]), x["A"], f(x["B"]), f(x["C"]), x["D"], f(x["z"]), x["dt_bias"], True,
                         h0=h0, chans=chans)
    return yr, lr, so


def check(x, chans=None):
    dt = x["dtype"]
    y, last, cso = gpu_fused(x)
    yr, lr, sor = reference(x, chans)
    b, d, L = x["u"].shape
    n = x["A"].shape[1]
    if chans is not None:
        idx = torch.as_tensor(np.asarray(chans), device="cuda")
        y, last = y.reshape(-1, L)[idx], last.reshape(-1, n)[idx]
        cso = None if cso is None else cso.reshape(b * d, -1)[idx]
    ey, el = oracle.rel_err(f64(y), yr), oracle.rel_err(f64(last), lr)
    note(f"  y err {ey:.3e}  last_state err {el:.3e}  (tol {TOL[dt]:g})")
    assert ey <= TOL[dt] and el <= TOL[dt], (ey, el)
    if cso is not None:
        assert np.array_equal(f64(cso).reshape(sor.shape), sor)
    return y, last, cso


# small cases, element by element: (batch, dim, dstate, seqlen, dtype, width, bias, state, h0)
SMALL = [
    (2, 100, 16, 512, "bf16", 4, True, True, False),
    (1, 64, 16, 256, "f32", 3, True, True, True),
    (2, 70, 16, 1000, "f32", 2, False, True, False),
    (3, 33, 16, 64, "bf16", 1, True, False, False),
    (1, 16, 16, 8, "bf16", 4, True, True, True),
    (2, 130, 16, 520, "bf16", 4, False, False, False),
    (1, 40, 16, 6, "f32", 4, True, True, False),     # rows of 24 bytes: the two-kernel route
    (2, 50, 4, 300, "bf16", 4, True, True, True),    # dstate 4: the two-kernel route
    (1, 64, 8, 128, "f32", 3, True, True, False),    # dstate 8: the two-kernel route
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:6])))
def test_fused_conv_scan_small(case):
    b, d, n, L, dt, K, bias, state, h0 = case
    note(f"fused conv+scan B={b} D={d} N={n} L={L} {dt} K={K} bias={bias} state={state} h0={h0}")
    check(conv_inputs(b, d, n, L, dt, K, seed=b * 13 + L, bias=bias, state=state, h0=h0))


def sampled(total, k, seed):
    c = np.random.default_rng(seed).choice(total, size=min(k, total), replace=False)
    return np.unique(np.concatenate([c, [0, min(63, total - 1), min(64, total - 1), total - 1]]))


PLANS = [  # (name, plan, batch, dim, dstate, seqlen, dtype)
    ("intervals", "intervals", 2, 10240, 16, 512, "bf16"),
    ("intervals-f32", "intervals", 1, 20480, 16, 256, "f32"),
    ("single", "single", 1, 10240, 16, 256, "bf16"),
    ("single-f32", "single", 1, 10240, 16, 256, "f32"),
    ("two-pass", "two-pass", 1, 256, 16, 40_000, "f32"),
    ("two-pass-bf16", "two-pass", 2, 64, 16, 65_536, "bf16"),
]


@pytest.mark.parametrize("case", PLANS, ids=lambda c: c[0])
def test_fused_conv_scan_launch_plans(case):
    name, mode, b, d, n, L, dt = case
    plan = ssm.scan_plan(b, d, n, L, torch.bfloat16 if dt == "bf16" else torch.float32,
                         torch.cuda.get_device_properties(0).multi_processor_count)
    note(f"fused conv+scan {name}: B={b} D={d} N={n} L={L} {dt} plan={plan}")
    assert plan["mode"] == mode
    x = conv_inputs(b, d, n, L, dt, 4, seed=len(name), h0=True)
    check(x, chans=sampled(b * d, 40, 3))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fused_equals_separate_kernels(dt):
    """Against causal_conv1d_fwd followed by the scan on the GPU: bit for bit in fp32 (the fused
    kernels); in bf16 (where the call takes the same two kernels) both within the tolerance."""
    b, d, n, L = 2, 10240, 16, 512   # the interval plan
    note(f"fused vs separate kernels {dt}")
    x = conv_inputs(b, d, n, L, dt, 4, seed=7, h0=True)
    y1, l1, s1 = gpu_fused(x)
    u, s2 = ssm.conv1d_fwd(cuda(x["u"]), cuda(x["cw"]), cuda(x["cb"]), True, cuda(x["cst"]))
    y2, l2 = ssm.scan_fwd(u, cuda(x["delta"]), cuda(x["A"]), cuda(x["B"]), cuda(x["C"]), cuda(x["D"]),
                          cuda(x["z"]), cuda(x["dt_bias"]), initial_state=cuda(x["h0"]))
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    if dt == "f32":
        assert torch.equal(y1, y2) and torch.equal(l1, l2)
    else:
        chans = sampled(b * d, 64, 9)
        idx = torch.as_tensor(chans, device="cuda")
        yr, lr, _ = reference(x, chans)
        for y, l in ((y1, l1), (y2, l2)):
            assert oracle.rel_err(f64(y.reshape(-1, L)[idx]), yr) <= TOL[dt]
            assert oracle.rel_err(f64(l.reshape(-1, n)[idx]), lr) <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fused_in_two_pieces_continues_both_states(dt):
    """A sequence as two fused calls, the second continuing from the first's convolution state
    and scan state, equals the whole sequence in one call (within the tolerance; the pieces run
    other launch plans)."""
    b, d, n, L, a = 2, 300, 16, 2048, 1232
    note(f"fused conv+scan in two pieces {dt}")
    x = conv_inputs(b, d, n, L, dt, 4, seed=11)
    y, last, cso = gpu_fused(x)
    p1 = dict(x, **{k: x[k][..., :a].contiguous() for k in ("u", "delta", "z", "B", "C")})
    p2 = dict(x, **{k: x[k][..., a:].contiguous() for k in ("u", "delta", "z", "B", "C")})
    y1, l1, s1 = gpu_fused(p1)
    p2["cst"], p2["h0"] = s1.cpu(), l1.cpu()
    y2, l2, s2 = gpu_fused(p2)
    assert torch.equal(s2, cso)
    yr, lr, _ = reference(x)
    ey = oracle.rel_err(f64(torch.cat([y1, y2], dim=-1)), yr)
    el = oracle.rel_err(f64(l2), lr)
    note(f"  pieces: y err {ey:.3e}  last_state err {el:.3e}")
    assert ey <= TOL[dt] and el <= TOL[dt]


def test_fused_empty_sequence():
    b, d, n, K = 2, 10, 16, 4
    note("fused conv+scan L = 0")
    x = conv_inputs(b, d, n, 0, "f32", K, seed=1, h0=True)
    y, last, cso = gpu_fused(x)
    assert y.shape == (b, d, 0)
    assert torch.equal(last.cpu(), x["h0"]) and torch.equal(cso.cpu(), x["cst"])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_conv_scan_full_layer_sampled(dt):
    """The 2.8B-shaped layer (B=4, D=5120, N=16, L=2048) in the launch configuration the bench times:
    fp32 rows on the fused kernels, bf16 rows on the convolution kernel then the scan; sampled channels
    against the oracle, the whole convolution state exactly."""
    b, d, n, L = 4, 5120, 16, 2048
    note(f"conv+scan 2.8B-shaped layer {dt}")
    x = conv_inputs(b, d, n, L, dt, 4, seed=21, h0=True)
    check(x, chans=sampled(b * d, 48, 22))
