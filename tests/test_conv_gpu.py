"""GPU parity of the causal conv1d (+ SiLU) and its decode step, through the C ABI.

Compared with the fp64 oracle (oracle.conv1d) element by element on small and
ragged shapes and on sampled rows of a 2.8B-shaped layer; the carried window
state must equal the oracle's exactly (it holds inputs, which fp32 represents
exactly).  The decode step must reproduce the whole-sequence kernel bit for bit,
as must a sequence split in two with the state carried between the halves.
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


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    ssm.load()


def make(batch, dim, L, K, dtype, seed, bias=True, state=True):
    g = np.random.default_rng(seed)
    x = gen.to_dtype(g.standard_normal((batch, dim, L), dtype=np.float32), dtype)
    w = torch.from_numpy(g.standard_normal((dim, K), dtype=np.float32) * 0.5)
    b = torch.from_numpy(g.standard_normal(dim, dtype=np.float32) * 0.1) if bias else None
    st = torch.from_numpy(g.standard_normal((batch, dim, K - 1), dtype=np.float32)) if state else None
    return x, w, b, st


def cuda(t):
    return None if t is None else t.cuda()


def f64(t):
    return t.detach().float().cpu().double().numpy()


SHAPES = [
    (1, 5, 1, 4, "f32", True, True, True),
    (2, 7, 13, 3, "bf16", True, True, True),
    (1, 64, 512, 4, "f32", True, True, False),
    (2, 33, 1000, 4, "bf16", True, False, True),
    (1, 3, 2, 4, "f32", True, True, True),      # shorter than the window
    (3, 130, 2049, 2, "f32", False, True, True),
    (2, 9, 77, 1, "bf16", True, True, False),
    (1, 300, 4096, 4, "bf16", True, True, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_conv_fwd_matches_oracle(shape):
    b, d, L, K, dt, silu, bias, state = shape
    note(f"conv fwd B={b} D={d} L={L} K={K} {dt} silu={silu} bias={bias} state={state}")
    x, w, bb, st = make(b, d, L, K, dt, seed=L + K, bias=bias, state=state)
    out, so = ssm.conv1d_fwd(x.cuda(), w.cuda(), cuda(bb), silu, cuda(st))
    torch.cuda.synchronize()
    ro, rs = oracle.conv1d(x, w, bb, silu, st)
    err = oracle.rel_err(f64(out), ro)
    note(f"  out err {err:.3e}")
    assert err <= TOL[dt]
    assert np.array_equal(f64(so), rs)


def test_conv_fwd_full_size_sampled():
    # 2.8B-shaped layer: x [4, 5120, 2048] bf16, width 4
    x, w, b, st = make(4, 5120, 2048, 4, "bf16", seed=2)
    note("conv fwd 2.8B-shaped layer, sampled rows")
    out, so = ssm.conv1d_fwd(x.cuda(), w.cuda(), b.cuda(), True, st.cuda())
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(4 * 5120, 300, replace=False), [0, 20479]]))
    xs = x.reshape(-1, 1, 2048)[rows]
    ws = w[torch.as_tensor(rows % 5120)]
    bs = b[torch.as_tensor(rows % 5120)]
    ss = st.reshape(-1, 1, 3)[rows]
    # the oracle treats each sampled row as its own (batch = rows, dim = 1) problem
    ro, rs = [], []
    for i in range(len(rows)):
        o1, s1 = oracle.conv1d(xs[i:i + 1], ws[i:i + 1], bs[i:i + 1], True, ss[i:i + 1])
        ro.append(o1[0, 0])
        rs.append(s1[0, 0])
    idx = torch.as_tensor(rows, device=out.device)
    err = oracle.rel_err(f64(out.reshape(-1, 2048)[idx]), np.stack(ro))
    note(f"  out err {err:.3e}")
    assert err <= TOL["bf16"]
    assert np.array_equal(f64(so.reshape(-1, 3)[idx]), np.stack(rs))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("K", [2, 4])
def test_decode_steps_reproduce_fwd_bit_for_bit(dt, K):
    b, d, L = 3, 200, 40
    x, w, bb, st = make(b, d, L, K, dt, seed=K)
    note(f"conv decode vs fwd {dt} K={K}")
    xg, wg, bg, sg = x.cuda(), w.cuda(), bb.cuda(), st.cuda()
    full, s_full = ssm.conv1d_fwd(xg, wg, bg, True, sg)
    s = sg.clone()
    for t in range(L):
        o = ssm.conv1d_update(s, xg[..., t].contiguous(), wg, bg, True)
        assert torch.equal(o, full[..., t]), t
    torch.cuda.synchronize()
    assert torch.equal(s, s_full)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_split_sequence_with_carried_state_is_bit_exact(dt):
    x, w, bb, st = make(2, 100, 1500, 4, dt, seed=9)
    note(f"conv split + carry {dt}")
    xg, wg, bg, sg = x.cuda(), w.cuda(), bb.cuda(), st.cuda()
    full, s_full = ssm.conv1d_fwd(xg, wg, bg, True, sg)
    o1, s1 = ssm.conv1d_fwd(xg[..., :777].contiguous(), wg, bg, True, sg)
    o2, s2 = ssm.conv1d_fwd(xg[..., 777:].contiguous(), wg, bg, True, s1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=-1), full)
    assert torch.equal(s2, s_full)


def test_empty_sequence_passes_the_state_on():
    _, w, _, st = make(2, 10, 1, 4, "f32", seed=1)
    x = torch.empty(2, 10, 0, device="cuda")
    _, so = ssm.conv1d_fwd(x, w.cuda(), None, True, st.cuda())
    torch.cuda.synchronize()
    assert torch.equal(so.cpu(), st)
    _, so = ssm.conv1d_fwd(x, w.cuda(), None, True, None)
    assert torch.count_nonzero(so) == 0
