"""The allocation-free scan entry point against the allocating one, through the C ABI.

selective_scan_fwd_noalloc takes its scratch from a fixed per-GPU array instead of the
stream-ordered pool; with the same inputs it runs the same launch plan and kernels, so its
outputs must equal selective_scan_fwd_resume's bit for bit (and both stay within the oracle
tolerance on sampled channels).  Calls follow each other on one array: the second is smaller
than the first, so stale flags, tickets or carries of a larger call would show.
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
UNSUPPORTED = -6


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def raw_args(g, y, last, h0):
    b, d, L = g["u"].shape
    n = g["A"].shape[1]
    p = lambda t: None if t is None else t.data_ptr()
    code = ssm.BF16 if g["u"].dtype == torch.bfloat16 else ssm.F32
    return [p(g["u"]), p(g["delta"]), p(g["A"]), p(g["B"]), p(g["C"]), p(g.get("D")), p(g.get("z")),
            p(g.get("dt_bias")), 1, p(h0), p(y), p(last), b, d, n, L, code,
            torch.cuda.current_stream().cuda_stream]


# (name, batch, dim, dstate, seqlen, dtype, plan): each later call smaller than the one before
CALLS = [
    ("intervals, larger", 4, 5120, 16, 512, "bf16", "intervals"),
    ("intervals, smaller", 2, 8192, 16, 256, "bf16", "intervals"),
    ("two-pass, smaller again", 1, 128, 16, 16384, "f32", "two-pass"),
    ("generic, smallest", 1, 70, 2, 333, "f32", "generic"),
]


def test_noalloc_matches_allocating_entry_point():
    assert torch.cuda.is_available()
    ssm.load()
    for i, (name, b, d, n, L, dt, mode) in enumerate(CALLS):
        plan = ssm.scan_plan(b, d, n, L, torch.bfloat16 if dt == "bf16" else torch.float32,
                             torch.cuda.get_device_properties(0).multi_processor_count)
        note(f"noalloc call {i}: {name}: B={b} D={d} N={n} L={L} {dt} plan={plan}")
        assert plan["mode"] == mode
        x = gen.random_scan_inputs(b, d, n, L, dt, seed=100 + i)
        g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
        h0 = torch.from_numpy(np.random.default_rng(i).standard_normal((b, d, n), dtype=np.float32)).cuda() \
            if i % 2 == 0 else None
        y_a, y_n = torch.empty_like(g["u"]), torch.full_like(g["u"], float("nan"))
        l_a = torch.empty((b, d, n), dtype=torch.float32, device="cuda")
        l_n = torch.full_like(l_a, float("nan"))
        assert ssm.selective_scan_fwd_resume(*raw_args(g, y_a, l_a, h0)) == 0, ssm.last_error()
        assert ssm.selective_scan_fwd_noalloc(*raw_args(g, y_n, l_n, h0)) == 0, ssm.last_error()
        torch.cuda.synchronize()
        assert torch.equal(y_a.view(torch.int16 if dt == "bf16" else torch.int32),
                           y_n.view(torch.int16 if dt == "bf16" else torch.int32)), name
        assert torch.equal(l_a.view(torch.int32), l_n.view(torch.int32)), name
        # and within the oracle tolerance on a few channels (the last one included)
        chans = np.unique(np.array([0, (b * d) // 2, b * d - 1]))
        yr, lr = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["dt_bias"], True,
                             chans=chans, h0=None if h0 is None else h0.cpu().numpy().reshape(-1, n)[chans])
        idx = torch.as_tensor(chans, device="cuda")
        ey = oracle.rel_err(y_n.reshape(-1, L)[idx].float().cpu().double().numpy(), yr)
        el = oracle.rel_err(l_n.reshape(-1, n)[idx].cpu().double().numpy(), lr)
        note(f"  bit-identical to selective_scan_fwd_resume; oracle y err {ey:.2e}, last_state err {el:.2e}")
        assert ey <= TOL[dt] and el <= TOL[dt], (ey, el)


def test_noalloc_refuses_what_the_array_cannot_hold():
    # 1 x 256 channels of dstate 64 over 2^20 steps: 512 segments of aggregates, 34 MB > 16 MiB
    b, d, n, L = 1, 256, 64, 1 << 20
    note(f"noalloc refusal: B={b} D={d} N={n} L={L} f32")
    big = torch.empty(b * d * L + 64, dtype=torch.float32, device="cuda")
    y = torch.full((b * d * L,), 7.0, dtype=torch.float32, device="cuda")
    last = torch.full((b * d * n,), 7.0, dtype=torch.float32, device="cuda")
    A = torch.full((d * n,), -1.0, dtype=torch.float32, device="cuda")
    bc = torch.empty(b * n * L, dtype=torch.float32, device="cuda")
    rc = ssm.selective_scan_fwd_noalloc(big.data_ptr(), big.data_ptr(), A.data_ptr(), bc.data_ptr(), bc.data_ptr(),
                                        None, None, None, 1, None, y.data_ptr(), last.data_ptr(), b, d, n, L,
                                        ssm.F32, torch.cuda.current_stream().cuda_stream)
    assert rc == UNSUPPORTED, rc
    assert "scratch" in ssm.last_error()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()) and bool((last == 7.0).all())
