"""GPU: non-finite inputs propagate and stay where the recurrence puts them.

The C ABI does not check inputs for NaN or infinity; it documents that they
propagate.  A NaN planted in one channel's u at step t0 makes that channel's
state NaN from t0 on (h_t = Abar h_{t-1} + Delta B u keeps it), so y[b, d, t]
is NaN exactly for t >= t0 and the final state of (b, d) is NaN.  Every other
output must be bit-identical to the run without the NaN: no other channel,
batch row or earlier step reads that value, under any launch plan (the
chained hand-over and the split's segment carries are per channel).  A NaN in
B[b, n, t0] reaches every channel of batch row b from t0 on and nothing else.
The decode step likewise confines a NaN in one state row to that row and its y.
"""
import sys

import pytest
import torch

import gen
import selective_scan_02_amd as ssm

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def run(t):
    y, last = ssm.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["dt_bias"])
    torch.cuda.synchronize()
    return y.float().cpu(), last.cpu()


# chained intervals (320 channel groups), one pass (160), two-pass split (4 groups), generic kernel
@pytest.mark.parametrize("shape", [(4, 5120, 256), (1, 10240, 256), (2, 96, 4096), (2, 96, 700)])
def test_nan_in_u_stays_in_its_channel(shape):
    B, D, L = shape
    b0, d0, t0 = B - 1, D // 3, L // 3
    note(f"NaN in u[{b0},{d0},{t0}] of B={B} D={D} L={L}")
    x = dev(gen.random_scan_inputs(B, D, 16, L, "bf16", seed=11))
    y_ref, last_ref = run(x)
    assert torch.isfinite(y_ref).all() and torch.isfinite(last_ref).all()
    x["u"] = x["u"].clone()
    x["u"][b0, d0, t0] = float("nan")
    y, last = run(x)
    hit = torch.zeros_like(y, dtype=torch.bool)
    hit[b0, d0, t0:] = True
    assert torch.isnan(y[hit]).all(), "the NaN must reach every later step of its channel"
    assert torch.equal(y[~hit], y_ref[~hit]), "every other output must be unchanged"
    assert torch.isnan(last[b0, d0]).all()
    keep = torch.ones(B, D, dtype=torch.bool)
    keep[b0, d0] = False
    assert torch.equal(last[keep], last_ref[keep])


@pytest.mark.parametrize("shape", [(4, 5120, 256), (2, 96, 4096)])
def test_nan_in_B_reaches_its_batch_row_only(shape):
    B, D, L = shape
    b0, n0, t0 = 1, 5, L // 2
    note(f"NaN in B[{b0},{n0},{t0}] of B={B} D={D} L={L}")
    x = dev(gen.random_scan_inputs(B, D, 16, L, "bf16", seed=12))
    y_ref, last_ref = run(x)
    x["B"] = x["B"].clone()
    x["B"][b0, n0, t0] = float("nan")
    y, last = run(x)
    assert torch.isnan(y[b0, :, t0:]).all()
    assert torch.equal(y[b0, :, :t0], y_ref[b0, :, :t0])
    others = [b for b in range(B) if b != b0]
    assert torch.equal(y[others], y_ref[others])
    assert torch.isnan(last[b0, :, n0]).all()
    assert torch.equal(last[others], last_ref[others])


def test_decode_nan_state_row_stays_in_its_row():
    Bt, D, N = 32, 512, 16
    note(f"decode NaN state row B={Bt} D={D}")
    p = dev(gen.random_scan_inputs(Bt, D, N, 4, "bf16", seed=13))
    step = {k: p[k][..., 2].contiguous() for k in ("u", "delta", "z", "B", "C")}
    s0 = torch.randn(Bt, D, N, device="cuda", dtype=torch.float32)

    def go(state):
        y = ssm.state_update(state, step["u"], step["delta"], p["A"], step["B"], step["C"], p["D"], step["z"],
                             p["dt_bias"])
        torch.cuda.synchronize()
        return y.float().cpu(), state.cpu()

    y_ref, s_ref = go(s0.clone())
    bad = s0.clone()
    bad[7, 100, 3] = float("nan")
    y, s = go(bad)
    assert torch.isnan(y[7, 100])
    assert torch.isnan(s[7, 100, 3])
    mask = torch.ones(Bt, D, dtype=torch.bool)
    mask[7, 100] = False
    assert torch.equal(y[mask], y_ref[mask])
    assert torch.equal(s[mask], s_ref[mask])
    # the row's other states do not mix with state 3 within the step
    assert torch.equal(s[7, 100, :3], s_ref[7, 100, :3]) and torch.equal(s[7, 100, 4:], s_ref[7, 100, 4:])
