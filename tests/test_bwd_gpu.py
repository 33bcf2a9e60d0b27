"""GPU parity of the backward scan (selective_scan_bwd) against the fp64 oracle.

Every gradient the C ABI returns is compared with oracle.scan_bwd element by
element, on small shapes that span several chunks, several sequence segments, a
ragged tail and a partial channel group, and on the full 2.8B-shaped layer
(batch 4, d_inner 5120, d_state 16, L 2048, bf16), which the oracle finishes in
seconds.  Tolerances as for the forward: 1e-4 for fp32 inputs, 2e-2 for bf16
inputs (outputs in bf16, fp32 state), on the metric of oracle.rel_err.
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
KEYS = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddt_bias", "dh0")


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


def upstream(x, seed):
    g = np.random.default_rng(500 + seed)
    return gen.to_dtype(g.standard_normal((x["batch"], x["dim"], x["seqlen"]), dtype=np.float32), x["dtype"])


def initial(x, seed):
    g = np.random.default_rng(900 + seed)
    return torch.from_numpy(g.standard_normal((x["batch"], x["dim"], x["dstate"]), dtype=np.float32))


def gpu_bwd(x, dy, h0=None):
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    g = ssm.scan_bwd(c["u"], c["delta"], c["A"], c["B"], c["C"], c.get("D"), c.get("z"), c.get("dt_bias"),
                     softplus=x.get("softplus", True), dy=dy.cuda(), initial_state=None if h0 is None else h0.cuda())
    torch.cuda.synchronize()
    g["dh0"] = g.pop("dinitial_state")
    return g


def ref_bwd(x, dy, h0=None):
    return oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x.get("D"), x.get("z"), x.get("dt_bias"),
                           x.get("softplus", True), h0=h0, dy=dy)


def compare(x, got, ref, tol):
    worst = {}
    for k in KEYS:
        if ref[k] is None:
            assert got[k] is None or k in ("dD", "ddt_bias"), k
            continue
        worst[k] = oracle.rel_err(f64(got[k]), ref[k])
    note("  " + " ".join(f"{k}={v:.1e}" for k, v in worst.items()))
    for k, v in worst.items():
        assert v <= tol, (k, v)


# (batch, dim, dstate, seqlen, dtype, options)
SMALL = [
    (1, 16, 4, 64, "f32", {}),                                   # the tiny workload's shape
    (2, 100, 16, 700, "f32", {}),                                # partial channel group, segments, ragged tail
    (2, 64, 16, 333, "bf16", {"h0": True}),
    (1, 70, 16, 1000, "f32", {"with_z": False, "with_D": False}),
    (1, 40, 16, 257, "f32", {"with_bias": False, "softplus": False, "delta_scale": 0.02}),
    (3, 9, 8, 130, "bf16", {"h0": True}),
    (1, 33, 1, 99, "f32", {}),
    (2, 17, 2, 300, "f32", {"h0": True}),
    (1, 65, 32, 200, "f32", {"a_mode": "random"}),
    (1, 20, 64, 77, "f32", {"h0": True}),
    (1, 5, 16, 1, "f32", {"h0": True}),
    (1, 192, 16, 2048, "bf16", {}),
    # 16-byte rows (fast path): partial staged tiles; the main pass with scanner and helper waves
    # (dstate 8-32: eight scanners with bf16 inputs up to dstate 16, else four) or with symmetric
    # waves (dstate 64)
    (2, 130, 16, 520, "bf16", {"h0": True}),
    (1, 64, 8, 264, "f32", {"with_z": False}),
    (2, 100, 64, 136, "bf16", {}),
    (1, 70, 32, 4104, "f32", {"h0": True}),
    (2, 100, 8, 264, "bf16", {"h0": True}),
    (1, 70, 32, 1032, "bf16", {}),
    (1, 64, 16, 24, "bf16", {"with_z": False, "h0": True}),     # one short last tile: three chunks
    (1, 130, 16, 808, "f32", {"softplus": False, "with_bias": False, "delta_scale": 0.02}),
    # at least as many chains (batch row x channel group) as CUs: the main pass on intervals, chains
    # split between two workgroups and the adjoint handed over at the split
    (4, 4100, 16, 136, "bf16", {"h0": True}),
    (4, 5000, 8, 264, "f32", {"with_z": False}),
    (2, 8200, 32, 64, "bf16", {}),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}x{c[3]}-{c[4]}")
def test_bwd_matches_oracle(case):
    b, d, n, L, dt, opt = case
    opt = dict(opt)
    use_h0 = opt.pop("h0", False)
    note(f"bwd B={b} D={d} N={n} L={L} {dt} h0={use_h0} {opt}")
    x = gen.random_scan_inputs(b, d, n, L, dt, seed=L + n, **opt)
    dy = upstream(x, L)
    h0 = initial(x, L) if use_h0 else None
    got = gpu_bwd(x, dy, h0)
    ref = ref_bwd(x, dy, h0)
    compare(x, got, ref, TOL[dt])


def test_bwd_full_2p8b_layer():
    x = gen.scan_inputs(2)
    note("bwd 2.8B-shaped layer, every output against the oracle")
    dy = upstream(x, 2)
    got = gpu_bwd(x, dy)
    ref = ref_bwd(x, dy)
    compare(x, got, ref, TOL["bf16"])


def test_bwd_full_130m_layer():
    x = gen.scan_inputs(1)
    note("bwd 130M-shaped layer (B=8, D=1536, N=16, L=2048, bf16), every output against the oracle")
    dy = upstream(x, 1)
    got = gpu_bwd(x, dy)
    ref = ref_bwd(x, dy)
    compare(x, got, ref, TOL["bf16"])


def test_bwd_is_deterministic():
    x = gen.random_scan_inputs(2, 300, 16, 1500, "f32", seed=4)
    note("bwd run twice, bitwise")
    dy = upstream(x, 4)
    a, b = gpu_bwd(x, dy), gpu_bwd(x, dy)
    for k in KEYS:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def test_bwd_empty_sequence_gives_zero_parameter_gradients():
    x = gen.random_scan_inputs(2, 10, 4, 0, "f32", seed=1)
    note("bwd L=0")
    got = gpu_bwd(x, upstream(x, 0), initial(x, 0))
    for k in ("dA", "dD", "ddt_bias", "dh0"):
        assert torch.count_nonzero(got[k]) == 0, k
    assert got["du"].numel() == 0 and got["dB"].numel() == 0


def test_bwd_intervals_deterministic():
    """The main pass on intervals (chains handed over between workgroups) is bitwise reproducible."""
    x = gen.random_scan_inputs(4, 4100, 16, 264, "bf16", seed=8)
    note("bwd on intervals run twice, bitwise")
    dy = upstream(x, 8)
    a, b = gpu_bwd(x, dy), gpu_bwd(x, dy)
    for k in KEYS:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def test_bwd_handover_giveup_poisons_and_counts():
    """A hand-over wait of the backward's main pass that gives up (forced from the host: the
    right parts of split chains skip their flags, the wait is bounded at a few polls) counts one
    give-up per scanner wave of every split chain and leaves NaN in the gradients that depend on
    the missing adjoint; every kernel still runs to its end, and the next normal call is
    bit-identical to one made before."""
    b, d, n, L = 4, 4100, 16, 264
    x = gen.random_scan_inputs(b, d, n, L, "bf16", seed=9)
    dy = upstream(x, 9)
    note(f"bwd hand-over give-up B={b} D={d} N={n} L={L}")
    ref = gpu_bwd(x, dy)
    ssm.handover_failures(reset=True)
    try:
        ssm.set_handover_wait(max_polls=64, publish=False)
        bad = gpu_bwd(x, dy)
    finally:
        ssm.set_handover_wait(0, True)
    count = ssm.handover_failures(reset=True)
    # the interval plan: chains laid end to end, cut into as many intervals as CUs (one
    # workgroup of the main pass per CU); a chain is split where an interval boundary falls
    # inside it
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    chains, tch = b * ((d + 63) // 64), L // 8
    wlen = -(-chains * tch // cus)
    units = -(-chains * tch // wlen)
    split = sum(1 for i in range(1, units) if (i * wlen) % tch)
    note(f"  {split} split chains, {count} waits gave up")
    assert split > 0 and count == 4 * split
    assert torch.isnan(bad["du"].float()).any() and torch.isnan(bad["dA"]).any()
    again = gpu_bwd(x, dy)
    assert ssm.handover_failures(reset=True) == 0
    for k in KEYS:
        if ref[k] is not None:
            assert torch.equal(again[k], ref[k]), k
