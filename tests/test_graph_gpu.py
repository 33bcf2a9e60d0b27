"""GPU: the forward scan and the decode step captured in a HIP graph.

The scan's chained launch plan keeps hand-over flags and an interval ticket in
scratch memory that a small fill kernel clears (no memset node), and the
split plan allocates its segment carries stream-ordered; both must behave the
same on every replay of a captured call.  Each test captures one call,
replays it several times with eager library work and synchronisations in
between, and checks every replay bit for bit against the eager result (the
kernels are deterministic).
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


def scan_args(t):
    return (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["dt_bias"])


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


# the launch plans of the chunked scan -- chained intervals (320 channel groups), one pass
# (160 groups), the aggregate/carry/output split (one group, 2^16 steps) -- and the generic
# kernel (a sequence length whose bf16 rows are not whole 16-byte pieces)
@pytest.mark.parametrize("shape", [(4, 5120, 256), (1, 10240, 256), (1, 64, 65536), (2, 96, 700)])
def test_scan_graph_replays_match_eager(shape):
    B, D, L = shape
    note(f"scan graph B={B} D={D} L={L}")
    assert torch.cuda.is_available()
    g = dev(gen.random_scan_inputs(B, D, 16, L, "bf16", seed=3))
    other = dev(gen.random_scan_inputs(B, D, 16, L, "bf16", seed=4))
    ye, le = ssm.scan_fwd(*scan_args(g))
    torch.cuda.synchronize()
    y = torch.empty_like(ye)
    last = torch.empty_like(le)
    graph = capture(lambda: ssm.scan_fwd(*scan_args(g), y=y, last_state=last))
    for r in range(4):
        y.fill_(0)
        last.fill_(0)
        ssm.scan_fwd(*scan_args(other))  # eager work on the same scratch pool between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ye), f"replay {r}: y differs from the eager call"
        assert torch.equal(last, le), f"replay {r}: final state differs from the eager call"


def test_decode_graph_replays_match_eager():
    B, D, N = 64, 512, 16
    note(f"decode graph B={B} D={D} N={N}")
    p = dev(gen.random_scan_inputs(B, D, N, 8, "bf16", seed=5))
    step = {k: p[k][..., 3].contiguous() for k in ("u", "delta", "z", "B", "C")}
    s0 = torch.randn(B, D, N, device="cuda", dtype=torch.float32)

    def run(state, y=None):
        return ssm.state_update(state, step["u"], step["delta"], p["A"], step["B"], step["C"], p["D"], step["z"],
                                p["dt_bias"], y=y)

    se = s0.clone()
    ye = run(se)
    torch.cuda.synchronize()
    state = s0.clone()
    y = torch.empty_like(ye)
    graph = capture(lambda: run(state, y))
    for r in range(4):
        state.copy_(s0)
        y.fill_(0)
        run(torch.randn_like(s0))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ye), f"replay {r}: y differs from the eager step"
        assert torch.equal(state, se), f"replay {r}: state differs from the eager step"
