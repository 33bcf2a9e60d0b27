"""The interval schedule's persistent per-stream control block (ticket and hand-over flags).

Outside graph capture and without a caller's workspace, a scan on the interval plan takes its
ticket and hand-over flags from a block kept per (device, stream): the ticket only grows and each
call looks for flags holding its own generation, so nothing is cleared between calls.  A stale
ticket base or a flag of an earlier call taken for this call's would show as wrong or NaN
outputs, or as a hand-over give-up.  Checked here, bit for bit against the first call and
against the allocation-free entry point (which clears flags of its own in a fixed array):
repeated calls on one stream, a call large enough to outgrow the block (a new block), calls of
another shape in between, and calls on a second stream.
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


def scan(g):
    y, last = ssm.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["dt_bias"])
    return y, last


def noalloc(g):
    b, d, L = g["u"].shape
    n = g["A"].shape[1]
    y = torch.empty_like(g["u"])
    last = torch.empty((b, d, n), dtype=torch.float32, device="cuda")
    p = lambda t: None if t is None else t.data_ptr()
    rc = ssm.selective_scan_fwd_noalloc(p(g["u"]), p(g["delta"]), p(g["A"]), p(g["B"]), p(g["C"]), p(g["D"]),
                                        p(g["z"]), p(g["dt_bias"]), 1, None, p(y), p(last), b, d, n, L, ssm.BF16,
                                        torch.cuda.current_stream().cuda_stream)
    assert rc == 0, ssm.last_error()
    return y, last


def same(a, b):
    return torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_interval_control_block_across_calls_and_streams():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    small = dev(gen.random_scan_inputs(2, 10240, 16, 1000, "bf16", seed=21))
    # 16 x 5120 channels: 1280 chains x 4 scanner waves = 5120 flags, more than a new block holds
    big = dev(gen.random_scan_inputs(16, 5120, 16, 136, "bf16", seed=22))
    for x in (small, big):
        b, d, n, L = x["batch"], x["dim"], x["dstate"], x["seqlen"]
        assert ssm.scan_plan(b, d, n, L, torch.bfloat16, cus)["mode"] == "intervals"
    ssm.handover_failures(reset=True)
    note("interval control block: small x3, big, small x3, second stream x3")
    ref = scan(small)
    ref_big = noalloc(big)
    torch.cuda.synchronize()
    assert same(ref, noalloc(small))
    for _ in range(2):
        assert same(scan(small), ref)
    got_big = scan(big)  # outgrows the stream's block: a new one
    for _ in range(3):
        assert same(scan(small), ref)
    assert same(got_big, ref_big)
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        outs = [scan(small) for _ in range(3)]
    s2.synchronize()
    for o in outs:
        assert same(o, ref)
    torch.cuda.synchronize()
    assert ssm.handover_failures(reset=True) == 0


def test_release_stream_then_calls_remake_what_they_need():
    """ssm_release_stream frees the stream's scratch and control block after its queued work; the
    calls after it make them again and give the same bits (the interval plan and the two-pass plan,
    on a side stream and on the current one)."""
    note("release the per-stream scratch and control block")
    g = dev(gen.random_scan_inputs(4, 5120, 16, 256, "bf16", seed=31))     # interval plan
    g2 = dev(gen.random_scan_inputs(1, 64, 16, 65536, "f32", seed=32))     # two-pass plan
    s = torch.cuda.Stream()
    for stream in (s, torch.cuda.current_stream()):
        with torch.cuda.stream(stream):
            r1, q1 = scan(g), scan(g2)
            ssm.release_stream(stream)
            r2, q2 = scan(g), scan(g2)
            ssm.release_stream(stream)
            r3 = scan(g)
        torch.cuda.synchronize()
        assert same(r1, r2) and same(r1, r3)
        assert torch.equal(q1[0], q2[0]) and torch.equal(q1[1], q2[1])
