"""C-ABI boundary tests that need no GPU.

The library must load without a device, export every function the public
header declares, and reject bad arguments on the host -- before any HIP call --
with the documented status codes.  Fake (never dereferenced) device addresses
are used: a rejected call touches nothing.
"""
import ctypes
import os
import re

import pytest

import selective_scan_02_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

NULL_ARG, BAD_SHAPE, BAD_DTYPE, MISALIGNED, ALIAS, UNSUPPORTED = -1, -2, -3, -4, -5, -6

# Fake 256-byte-aligned device addresses, far apart (1 TiB) so nothing overlaps by accident.
BASE = 1 << 44
def addr(i):
    return BASE + (i << 40)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssm.lib_path()):
        import selective_scan_02_amd.build as b
        b.build()
    return ssm.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for name in ("selective_scan_fwd", "selective_scan_fwd_resume", "selective_scan_fwd_noalloc",
                 "selective_scan_fwd_conv",
                 "selective_scan_bwd", "ssd_scan_fwd", "ssd_scan_bwd",
                 "selective_state_update",
                 "causal_conv1d_fwd",
                 "causal_conv1d_update", "ssm_scan_plan", "ssm_handover_failures", "ssm_test_handover_wait",
                 "ssm_release_stream", "ssm_last_error", "ssm_abi_version"):
        assert name in fns
    assert set(fns) == set(ssm.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version(lib):
    assert lib.ssm_abi_version() == 10


def scan_args(**over):
    a = dict(u=addr(1), delta=addr(2), A=addr(3), B=addr(4), C=addr(5), D=addr(6), z=addr(7), dt_bias=addr(8),
             softplus=1, y=addr(9), last=addr(10), batch=2, dim=64, dstate=16, seqlen=128, dtype=1, stream=None)
    a.update(over)
    return [a[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "dt_bias", "softplus", "y", "last", "batch", "dim",
                           "dstate", "seqlen", "dtype", "stream")]


def resume_args(h0=addr(11), **over):
    a = scan_args(**over)
    return a[:9] + [h0] + a[9:]


def step_args(**over):
    a = dict(state=addr(1), u=addr(2), delta=addr(3), A=addr(4), B=addr(5), C=addr(6), D=addr(7), z=addr(8),
             dt_bias=addr(9), y=addr(10), batch=4, dim=64, dstate=16, dtype=1, stream=None)
    a.update(over)
    return [a[k] for k in ("state", "u", "delta", "A", "B", "C", "D", "z", "dt_bias", "y", "batch", "dim", "dstate",
                           "dtype", "stream")]


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "y"])
def test_scan_null_required(lib, field):
    assert lib.selective_scan_fwd(*scan_args(**{field: None})) == NULL_ARG
    assert field in ssm.last_error()


@pytest.mark.parametrize("field", ["state", "u", "delta", "A", "B", "C", "y"])
def test_step_null_required(lib, field):
    assert lib.selective_state_update(*step_args(**{field: None})) == NULL_ARG


@pytest.mark.parametrize("over", [dict(batch=0), dict(dim=0), dict(dstate=0), dict(seqlen=-1), dict(batch=-3),
                                  dict(batch=1 << 20, dim=1 << 20, seqlen=1 << 20), dict(softplus=2)])
def test_scan_bad_shape(lib, over):
    assert lib.selective_scan_fwd(*scan_args(**over)) == BAD_SHAPE


def test_bad_dtype(lib):
    assert lib.selective_scan_fwd(*scan_args(dtype=7)) == BAD_DTYPE
    assert lib.selective_state_update(*step_args(dtype=-1)) == BAD_DTYPE


@pytest.mark.parametrize("n", [3, 5, 12, 128, 1000])
def test_unsupported_dstate(lib, n):
    assert lib.selective_scan_fwd(*scan_args(dstate=n)) == UNSUPPORTED
    assert lib.selective_state_update(*step_args(dstate=n)) == UNSUPPORTED
    assert str(n) in ssm.last_error()


def test_misaligned(lib):
    assert lib.selective_scan_fwd(*scan_args(u=addr(1) + 1)) == MISALIGNED          # bf16 needs 2 bytes
    assert lib.selective_scan_fwd(*scan_args(dtype=0, delta=addr(2) + 2)) == MISALIGNED  # fp32 needs 4
    assert lib.selective_scan_fwd(*scan_args(A=addr(3) + 2)) == MISALIGNED
    assert lib.selective_state_update(*step_args(state=addr(1) + 4)) == MISALIGNED   # float4 state rows
    assert lib.selective_state_update(*step_args(A=addr(4) + 4)) == MISALIGNED       # float4 rows of A
    assert lib.selective_state_update(*step_args(B=addr(5) + 2)) == MISALIGNED       # 4 bf16 of B at once


def test_alias(lib):
    # y placed inside u
    assert lib.selective_scan_fwd(*scan_args(y=addr(1) + 64)) == ALIAS
    # last_state overlapping B
    assert lib.selective_scan_fwd(*scan_args(last=addr(4) + 16)) == ALIAS
    # y overlapping last_state
    assert lib.selective_scan_fwd(*scan_args(last=addr(9) + 32)) == ALIAS
    # decode: state overlapping u, y overlapping state
    assert lib.selective_state_update(*step_args(state=addr(2))) == ALIAS
    assert lib.selective_state_update(*step_args(y=addr(1) + 16)) == ALIAS
    assert "overlaps" in ssm.last_error()


def test_resume_validation(lib):
    # the resumed scan validates like the plain one, plus the initial state
    assert lib.selective_scan_fwd_resume(*resume_args(u=None)) == NULL_ARG
    assert lib.selective_scan_fwd_resume(*resume_args(dtype=5)) == BAD_DTYPE
    assert lib.selective_scan_fwd_resume(*resume_args(dstate=3)) == UNSUPPORTED
    assert lib.selective_scan_fwd_resume(*resume_args(h0=addr(11) + 2)) == MISALIGNED
    # y may not overlap the initial state; last_state may only be the very same buffer
    assert lib.selective_scan_fwd_resume(*resume_args(h0=addr(9) + 64)) == ALIAS
    assert "initial_state" in ssm.last_error()
    assert lib.selective_scan_fwd_resume(*resume_args(h0=addr(10) + 64)) == ALIAS
    assert lib.selective_scan_fwd_resume(*resume_args(h0=addr(10), last=addr(10) + 4)) == ALIAS
    # last_state overlapping the initial state only in part
    assert lib.selective_scan_fwd_resume(*resume_args(h0=addr(10), last=addr(10) - 4)) == ALIAS


def test_error_text_is_per_call(lib):
    lib.selective_scan_fwd(*scan_args(u=None))
    assert ssm.last_error()
    lib.selective_scan_fwd(*scan_args(dtype=9))
    assert "dtype" in ssm.last_error()


def test_python_wrapper_refuses_cpu_tensors(lib):
    import torch
    u = torch.zeros(1, 4, 8)
    with pytest.raises((ValueError, TypeError)):
        ssm.scan_fwd(u, u, torch.zeros(4, 4), torch.zeros(1, 4, 8), torch.zeros(1, 4, 8))


def test_empty_sequence_allows_null_sequence_tensors(lib):
    # seqlen == 0: u, delta, B, C, y are empty and may be NULL; A is still required
    assert lib.selective_scan_fwd(*scan_args(seqlen=0, A=None, u=None)) == NULL_ARG
    assert "A" in ssm.last_error()


def test_scan_plan_workloads(lib):
    # 2.8B-shaped layer: 320 channel groups of 128 chunks on 256 CUs -> 256 intervals of 160 chunks
    p = ssm.scan_plan(4, 5120, 16, 2048)
    assert p == {"mode": "intervals", "groups": 320, "segments": 256, "seg_len": 2560, "units": 256}
    # 130M-shaped layer: 192 groups < 256 CUs -> one pass per group
    p = ssm.scan_plan(8, 1536, 16, 2048)
    assert p["mode"] == "single" and p["groups"] == 192 and p["segments"] == 1
    # 1M-step DNA-like scan: 4 groups -> aggregate pass over ~8 segments per CU, carry, and an
    # output pass of one workgroup per CU, each through several segments
    p = ssm.scan_plan(1, 256, 16, 1 << 20, torch_dtype_f32())
    assert p["mode"] == "two-pass" and p["groups"] == 4 and p["segments"] >= 512 and p["units"] == 256
    assert p["seg_len"] % 16 == 0 and p["segments"] * p["seg_len"] >= 1 << 20
    # tiny fp32 workload: one group, short -> two-pass over a few segments
    p = ssm.scan_plan(1, 16, 4, 64, torch_dtype_f32())
    assert p["groups"] == 1 and p["segments"] * p["seg_len"] >= 64
    # generic kernels: dstate < 4, or rows that are not whole 16-byte pieces
    assert ssm.scan_plan(1, 64, 2, 256)["mode"] == "generic"
    assert ssm.scan_plan(1, 64, 16, 777)["mode"] == "generic"


def test_scan_plan_intervals_cover_and_balance(lib):
    # intervals: every workgroup but the last gets the same number of chunks, the intervals
    # cover all chains exactly, and an interval is at least one chain long (a chain is split
    # at most once, and a tail piece starts no earlier than the head it continues ends)
    for b, d, L in [(4, 5120, 2048), (2, 10240, 1000), (1, 20480, 512), (8, 5120, 4096), (4, 4096, 2048),
                    (1, 64 * 257, 2048), (8, 5120, 512)]:
        p = ssm.scan_plan(b, d, 16, L)
        chunks = -(-L // 16)
        total = p["groups"] * chunks
        w = p["seg_len"] // 16
        assert p["mode"] == "intervals" and p["seg_len"] % 16 == 0
        assert p["units"] == -(-total // w) and (p["units"] - 1) * w < total <= p["units"] * w
        assert w >= chunks and p["units"] <= 256


def torch_dtype_f32():
    import torch
    return torch.float32


def conv_args(**over):
    a = dict(x=addr(1), w=addr(2), bias=addr(3), st_in=addr(4), silu=1, out=addr(5), st_out=addr(6), batch=2,
             dim=64, seqlen=100, width=4, dtype=1, stream=None)
    a.update(over)
    return [a[k] for k in ("x", "w", "bias", "st_in", "silu", "out", "st_out", "batch", "dim", "seqlen", "width",
                           "dtype", "stream")]


def conv_step_args(**over):
    a = dict(state=addr(1), x=addr(2), w=addr(3), bias=addr(4), silu=1, out=addr(5), batch=2, dim=64, width=4,
             dtype=1, stream=None)
    a.update(over)
    return [a[k] for k in ("state", "x", "w", "bias", "silu", "out", "batch", "dim", "width", "dtype", "stream")]


def test_conv_validation(lib):
    f, u = lib.causal_conv1d_fwd, lib.causal_conv1d_update
    assert f(*conv_args(x=None)) == NULL_ARG
    assert f(*conv_args(w=None)) == NULL_ARG
    assert f(*conv_args(out=None)) == NULL_ARG
    assert f(*conv_args(seqlen=0, x=None, out=None, w=None)) == NULL_ARG  # weight still required
    assert f(*conv_args(width=5)) == UNSUPPORTED and "width" in ssm.last_error()
    assert f(*conv_args(width=0)) == BAD_SHAPE
    assert f(*conv_args(silu=3)) == BAD_SHAPE
    assert f(*conv_args(dtype=4)) == BAD_DTYPE
    assert f(*conv_args(x=addr(1) + 1)) == MISALIGNED
    assert f(*conv_args(out=addr(1) + 64)) == ALIAS                 # out inside x
    assert f(*conv_args(st_out=addr(4) + 8)) == ALIAS               # state out overlapping state in
    assert f(*conv_args(st_out=addr(4))) == ALIAS and "conv_state_out" in ssm.last_error()
    assert u(*conv_step_args(state=None)) == NULL_ARG
    assert u(*conv_step_args(x=None)) == NULL_ARG
    assert u(*conv_step_args(width=7)) == UNSUPPORTED
    assert u(*conv_step_args(out=addr(1) + 4)) == ALIAS             # out inside the state
    assert u(*conv_step_args(state=addr(3))) == ALIAS               # state overlapping the weights


BWD_FIELDS = ("u", "delta", "A", "B", "C", "D", "z", "dt_bias", "softplus", "h0", "dy", "du", "ddelta", "dA", "dB",
              "dC", "dD", "dz", "ddt_bias", "dh0", "batch", "dim", "dstate", "seqlen", "dtype", "stream")


def bwd_args(**over):
    a = dict(zip(BWD_FIELDS[:8], [addr(i) for i in range(1, 9)]))
    a.update(softplus=1, h0=addr(9), dy=addr(10), du=addr(11), ddelta=addr(12), dA=addr(13), dB=addr(14),
             dC=addr(15), dD=addr(16), dz=addr(17), ddt_bias=addr(18), dh0=addr(19), batch=2, dim=64, dstate=16,
             seqlen=128, dtype=1, stream=None)
    a.update(over)
    return [a[k] for k in BWD_FIELDS]


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "dy", "du", "ddelta", "dA", "dB", "dC", "dz"])
def test_bwd_null_required(lib, field):
    assert lib.selective_scan_bwd(*bwd_args(**{field: None})) == NULL_ARG
    assert field in ssm.last_error()


def test_bwd_validation(lib):
    assert lib.selective_scan_bwd(*bwd_args(dtype=3)) == BAD_DTYPE
    assert lib.selective_scan_bwd(*bwd_args(dstate=12)) == UNSUPPORTED
    assert lib.selective_scan_bwd(*bwd_args(batch=0)) == BAD_SHAPE
    assert lib.selective_scan_bwd(*bwd_args(softplus=5)) == BAD_SHAPE
    assert lib.selective_scan_bwd(*bwd_args(dy=addr(10) + 1)) == MISALIGNED
    assert lib.selective_scan_bwd(*bwd_args(dA=addr(13) + 2)) == MISALIGNED
    # outputs may overlap neither an input nor each other
    assert lib.selective_scan_bwd(*bwd_args(du=addr(10) + 64)) == ALIAS
    assert lib.selective_scan_bwd(*bwd_args(dC=addr(14) + 64)) == ALIAS
    assert lib.selective_scan_bwd(*bwd_args(dh0=addr(9))) == ALIAS
    assert lib.selective_scan_bwd(*bwd_args(dD=addr(13) + 4)) == ALIAS
    assert "overlaps" in ssm.last_error()


SSD_FIELDS = ("x", "dt", "A", "B", "C", "D", "z", "dt_bias", "softplus", "h0", "y", "last", "batch", "heads",
              "headdim", "dstate", "seqlen", "dtype", "stream")


def ssd_args(**over):
    a = dict(zip(SSD_FIELDS[:8], [addr(i) for i in range(1, 9)]))
    a.update(softplus=1, h0=addr(9), y=addr(10), last=addr(11), batch=2, heads=4, headdim=64, dstate=16,
             seqlen=256, dtype=1, stream=None)
    a.update(over)
    return [a[k] for k in SSD_FIELDS]


def test_ssd_validation(lib):
    for f in ("x", "dt", "A", "B", "C", "y"):
        assert lib.ssd_scan_fwd(*ssd_args(**{f: None})) == NULL_ARG, f
    assert lib.ssd_scan_fwd(*ssd_args(dtype=0)) == UNSUPPORTED          # bf16 only
    assert lib.ssd_scan_fwd(*ssd_args(headdim=48)) == UNSUPPORTED      # heads of 32, 64 or 128 channels
    assert lib.ssd_scan_fwd(*ssd_args(headdim=16)) == UNSUPPORTED
    assert lib.ssd_scan_fwd(*ssd_args(headdim=128, dstate=64)) == UNSUPPORTED
    assert lib.ssd_scan_fwd(*ssd_args(dstate=8)) == UNSUPPORTED
    assert lib.ssd_scan_fwd(*ssd_args(seqlen=100)) == UNSUPPORTED       # not a multiple of 8
    assert lib.ssd_scan_fwd(*ssd_args(batch=0)) == BAD_SHAPE
    assert lib.ssd_scan_fwd(*ssd_args(x=addr(1) + 8)) == MISALIGNED     # 16-byte rows
    assert lib.ssd_scan_fwd(*ssd_args(y=addr(1) + 64)) == ALIAS
    assert lib.ssd_scan_fwd(*ssd_args(last=addr(9) + 64)) == ALIAS


SSD_BWD_FIELDS = ("x", "dt", "A", "B", "C", "D", "z", "dt_bias", "softplus", "h0", "dy", "dx", "ddt", "dA", "dB",
                  "dC", "dD", "dz", "ddt_bias", "dh0", "batch", "heads", "headdim", "dstate", "seqlen", "dtype",
                  "stream")


def ssd_bwd_args(**over):
    a = dict(zip(SSD_BWD_FIELDS[:8], [addr(i) for i in range(1, 9)]))
    a.update(softplus=1, h0=addr(9), dy=addr(10), dx=addr(11), ddt=addr(12), dA=addr(13), dB=addr(14),
             dC=addr(15), dD=addr(16), dz=addr(17), ddt_bias=addr(18), dh0=addr(19), batch=2, heads=4, headdim=64,
             dstate=16, seqlen=128, dtype=1, stream=None)
    a.update(over)
    return [a[k] for k in SSD_BWD_FIELDS]


@pytest.mark.parametrize("field", ["x", "dt", "A", "B", "C", "dy", "dx", "ddt", "dA", "dB", "dC", "dz"])
def test_ssd_bwd_null_required(lib, field):
    assert lib.ssd_scan_bwd(*ssd_bwd_args(**{field: None})) == NULL_ARG
    assert field in ssm.last_error()


def test_ssd_bwd_validation(lib):
    f = lib.ssd_scan_bwd
    assert f(*ssd_bwd_args(dtype=3)) == BAD_DTYPE
    assert f(*ssd_bwd_args(dstate=12)) == UNSUPPORTED
    assert f(*ssd_bwd_args(batch=0)) == BAD_SHAPE
    assert f(*ssd_bwd_args(headdim=0)) == BAD_SHAPE
    assert f(*ssd_bwd_args(softplus=2)) == BAD_SHAPE
    assert f(*ssd_bwd_args(dy=addr(10) + 1)) == MISALIGNED
    assert f(*ssd_bwd_args(dA=addr(13) + 2)) == MISALIGNED
    assert f(*ssd_bwd_args(dx=addr(10) + 64)) == ALIAS          # dx inside dy
    assert f(*ssd_bwd_args(ddt=addr(2) + 64)) == ALIAS          # ddt inside dt
    assert f(*ssd_bwd_args(dh0=addr(9))) == ALIAS
    assert "overlaps" in ssm.last_error()
    # an empty sequence still needs A and dA; the sequence tensors may be absent
    assert f(*ssd_bwd_args(seqlen=0, dA=None)) == NULL_ARG


def test_size_limits(lib):
    # the SSD kernels put batch * heads on one launch dimension (at most 65535); the decode step
    # caps the channel count at 2^34 so that its grid of channel tiles fits
    assert lib.ssd_scan_fwd(*ssd_args(batch=65536, heads=1, seqlen=8)) == BAD_SHAPE
    assert lib.ssd_scan_fwd(*ssd_args(batch=257, heads=256, seqlen=8)) == BAD_SHAPE
    assert lib.selective_state_update(*step_args(batch=1, dim=1 << 34, dstate=1)) == BAD_SHAPE
    assert "too large" in ssm.last_error()


def test_noalloc_validation(lib):
    """The allocation-free scan validates like the resume call, and refuses on the host a plan
    whose scratch exceeds its fixed array (1 x 256 channels, dstate 64, 2^20 steps in fp32: 512
    segments of aggregates, 34 MB against 16 MiB) -- before any launch."""
    f = lib.selective_scan_fwd_noalloc
    assert f(*resume_args(u=None)) == NULL_ARG
    assert f(*resume_args(dtype=5)) == BAD_DTYPE
    assert f(*resume_args(dstate=3)) == UNSUPPORTED
    assert f(*resume_args(h0=addr(11) + 2)) == MISALIGNED
    assert f(*resume_args(h0=addr(9) + 64)) == ALIAS
    assert f(*resume_args(batch=1, dim=256, dstate=64, seqlen=1 << 20, dtype=0)) == UNSUPPORTED
    assert "scratch" in ssm.last_error()


def test_handover_diagnostics_validation(lib):
    assert lib.ssm_handover_failures(None, 0) == NULL_ARG
    assert lib.ssm_test_handover_wait(0, 1) == 0   # the normal setting, restored


def conv_scan_args(x=addr(1), w=addr(12), cb=addr(13), cst=addr(14), cso=addr(15), width=4, h0=None, **over):
    a = scan_args(**over)
    # (x, w, cb, st_in, st_out, width, delta, A, B, C, D, z, dt_bias, softplus, h0, y, last, sizes..., dtype, stream)
    return [x if "u" not in over else a[0], w, cb, cst, cso, width] + a[1:9] + [h0] + a[9:]


def test_conv_scan_validation(lib):
    f = lib.selective_scan_fwd_conv
    assert f(*conv_scan_args(w=None)) == NULL_ARG
    assert f(*conv_scan_args(x=None)) == NULL_ARG
    assert "x is NULL" in ssm.last_error()
    assert f(*conv_scan_args(width=5)) == UNSUPPORTED
    assert f(*conv_scan_args(width=0)) == UNSUPPORTED
    assert f(*conv_scan_args(dstate=3)) == UNSUPPORTED
    assert f(*conv_scan_args(w=addr(12) + 2)) == MISALIGNED
    assert f(*conv_scan_args(cso=addr(14))) == ALIAS          # state out on state in
    assert f(*conv_scan_args(cso=addr(9) + 64)) == ALIAS      # state out inside y
    assert f(*conv_scan_args(cst=addr(9))) == ALIAS            # y over the state in
