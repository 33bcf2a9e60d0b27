"""MI355X-native selective state-space (Mamba S6) scan -- Python binding.

A thin ctypes layer over the C ABI in ``include/ssm_scan.h`` (library
``libssm_scan.so``, built in-tree by ``selective_scan_02_amd.build``).  Every step
of the computation runs in the library's HIP kernels; this module only checks
tensor shapes, allocates outputs with torch and passes device pointers and the
current HIP stream.  There is no CPU fallback: without the built library or a
GPU these functions raise.

    y, last_state = scan_fwd(u, delta, A, B, C, D, z, dt_bias, softplus=True)
    y = state_update(state, u, delta, A, B, C, D, z, dt_bias)   # state updated in place
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["load", "lib_path", "scan_fwd", "scan_bwd", "ssd_fwd", "ssd_bwd", "state_update", "conv1d_fwd", "conv1d_update", "scan_plan", "SsmError",
           "STATUS", "scan_fwd_conv", "selective_scan_fwd", "selective_scan_fwd_resume", "selective_scan_fwd_noalloc",
           "selective_scan_fwd_conv", "selective_scan_bwd", "ssd_scan_fwd", "ssd_scan_bwd", "selective_state_update",
           "causal_conv1d_fwd",
           "causal_conv1d_update", "last_error", "handover_failures", "set_handover_wait"]

_PKG = os.path.dirname(os.path.abspath(__file__))
# SSM_SCAN_LIB names another build of the same library (the host-sanitizer build of the tests)
_LIB = os.environ.get("SSM_SCAN_LIB") or os.path.join(_PKG, "libssm_scan.so")
_lib = None

STATUS = {0: "SSM_OK", -1: "SSM_ERR_NULL_ARG", -2: "SSM_ERR_BAD_SHAPE", -3: "SSM_ERR_BAD_DTYPE",
          -4: "SSM_ERR_MISALIGNED", -5: "SSM_ERR_ALIAS", -6: "SSM_ERR_UNSUPPORTED", -7: "SSM_ERR_HIP"}
F32, BF16 = 0, 1
EXPORTS = ("selective_scan_fwd", "selective_scan_fwd_resume", "selective_scan_fwd_noalloc", "selective_scan_fwd_conv",
           "selective_scan_bwd",
           "ssd_scan_fwd", "ssd_scan_bwd",
           "selective_state_update", "causal_conv1d_fwd",
           "causal_conv1d_update", "ssm_scan_plan", "ssm_handover_failures", "ssm_test_handover_wait",
           "ssm_release_stream", "ssm_last_error", "ssm_abi_version")


class SsmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def lib_path() -> str:
    return _LIB


def load():
    """Load libssm_scan.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is not built; run `python -m selective_scan_02_amd.build`")
        lib = ctypes.CDLL(_LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.selective_scan_fwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, I64, I64, I64, I64, I, P]
        lib.selective_scan_fwd.restype = I
        lib.selective_scan_fwd_resume.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, I64, I64, I64, I64, I, P]
        lib.selective_scan_fwd_resume.restype = I
        lib.selective_scan_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, I64, I64, I64, I64, I, P]
        lib.selective_scan_fwd_noalloc.restype = I
        lib.selective_scan_fwd_conv.argtypes = [P, P, P, P, P, I64, P, P, P, P, P, P, P, I, P, P, P, I64, I64,
                                                I64, I64, I, P]
        lib.selective_scan_fwd_conv.restype = I
        lib.selective_scan_bwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, P, P, P, P, P, P, P, P, I64, I64,
                                           I64, I64, I, P]
        lib.selective_scan_bwd.restype = I
        lib.ssd_scan_fwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, I64, I64, I64, I64, I64, I, P]
        lib.ssd_scan_bwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, P, P, P, P, P, P, P, P, I64, I64, I64,
                                     I64, I64, I, P]
        lib.ssd_scan_bwd.restype = I
        lib.ssd_scan_fwd.restype = I
        lib.selective_state_update.argtypes = [P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I, P]
        lib.selective_state_update.restype = I
        lib.causal_conv1d_fwd.argtypes = [P, P, P, P, I, P, P, I64, I64, I64, I64, I, P]
        lib.causal_conv1d_fwd.restype = I
        lib.causal_conv1d_update.argtypes = [P, P, P, P, I, P, I64, I64, I64, I, P]
        lib.causal_conv1d_update.restype = I
        lib.ssm_last_error.argtypes = []
        lib.ssm_last_error.restype = ctypes.c_char_p
        lib.ssm_abi_version.argtypes = []
        lib.ssm_abi_version.restype = I
        lib.ssm_scan_plan.argtypes = [I64, I64, I64, I64, I, I, ctypes.POINTER(ctypes.c_int64)]
        lib.ssm_scan_plan.restype = I
        lib.ssm_handover_failures.argtypes = [ctypes.POINTER(ctypes.c_int64), I]
        lib.ssm_handover_failures.restype = I
        lib.ssm_test_handover_wait.argtypes = [I, I]
        lib.ssm_test_handover_wait.restype = I
        lib.ssm_release_stream.argtypes = [P]
        lib.ssm_release_stream.restype = I
        _lib = lib
    return _lib


PLAN_MODES = {0: "intervals", 1: "single", 2: "two-pass", 3: "generic"}


def scan_plan(batch: int, dim: int, dstate: int, seqlen: int, dtype=torch.bfloat16, num_cus: int = 256) -> dict:
    """The launch plan selective_scan_fwd uses for these sizes (host-only, no GPU)."""
    out = (ctypes.c_int64 * 5)()
    code = BF16 if dtype in (torch.bfloat16, "bf16", BF16) else F32
    _check(load().ssm_scan_plan(batch, dim, dstate, seqlen, code, num_cus, out))
    return {"mode": PLAN_MODES[out[0]], "groups": out[1], "segments": out[2], "seg_len": out[3], "units": out[4]}


def release_stream(stream=None) -> None:
    """Free the scratch and control block the library keeps for `stream` (a torch stream, or None
    for torch's current stream) on the current device, after the work queued on it."""
    s = torch.cuda.current_stream() if stream is None else stream
    _check(load().ssm_release_stream(ctypes.c_void_p(s.cuda_stream)))


def handover_failures(reset: bool = False) -> int:
    """Interval hand-over waits that gave up on the current device (their pieces are NaN)."""
    v = ctypes.c_int64(0)
    _check(load().ssm_handover_failures(ctypes.byref(v), 1 if reset else 0))
    return int(v.value)


def set_handover_wait(max_polls: int = 0, publish: bool = True) -> None:
    """Test hook: bound the hand-over wait and optionally suppress the flags (see the header)."""
    _check(load().ssm_test_handover_wait(int(max_polls), 1 if publish else 0))


def last_error() -> str:
    return load().ssm_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise SsmError(rc, last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"u must be float32 or bfloat16, got {t.dtype}")


def _require(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on {device} (a GPU tensor)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# Raw C-ABI calls (device pointers as ints), used by the tests of the boundary.
def selective_scan_fwd(*args) -> int:
    return int(load().selective_scan_fwd(*args))


def selective_scan_fwd_resume(*args) -> int:
    return int(load().selective_scan_fwd_resume(*args))


def selective_scan_fwd_noalloc(*args) -> int:
    return int(load().selective_scan_fwd_noalloc(*args))


def selective_scan_fwd_conv(*args) -> int:
    return int(load().selective_scan_fwd_conv(*args))


def selective_scan_bwd(*args) -> int:
    return int(load().selective_scan_bwd(*args))


def ssd_scan_fwd(*args) -> int:
    return int(load().ssd_scan_fwd(*args))


def ssd_scan_bwd(*args) -> int:
    return int(load().ssd_scan_bwd(*args))


def selective_state_update(*args) -> int:
    return int(load().selective_state_update(*args))


def causal_conv1d_fwd(*args) -> int:
    return int(load().causal_conv1d_fwd(*args))


def causal_conv1d_update(*args) -> int:
    return int(load().causal_conv1d_update(*args))


def scan_fwd(u, delta, A, B, C, D=None, z=None, dt_bias=None, softplus: bool = True,
             return_last_state: bool = True, y=None, last_state=None, initial_state=None):
    """Forward selective scan.  u, delta, z: [batch, dim, L]; B, C: [batch, N, L]
    (dtype of u); A: [dim, N] fp32; D, dt_bias: [dim] fp32.  Returns (y, last_state).
    ``initial_state`` [batch, dim, N] fp32 resumes the scan from that state (it may be
    passed as ``last_state`` too, to advance it in place)."""
    lib = load()
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [batch, dim, seqlen] and A [dim, dstate]")
    batch, dim, L = u.shape
    N = A.shape[1]
    dev = u.device
    dt = u.dtype
    _require(u, "u", (batch, dim, L), dt, dev)
    _require(delta, "delta", (batch, dim, L), dt, dev)
    _require(z, "z", (batch, dim, L), dt, dev)
    _require(B, "B", (batch, N, L), dt, dev)
    _require(C, "C", (batch, N, L), dt, dev)
    _require(A, "A", (dim, N), torch.float32, dev)
    _require(D, "D", (dim,), torch.float32, dev)
    _require(dt_bias, "dt_bias", (dim,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(u)
    _require(y, "y", (batch, dim, L), dt, dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    if last_state is not None:
        _require(last_state, "last_state", (batch, dim, N), torch.float32, dev)
    if initial_state is not None:
        _require(initial_state, "initial_state", (batch, dim, N), torch.float32, dev)
        rc = lib.selective_scan_fwd_resume(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                           _ptr(dt_bias), 1 if softplus else 0, _ptr(initial_state), _ptr(y),
                                           _ptr(last_state), batch, dim, N, L, _dtype_code(u), _stream(dev))
    else:
        rc = lib.selective_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                    _ptr(dt_bias), 1 if softplus else 0, _ptr(y), _ptr(last_state), batch, dim, N,
                                    L, _dtype_code(u), _stream(dev))
    _check(rc)
    return y, last_state


def scan_fwd_conv(x, conv_weight, delta, A, B, C, D=None, z=None, dt_bias=None, softplus: bool = True,
                  conv_bias=None, conv_state=None, return_conv_state: bool = True, initial_state=None,
                  return_last_state: bool = True, y=None, last_state=None, conv_state_out=None):
    """Causal conv1d + SiLU fused ahead of the forward scan: u = silu(conv(x)) is computed inside
    the scan kernels.  x, delta, z: [batch, dim, L]; conv_weight [dim, K] fp32 (K <= 4); conv_bias
    [dim]; conv_state [batch, dim, K-1] fp32 (inputs before step 0).  Returns
    (y, last_state, conv_state_out)."""
    lib = load()
    if x.dim() != 3 or A.dim() != 2 or conv_weight.dim() != 2:
        raise ValueError("x must be [batch, dim, seqlen], A [dim, dstate], conv_weight [dim, width]")
    batch, dim, L = x.shape
    N = A.shape[1]
    K = conv_weight.shape[1]
    dev, dt = x.device, x.dtype
    for t, name, shape in ((x, "x", (batch, dim, L)), (delta, "delta", (batch, dim, L)), (z, "z", (batch, dim, L)),
                           (B, "B", (batch, N, L)), (C, "C", (batch, N, L))):
        _require(t, name, shape, dt, dev)
    _require(A, "A", (dim, N), torch.float32, dev)
    _require(D, "D", (dim,), torch.float32, dev)
    _require(dt_bias, "dt_bias", (dim,), torch.float32, dev)
    _require(conv_weight, "conv_weight", (dim, K), torch.float32, dev)
    _require(conv_bias, "conv_bias", (dim,), torch.float32, dev)
    _require(conv_state, "conv_state", (batch, dim, K - 1), torch.float32, dev)
    _require(initial_state, "initial_state", (batch, dim, N), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    _require(y, "y", (batch, dim, L), dt, dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _require(last_state, "last_state", (batch, dim, N), torch.float32, dev)
    if return_conv_state and conv_state_out is None and K > 1:
        conv_state_out = torch.empty((batch, dim, K - 1), dtype=torch.float32, device=dev)
    _require(conv_state_out, "conv_state_out", (batch, dim, K - 1), torch.float32, dev)
    _check(lib.selective_scan_fwd_conv(_ptr(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state),
                                       _ptr(conv_state_out), K, _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                       _ptr(z), _ptr(dt_bias), 1 if softplus else 0, _ptr(initial_state), _ptr(y),
                                       _ptr(last_state), batch, dim, N, L, _dtype_code(x), _stream(dev)))
    return y, last_state, conv_state_out


def scan_bwd(u, delta, A, B, C, D=None, z=None, dt_bias=None, softplus: bool = True, dy=None,
             initial_state=None, need_dD: bool = True, need_ddt_bias: bool = True,
             need_dinitial_state: bool = True) -> dict:
    """Gradients of sum(dy * y) for the forward scan with the same inputs (states are
    recomputed).  Returns a dict: du, ddelta, dz (None without z) [batch, dim, L] and dB, dC
    [batch, N, L] in the dtype of u; dA [dim, N], dD, ddt_bias [dim] and dinitial_state
    [batch, dim, N] in fp32 (None when not requested)."""
    lib = load()
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [batch, dim, seqlen] and A [dim, dstate]")
    batch, dim, L = u.shape
    N = A.shape[1]
    dev = u.device
    dt = u.dtype
    for t, name, shape in ((u, "u", (batch, dim, L)), (delta, "delta", (batch, dim, L)), (z, "z", (batch, dim, L)),
                           (dy, "dy", (batch, dim, L)), (B, "B", (batch, N, L)), (C, "C", (batch, N, L))):
        _require(t, name, shape, dt, dev)
    if dy is None:
        raise ValueError("dy is required")
    _require(A, "A", (dim, N), torch.float32, dev)
    _require(D, "D", (dim,), torch.float32, dev)
    _require(dt_bias, "dt_bias", (dim,), torch.float32, dev)
    _require(initial_state, "initial_state", (batch, dim, N), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u), "dz": torch.empty_like(u) if z is not None else None,
         "dA": torch.empty((dim, N), **f32), "dB": torch.empty_like(B), "dC": torch.empty_like(C),
         "dD": torch.empty((dim,), **f32) if need_dD else None,
         "ddt_bias": torch.empty((dim,), **f32) if need_ddt_bias else None,
         "dinitial_state": torch.empty((batch, dim, N), **f32) if need_dinitial_state else None}
    _check(lib.selective_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                                  1 if softplus else 0, _ptr(initial_state), _ptr(dy), _ptr(g["du"]),
                                  _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
                                  _ptr(g["dz"]), _ptr(g["ddt_bias"]), _ptr(g["dinitial_state"]), batch, dim, N, L,
                                  _dtype_code(u), _stream(dev)))
    return g


def ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus: bool = True, initial_state=None,
            return_last_state: bool = True, y=None, last_state=None, headdim: int = 64):
    """Mamba-2 SSD scan (scalar decay per head) on the matrix cores.  x, z: [batch, H*P, L];
    dt: [batch, H, L]; B, C: [batch, N, L] (bf16); A, dt_bias: [H] fp32; D: [H*P] fp32.
    Returns (y, last_state)."""
    lib = load()
    if x.dim() != 3 or A.dim() != 1:
        raise ValueError("x must be [batch, heads*headdim, seqlen] and A [heads]")
    batch, dim, L = x.shape
    H = A.shape[0]
    if H * headdim != dim:
        raise ValueError(f"x has {dim} channels, not heads*headdim = {H}*{headdim}")
    N = B.shape[1]
    dev, dtp = x.device, x.dtype
    _require(x, "x", (batch, dim, L), dtp, dev)
    _require(dt, "dt", (batch, H, L), dtp, dev)
    _require(z, "z", (batch, dim, L), dtp, dev)
    _require(B, "B", (batch, N, L), dtp, dev)
    _require(C, "C", (batch, N, L), dtp, dev)
    _require(A, "A", (H,), torch.float32, dev)
    _require(D, "D", (dim,), torch.float32, dev)
    _require(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _require(initial_state, "initial_state", (batch, dim, N), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    _require(y, "y", (batch, dim, L), dtp, dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _require(last_state, "last_state", (batch, dim, N), torch.float32, dev)
    _check(lib.ssd_scan_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                            1 if softplus else 0, _ptr(initial_state), _ptr(y), _ptr(last_state), batch, H,
                            headdim, N, L, _dtype_code(x), _stream(dev)))
    return y, last_state


def ssd_bwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus: bool = True, dy=None, initial_state=None,
            headdim: int = 64, need_dD: bool = True, need_ddt_bias: bool = True,
            need_dinitial_state: bool = True) -> dict:
    """Gradients of sum(dy * y) for the SSD scan with the same inputs.  Returns a dict: dx, dz
    (None without z) [batch, H*P, L], ddt [batch, H, L] and dB, dC [batch, N, L] in the dtype of
    x; dA, ddt_bias [H], dD [H*P] and dinitial_state [batch, H*P, N] in fp32 (None when not
    requested)."""
    lib = load()
    if x.dim() != 3 or A.dim() != 1:
        raise ValueError("x must be [batch, heads*headdim, seqlen] and A [heads]")
    batch, dim, L = x.shape
    H = A.shape[0]
    if H * headdim != dim:
        raise ValueError(f"x has {dim} channels, not heads*headdim = {H}*{headdim}")
    N = B.shape[1]
    dev, dtp = x.device, x.dtype
    if dy is None:
        raise ValueError("dy is required")
    for t, name, shape in ((x, "x", (batch, dim, L)), (dt, "dt", (batch, H, L)), (z, "z", (batch, dim, L)),
                           (dy, "dy", (batch, dim, L)), (B, "B", (batch, N, L)), (C, "C", (batch, N, L))):
        _require(t, name, shape, dtp, dev)
    _require(A, "A", (H,), torch.float32, dev)
    _require(D, "D", (dim,), torch.float32, dev)
    _require(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _require(initial_state, "initial_state", (batch, dim, N), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt), "dz": torch.empty_like(x) if z is not None else None,
         "dA": torch.empty((H,), **f32), "dB": torch.empty_like(B), "dC": torch.empty_like(C),
         "dD": torch.empty((dim,), **f32) if need_dD else None,
         "ddt_bias": torch.empty((H,), **f32) if need_ddt_bias else None,
         "dinitial_state": torch.empty((batch, dim, N), **f32) if need_dinitial_state else None}
    _check(lib.ssd_scan_bwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                            1 if softplus else 0, _ptr(initial_state), _ptr(dy), _ptr(g["dx"]), _ptr(g["ddt"]),
                            _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
                            _ptr(g["ddt_bias"]), _ptr(g["dinitial_state"]), batch, H, headdim, N, L,
                            _dtype_code(x), _stream(dev)))
    return g


def state_update(state, u, delta, A, B, C, D=None, z=None, dt_bias=None, y=None):
    """One decode step; ``state`` [batch, dim, N] fp32 is updated in place.
    u, delta, z: [batch, dim]; B, C: [batch, N] (dtype of u).  Returns y [batch, dim]."""
    lib = load()
    if u.dim() != 2 or state.dim() != 3:
        raise ValueError("u must be [batch, dim] and state [batch, dim, dstate]")
    batch, dim = u.shape
    N = state.shape[2]
    dev = u.device
    dt = u.dtype
    _require(state, "state", (batch, dim, N), torch.float32, dev)
    _require(u, "u", (batch, dim), dt, dev)
    _require(delta, "delta", (batch, dim), dt, dev)
    _require(z, "z", (batch, dim), dt, dev)
    _require(B, "B", (batch, N), dt, dev)
    _require(C, "C", (batch, N), dt, dev)
    _require(A, "A", (dim, N), torch.float32, dev)
    _require(D, "D", (dim,), torch.float32, dev)
    _require(dt_bias, "dt_bias", (dim,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(u)
    _require(y, "y", (batch, dim), dt, dev)
    rc = lib.selective_state_update(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                    _ptr(z), _ptr(dt_bias), _ptr(y), batch, dim, N, _dtype_code(u),
                                    _stream(dev))
    _check(rc)
    return y


def conv1d_fwd(x, weight, bias=None, silu: bool = True, state=None, return_state: bool = True, out=None,
               state_out=None):
    """Causal depthwise conv1d (+ SiLU).  x: [batch, dim, L] (fp32 or bf16); weight: [dim, K]
    fp32 (K <= 4); bias: [dim] fp32; state: [batch, dim, K-1] fp32 inputs before step 0.
    Returns (out, state_out) -- state_out holds the last K-1 inputs."""
    lib = load()
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be [batch, dim, seqlen] and weight [dim, width]")
    batch, dim, L = x.shape
    K = weight.shape[1]
    dev = x.device
    _require(x, "x", (batch, dim, L), x.dtype, dev)
    _require(weight, "weight", (dim, K), torch.float32, dev)
    _require(bias, "bias", (dim,), torch.float32, dev)
    _require(state, "state", (batch, dim, K - 1), torch.float32, dev)
    if out is None:
        out = torch.empty_like(x)
    _require(out, "out", (batch, dim, L), x.dtype, dev)
    if return_state and state_out is None:
        state_out = torch.empty((batch, dim, K - 1), dtype=torch.float32, device=dev)
    _require(state_out, "state_out", (batch, dim, K - 1), torch.float32, dev)
    _check(lib.causal_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(state), 1 if silu else 0, _ptr(out),
                                 _ptr(state_out), batch, dim, L, K, _dtype_code(x), _stream(dev)))
    return out, state_out


def conv1d_update(state, x, weight, bias=None, silu: bool = True, out=None):
    """One decode step of the conv; ``state`` [batch, dim, K-1] fp32 is advanced in place.
    x: [batch, dim].  Returns out [batch, dim]."""
    lib = load()
    if x.dim() != 2 or weight.dim() != 2:
        raise ValueError("x must be [batch, dim] and weight [dim, width]")
    batch, dim = x.shape
    K = weight.shape[1]
    dev = x.device
    _require(state, "state", (batch, dim, K - 1), torch.float32, dev)
    _require(x, "x", (batch, dim), x.dtype, dev)
    _require(weight, "weight", (dim, K), torch.float32, dev)
    _require(bias, "bias", (dim,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(x)
    _require(out, "out", (batch, dim), x.dtype, dev)
    _check(lib.causal_conv1d_update(_ptr(state), _ptr(x), _ptr(weight), _ptr(bias), 1 if silu else 0, _ptr(out),
                                    batch, dim, K, _dtype_code(x), _stream(dev)))
    return out
