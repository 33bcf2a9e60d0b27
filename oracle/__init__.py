"""CPU fp64 oracle of the selective-SSM (S6) scan and decode step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The GPU library (``selective_scan_02_amd``) never imports,
links or calls anything here, and this package never imports the GPU library: the
two share no code.  The arithmetic lives in ``ssm_oracle.c`` (plain sequential
fp64 recurrence, see its header for the definition and the page passages it
follows); this module only builds it with gcc and marshals arguments.

Pins: ``tests/test_oracle.py`` checks this oracle against brute force (mpmath),
closed forms (LTI convolution, step response, memoryless limit), exact special
cases (Delta = 0) and invariants.  Every function here is pinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
# SSM_ORACLE_LIB names another build of the oracle (the sanitizer build of the tests)
_LIB_PATH = os.environ.get("SSM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True, out: str | None = None, sanitize: bool = False) -> str:
    """Compile ssm_oracle.c -> liboracle.so (gcc -O2 -fopenmp, IEEE: no fast-math).  With
    ``sanitize``: AddressSanitizer and UndefinedBehaviorSanitizer, at ``out``."""
    path = out or _LIB_PATH
    if force or not os.path.exists(path):
        tmp = path + ".tmp%d" % os.getpid()
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
               "-g"] if sanitize else []
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", *san, "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_scan.argtypes = [P, P, P, P, P, P, P, P, I, P, I64, I64, I64, I64, I, P, I64, P, P, I]
        lib.oracle_scan.restype = I
        lib.oracle_step.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I, P, I64, P, P, I]
        lib.oracle_step.restype = I
        lib.oracle_conv1d.argtypes = [P, P, P, P, I, I64, I64, I64, I64, I, P, P, I]
        lib.oracle_conv1d.restype = I
        lib.oracle_scan_bwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, I64, I64, I64, I64, I, P, P, P, P, P, P, P,
                                         P, P, I]
        lib.oracle_scan_bwd.restype = I
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = I
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _raw(x, keep):
    """Pointer to the exact bytes of a CPU tensor / array (fp32 or bf16), or None."""
    if x is None:
        return None, None
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            a = x.view(torch.int16).numpy()
            dt = 1
        elif x.dtype == torch.float32:
            a = x.numpy()
            dt = 0
        else:
            raise TypeError(f"oracle takes fp32 or bf16 tensors, got {x.dtype}")
    else:
        a = np.ascontiguousarray(x)
        if a.dtype == np.float32:
            dt = 0
        else:
            raise TypeError(f"oracle takes fp32 arrays, got {a.dtype}")
    keep.append(a)
    return a.ctypes.data, dt


def _f32(x, keep):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().to(torch.float32).contiguous().numpy()
    a = np.ascontiguousarray(x, dtype=np.float32)
    keep.append(a)
    return a.ctypes.data


def _chans(chans, total, keep):
    if chans is None:
        return None, total
    c = np.ascontiguousarray(np.asarray(chans, dtype=np.int64))
    if c.size and (c.min() < 0 or c.max() >= total):
        raise IndexError("channel index out of range")
    keep.append(c)
    return c.ctypes.data, int(c.size)


def scan(u, delta, A, B, C, D=None, z=None, dt_bias=None, softplus=True, h0=None, chans=None,
         threads: int = 0):
    """Sequential fp64 scan.  Shapes: u, delta, z [B,D,L]; B, C [B,N,L]; A [D,N].

    Returns (y, last_state) as float64 numpy arrays of shape [B,D,L] and [B,D,N]
    (or [k,L], [k,N] for a channel subset ``chans`` of flat indices b*D + d).
    ``h0``: optional initial state, [B,D,N] (or [k,N] with ``chans``).
    """
    keep = []
    batch, dim, seqlen = (int(s) for s in u.shape)
    dstate = int(A.shape[1])
    pu, dtype = _raw(u, keep)
    pdl, dt2 = _raw(delta, keep)
    pB, dt3 = _raw(B, keep)
    pC, dt4 = _raw(C, keep)
    pz, dt5 = _raw(z, keep)
    if len({dtype, dt2, dt3, dt4} | ({dt5} if z is not None else set())) != 1:
        raise TypeError("u, delta, B, C, z must share one dtype")
    pchans, rows = _chans(chans, batch * dim, keep)
    ph0 = None
    if h0 is not None:
        h = h0.detach().cpu().double().numpy() if isinstance(h0, torch.Tensor) else np.asarray(h0, np.float64)
        h = np.ascontiguousarray(h.reshape(rows, dstate), dtype=np.float64)
        keep.append(h)
        ph0 = h.ctypes.data
    y = np.empty((rows, seqlen), dtype=np.float64)
    last = np.empty((rows, dstate), dtype=np.float64)
    rc = _load().oracle_scan(pu, pdl, _f32(A, keep), pB, pC, _f32(D, keep), pz, _f32(dt_bias, keep),
                             1 if softplus else 0, ph0, batch, dim, dstate, seqlen, dtype, pchans, rows,
                             y.ctypes.data, last.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_scan failed ({rc})")
    if chans is None:
        return y.reshape(batch, dim, seqlen), last.reshape(batch, dim, dstate)
    return y, last


def step(state, u, delta, A, B, C, D=None, z=None, dt_bias=None, chans=None, threads: int = 0):
    """One fp64 decode step.  state [B,D,N] (any float dtype; or [k,N] with ``chans``),
    u, delta, z [B,D], B, C [B,N].  Returns (y, new_state) float64: [B,D], [B,D,N]
    (or [k], [k,N]).  Softplus is always applied."""
    keep = []
    batch, dim = (int(s) for s in u.shape)
    dstate = int(A.shape[1])
    pu, dtype = _raw(u, keep)
    pdl, dt2 = _raw(delta, keep)
    pB, dt3 = _raw(B, keep)
    pC, dt4 = _raw(C, keep)
    pz, dt5 = _raw(z, keep)
    if len({dtype, dt2, dt3, dt4} | ({dt5} if z is not None else set())) != 1:
        raise TypeError("u, delta, B, C, z must share one dtype")
    pchans, rows = _chans(chans, batch * dim, keep)
    s = state.detach().cpu().double().numpy() if isinstance(state, torch.Tensor) else np.asarray(state)
    s = np.ascontiguousarray(s.reshape(rows, dstate), dtype=np.float64)
    keep.append(s)
    y = np.empty((rows,), dtype=np.float64)
    out = np.empty((rows, dstate), dtype=np.float64)
    rc = _load().oracle_step(s.ctypes.data, pu, pdl, _f32(A, keep), pB, pC, _f32(D, keep), pz,
                             _f32(dt_bias, keep), batch, dim, dstate, dtype, pchans, rows, y.ctypes.data,
                             out.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_step failed ({rc})")
    if chans is None:
        return y.reshape(batch, dim), out.reshape(batch, dim, dstate)
    return y, out


def rel_err(got, ref) -> float:
    """Max error relative to max(|ref_i|, rms(ref)) -- the parity metric.

    Pure elementwise relative error is meaningless where a reference entry is
    near zero, so each entry's error is scaled by the larger of its own
    magnitude and the RMS of the whole reference tensor."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if r.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    rms = float(np.sqrt(np.mean(r * r)))
    floor = max(rms, np.finfo(np.float64).tiny)
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor)))


def conv1d(x, weight, bias=None, silu=True, state=None, threads: int = 0):
    """Causal depthwise conv (+ SiLU) in fp64.  x [B,D,L] (fp32 or bf16), weight [D,K],
    bias [D] fp32, state [B,D,K-1] (inputs before step 0, oldest first; None = zeros).
    Returns (out [B,D,L], state_out [B,D,K-1]) as float64 numpy arrays."""
    keep = []
    batch, dim, seqlen = (int(s) for s in x.shape)
    width = int(weight.shape[1])
    px, dtype = _raw(x, keep)
    ps = None
    if state is not None:
        st = state.detach().cpu().double().numpy() if isinstance(state, torch.Tensor) else np.asarray(state, np.float64)
        st = np.ascontiguousarray(st.reshape(batch * dim, width - 1), dtype=np.float64)
        keep.append(st)
        ps = st.ctypes.data
    out = np.empty((batch * dim, seqlen), dtype=np.float64)
    st_out = np.empty((batch * dim, max(width - 1, 1)), dtype=np.float64)
    rc = _load().oracle_conv1d(px, _f32(weight, keep), _f32(bias, keep), ps, 1 if silu else 0, batch, dim, seqlen,
                               width, dtype, out.ctypes.data, st_out.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_conv1d failed ({rc})")
    return out.reshape(batch, dim, seqlen), st_out[:, :width - 1].reshape(batch, dim, width - 1)


def scan_bwd(u, delta, A, B, C, D=None, z=None, dt_bias=None, softplus=True, h0=None, dy=None,
             threads: int = 0) -> dict:
    """Gradients of sum(dy * y) for the forward scan, fp64 (adjoint method; see ssm_oracle.c).
    Same inputs as scan() plus dy [B,D,L] (dtype of u).  Returns a dict of float64 arrays:
    du, ddelta, dz [B,D,L] (dz None without z); dB, dC [B,N,L]; dA [D,N]; dD, ddt_bias [D]
    (None when the input is absent); dh0 [B,D,N]."""
    keep = []
    batch, dim, seqlen = (int(s) for s in u.shape)
    dstate = int(A.shape[1])
    pu, dtype = _raw(u, keep)
    pdl, _ = _raw(delta, keep)
    pB, _ = _raw(B, keep)
    pC, _ = _raw(C, keep)
    pz, _ = _raw(z, keep)
    pdy, dt6 = _raw(dy, keep)
    if dt6 != dtype:
        raise TypeError("dy must have the dtype of u")
    ph0 = None
    if h0 is not None:
        h = h0.detach().cpu().double().numpy() if isinstance(h0, torch.Tensor) else np.asarray(h0, np.float64)
        h = np.ascontiguousarray(h.reshape(batch * dim, dstate), dtype=np.float64)
        keep.append(h)
        ph0 = h.ctypes.data
    out = {k: np.zeros(shape, dtype=np.float64) for k, shape in
           [("du", (batch, dim, seqlen)), ("ddelta", (batch, dim, seqlen)), ("dz", (batch, dim, seqlen)),
            ("dA", (dim, dstate)), ("dB", (batch, dstate, seqlen)), ("dC", (batch, dstate, seqlen)),
            ("dD", (dim,)), ("ddt_bias", (dim,)), ("dh0", (batch, dim, dstate))]}
    rc = _load().oracle_scan_bwd(pu, pdl, _f32(A, keep), pB, pC, _f32(D, keep), pz, _f32(dt_bias, keep),
                                 1 if softplus else 0, ph0, pdy, batch, dim, dstate, seqlen, dtype,
                                 *(out[k].ctypes.data for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD",
                                                                "ddt_bias", "dh0")), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_scan_bwd failed ({rc})")
    if z is None:
        out["dz"] = None
    if D is None:
        out["dD"] = None
    if dt_bias is None:
        out["ddt_bias"] = None
    return out


def ssd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True, headdim: int = 64, h0=None, chans=None,
        threads: int = 0):
    """Mamba-2 SSD forward (state-space duality, scalar A per head), fp64.

    The SSD layer is the selective recurrence of ``scan`` with one decay rate and one step size per
    head: every channel d of head h = d // headdim uses A[d, n] = A_heads[h] for all n and
    delta[b, d, t] = dt[b, h, t] (dt_bias likewise per head).  This function is exactly that: it
    broadcasts the per-head parameters to the channels and runs the sequential oracle.  Shapes: x, z
    [B, H*P, L]; dt [B, H, L] (dtype of x); A [H] fp32; B, C [B, N, L]; D [H*P] fp32; dt_bias [H]
    fp32.  Returns (y, last_state) like ``scan``.  Pinned by tests/test_oracle_ssd.py against the
    explicit semiseparable matrix and a chunked evaluation."""
    batch, dim, seqlen = (int(s) for s in x.shape)
    heads = int(A.shape[0])
    if heads * headdim != dim:
        raise ValueError("x's channel count must be heads * headdim")
    dstate = int(B.shape[1])
    delta = torch.as_tensor(dt).repeat_interleave(headdim, dim=1).contiguous()
    a = torch.as_tensor(A, dtype=torch.float32).repeat_interleave(headdim)[:, None].expand(dim, dstate).contiguous()
    bias = None if dt_bias is None else torch.as_tensor(dt_bias, dtype=torch.float32).repeat_interleave(headdim)
    return scan(x, delta, a, B, C, D, z, bias, softplus, h0=h0, chans=chans, threads=threads)


def ssd_bwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True, headdim: int = 64, h0=None, dy=None,
            threads: int = 0) -> dict:
    """Gradients of sum(dy * y) for the SSD forward ``ssd``, fp64.

    ``ssd`` is ``scan`` with the per-head decay and step size broadcast to the head's channels
    (A[d, n] = A_heads[d // headdim] for every n, delta[b, d, t] = dt[b, d // headdim, t], dt_bias
    likewise), so by the chain rule its gradients are those of ``scan_bwd`` on the broadcast
    problem, with the broadcast parameters' gradients summed back over what they were broadcast to:
    ddt[b, h, t] = sum over the head's channels of ddelta; dA[h] = sum over its channels and all
    states of dA; ddt_bias[h] = sum over its channels.  Shapes as for ``ssd`` plus dy [B, H*P, L]
    (dtype of x).  Returns float64 arrays: dx, dz [B, H*P, L] (dz None without z); ddt [B, H, L];
    dA [H]; dB, dC [B, N, L]; dD [H*P] (None without D); ddt_bias [H] (None without dt_bias);
    dh0 [B, H*P, N].  Pinned by tests/test_oracle_ssd_bwd.py against central differences of
    ``ssd``."""
    batch, dim, seqlen = (int(s) for s in x.shape)
    heads = int(A.shape[0])
    if heads * headdim != dim:
        raise ValueError("x's channel count must be heads * headdim")
    dstate = int(B.shape[1])
    delta = torch.as_tensor(dt).repeat_interleave(headdim, dim=1).contiguous()
    a = torch.as_tensor(A, dtype=torch.float32).repeat_interleave(headdim)[:, None].expand(dim, dstate).contiguous()
    bias = None if dt_bias is None else torch.as_tensor(dt_bias, dtype=torch.float32).repeat_interleave(headdim)
    g = scan_bwd(x, delta, a, B, C, D, z, bias, softplus, h0=h0, dy=dy, threads=threads)
    return {
        "dx": g["du"],
        "ddt": g["ddelta"].reshape(batch, heads, headdim, seqlen).sum(axis=2),
        "dz": g["dz"],
        "dA": g["dA"].reshape(heads, headdim * dstate).sum(axis=1),
        "dB": g["dB"],
        "dC": g["dC"],
        "dD": g["dD"],
        "ddt_bias": None if g["ddt_bias"] is None else g["ddt_bias"].reshape(heads, headdim).sum(axis=1),
        "dh0": g["dh0"],
    }
