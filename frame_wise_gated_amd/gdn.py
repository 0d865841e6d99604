"""ctypes binding of libgdn (the HIP/gfx950 frame-wise GDN library).

Argument marshalling only: shapes and dtypes are read off the tensors, device
pointers and the current HIP stream are passed to the C entry points of the
same names (declared in include/gdn.h), and PyTorch provides the device
memory for outputs and the workspace. Every step of the computation runs in
the library's kernels; there is no fallback when the library is missing.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "gdn.h")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EWORKSPACE, GDN_EHIP = range(5)
GDN_F32, GDN_BF16 = 0, 1
GDN_KEYS_RAW, GDN_KEYS_PREPARED, GDN_QK_RMSNORM, GDN_REUSE_FWD_TERMS = 0, 1, 2, 4
GDN_MAX_TIME_CHUNKS = 256
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gdn_status_str(status)} (status {status})")


class gdn_desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("S", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("key_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class gdn_trace(ctypes.Structure):
    _fields_ = [
        ("events", ctypes.POINTER(ctypes.c_void_p)),
        ("phases", ctypes.POINTER(ctypes.c_int32)),
        ("capacity", ctypes.c_int32),
        ("count", ctypes.c_int32),
    ]


# gdn_phase ids (include/gdn.h) -> names
PHASES = {0: "call_begin", 1: "terms", 2: "terms_reduce", 3: "scan", 4: "combine", 5: "replay",
          6: "reverse", 7: "readout", 8: "bwd_terms", 9: "bwd_edq", 10: "bwd_init",
          11: "bwd_adjoint", 12: "bwd_frame", 13: "bwd_token", 14: "other"}

_lib = None
_vp = ctypes.c_void_p
_st = ctypes.c_int32


def exported_names_in_header() -> list[str]:
    with open(HEADER_PATH) as f:
        return re.findall(r"GDN_API\s+[\w\s\*]+?\b(gdn_\w+)\s*\(", f.read())


def lib() -> ctypes.CDLL:
    """Load libgdn.so (built in-tree by frame_wise_gated_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m frame_wise_gated_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.gdn_status_str.restype = ctypes.c_char_p
    L.gdn_status_str.argtypes = [ctypes.c_int32]
    L.gdn_workspace_bytes.restype = _st
    L.gdn_workspace_bytes.argtypes = [P(gdn_desc), ctypes.c_int32, P(ctypes.c_size_t)]
    L.gdn_prepare.restype = _st
    L.gdn_prepare.argtypes = [P(gdn_desc), _vp, _vp, _vp]
    L.gdn_frame_terms.restype = _st
    L.gdn_frame_terms.argtypes = [P(gdn_desc), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.gdn_scan_fwd.restype = _st
    L.gdn_scan_fwd.argtypes = [P(gdn_desc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               ctypes.c_int32, _vp, ctypes.c_size_t, _vp]
    L.gdn_scan_bidir_chunked.restype = _st
    L.gdn_scan_bidir_chunked.argtypes = [P(gdn_desc), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                         _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, ctypes.c_size_t, _vp]
    L.gdn_step.restype = _st
    L.gdn_step.argtypes = [P(gdn_desc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           ctypes.c_size_t, _vp]
    L.gdn_step_noalloc.restype = _st
    L.gdn_step_noalloc.argtypes = [P(gdn_desc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.gdn_compose.restype = _st
    L.gdn_compose.argtypes = [P(gdn_desc), _vp, _vp, _vp, _vp, P(ctypes.c_int32), ctypes.c_int32,
                              _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.gdn_bwd_workspace_bytes.restype = _st
    L.gdn_bwd_workspace_bytes.argtypes = [P(gdn_desc), P(ctypes.c_size_t)]
    L.gdn_scan_bwd.restype = _st
    L.gdn_scan_bwd.argtypes = [P(gdn_desc)] + [_vp] * 15 + [_vp, ctypes.c_size_t, _vp]
    L.gdn_bidir_bwd_workspace_bytes.restype = _st
    L.gdn_bidir_bwd_workspace_bytes.argtypes = [P(gdn_desc), ctypes.c_int32, P(ctypes.c_size_t)]
    L.gdn_scan_bidir_chunked_bwd.restype = _st
    L.gdn_scan_bidir_chunked_bwd.argtypes = ([P(gdn_desc), ctypes.c_int32] + [_vp] * 16
                                             + [_vp, ctypes.c_size_t, _vp])
    L.gdn_readout.restype = _st
    L.gdn_readout.argtypes = [P(gdn_desc), _vp, _vp, _vp, _vp, _vp]
    L.gdn_trace_set.restype = _st
    L.gdn_trace_set.argtypes = [P(gdn_trace)]
    _lib = L
    return L


def gdn_status_str(status: int) -> str:
    return lib().gdn_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != GDN_OK:
        raise GdnError(status, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_desc(B, H, T, S, D, io_dtype, key_scale=0.0, keys_prepared=False,
              qk_rmsnorm=False, reuse_fwd_terms=False) -> gdn_desc:
    flags = (GDN_KEYS_PREPARED if keys_prepared else GDN_KEYS_RAW) | \
        (GDN_QK_RMSNORM if qk_rmsnorm else 0) | (GDN_REUSE_FWD_TERMS if reuse_fwd_terms else 0)
    return gdn_desc(B, H, T, S, D, io_dtype, float(key_scale), flags)


def _desc_from(k: torch.Tensor, key_scale, keys_prepared, qk_rmsnorm=False,
               reuse_fwd_terms=False) -> gdn_desc:
    if k.dim() != 5:
        raise ValueError("k must be [B, H, T, S, D]")
    if k.dtype == torch.float32:
        io = GDN_F32
    elif k.dtype == torch.bfloat16:
        io = GDN_BF16
    else:
        raise ValueError(f"unsupported io dtype {k.dtype}")
    B, H, T, S, D = k.shape
    return make_desc(B, H, T, S, D, io, key_scale, keys_prepared, qk_rmsnorm, reuse_fwd_terms)


def _need(t: torch.Tensor | None, name: str, shape, dtype) -> None:
    """Every tensor handed to the library is contiguous, of the expected shape
    and dtype, and lives on the current GPU (its address goes to the kernels
    as is: a host tensor or one on another device would fault there)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
    if not t.is_cuda or t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: expected a tensor on the current GPU "
                         f"(cuda:{torch.cuda.current_device() if t.is_cuda else '?'}), got {t.device}")


def _out(given, want: bool, shape, dtype, device):
    if given is not None:
        return given
    return torch.empty(shape, dtype=dtype, device=device) if want else None


def gdn_workspace_bytes(desc: gdn_desc, n_time_chunks: int = 1) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_workspace_bytes(ctypes.byref(desc), int(n_time_chunks), ctypes.byref(n)),
           "gdn_workspace_bytes")
    return int(n.value)


def workspace(desc: gdn_desc, n_time_chunks: int = 1, device="cuda") -> torch.Tensor:
    """A workspace tensor of the size the library asks for."""
    return torch.empty(max(gdn_workspace_bytes(desc, n_time_chunks), 1), dtype=torch.uint8, device=device)


def _ws(ws, desc, n_time_chunks, device):
    if ws is None:
        ws = workspace(desc, n_time_chunks, device)
    return ws, ws.numel() * ws.element_size()


def gdn_prepare(k, k_hat=None, key_scale=0.0, qk_rmsnorm=False, stream=None):
    d = _desc_from(k, key_scale, False, qk_rmsnorm)
    k_hat = _out(k_hat, True, k.shape, k.dtype, k.device)
    _need(k, "k", k.shape, k.dtype)
    _need(k_hat, "k_hat", k.shape, k.dtype)
    _check(lib().gdn_prepare(ctypes.byref(d), _ptr(k), _ptr(k_hat), _stream(stream)), "gdn_prepare")
    return k_hat


def gdn_frame_terms(k, v, beta, A=None, U=None, key_scale=0.0, keys_prepared=False, ws=None,
                    stream=None, qk_rmsnorm=False):
    d = _desc_from(k, key_scale, keys_prepared, qk_rmsnorm)
    B, H, T, S, D = k.shape
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, k.shape, k.dtype)
    _need(beta, "beta", (B, H, T, S), torch.float32)
    A = _out(A, True, (B, H, T, D, D), torch.float32, k.device)
    U = _out(U, True, (B, H, T, D, D), torch.float32, k.device)
    ws, nb = _ws(ws, d, 1, k.device)
    _check(lib().gdn_frame_terms(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(beta), _ptr(A), _ptr(U),
                                 _ptr(ws), nb, _stream(stream)), "gdn_frame_terms")
    return A, U


def gdn_scan_fwd(q, k, v, beta, gamma, s0=None, n_time_chunks=1, key_scale=0.0,
                 keys_prepared=False, want_states=True, want_s_final=True, want_o=True,
                 states=None, s_final=None, o=None, ws=None, stream=None, qk_rmsnorm=False):
    d = _desc_from(k, key_scale, keys_prepared, qk_rmsnorm)
    B, H, T, S, D = k.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need(t, n, k.shape, k.dtype)
    _need(beta, "beta", (B, H, T, S), torch.float32)
    _need(gamma, "gamma", (B, H, T), torch.float32)
    _need(s0, "s0", (B, H, D, D), torch.float32)
    states = _out(states, want_states, (B, H, T, D, D), torch.float32, k.device)
    s_final = _out(s_final, want_s_final, (B, H, D, D), torch.float32, k.device)
    o = _out(o, want_o, k.shape, k.dtype, k.device)
    _need(states, "states", (B, H, T, D, D), torch.float32)
    _need(s_final, "s_final", (B, H, D, D), torch.float32)
    ws, nb = _ws(ws, d, n_time_chunks, k.device)
    _check(lib().gdn_scan_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gamma),
                              _ptr(s0), _ptr(states), _ptr(s_final), _ptr(o), int(n_time_chunks),
                              _ptr(ws), nb, _stream(stream)), "gdn_scan_fwd")
    return {"states": states, "s_final": s_final, "o": o}


def gdn_scan_bidir_chunked(q, k, v, beta, gamma, chunk_len, s0=None, n_time_chunks=1,
                           key_scale=0.0, keys_prepared=False, want_states=True, want_s_final=True,
                           want_o=True, states_fwd=None, states_rev=None, s_final=None, o=None,
                           ws=None, stream=None, qk_rmsnorm=False):
    d = _desc_from(k, key_scale, keys_prepared, qk_rmsnorm)
    B, H, T, S, D = k.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need(t, n, k.shape, k.dtype)
    _need(beta, "beta", (B, H, T, S), torch.float32)
    _need(gamma, "gamma", (B, H, T), torch.float32)
    _need(s0, "s0", (B, H, D, D), torch.float32)
    states_fwd = _out(states_fwd, want_states, (B, H, T, D, D), torch.float32, k.device)
    states_rev = _out(states_rev, want_states, (B, H, T, D, D), torch.float32, k.device)
    s_final = _out(s_final, want_s_final, (B, H, D, D), torch.float32, k.device)
    o = _out(o, want_o, k.shape, k.dtype, k.device)
    ws, nb = _ws(ws, d, n_time_chunks, k.device)
    _check(lib().gdn_scan_bidir_chunked(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                        _ptr(gamma), _ptr(s0), int(chunk_len), _ptr(states_fwd),
                                        _ptr(states_rev), _ptr(s_final), _ptr(o),
                                        int(n_time_chunks), _ptr(ws), nb, _stream(stream)),
           "gdn_scan_bidir_chunked")
    return {"states_fwd": states_fwd, "states_rev": states_rev, "s_final": s_final, "o": o}


def gdn_step(q, k, v, beta, gamma, carry_in=None, carry_out=None, key_scale=0.0,
             keys_prepared=False, want_o=True, want_states=False, o=None, states_fwd=None,
             states_rev=None, ws=None, stream=None, qk_rmsnorm=False):
    """One streaming block (k.shape[2] frames): bidirectional inside the block,
    forward state carried in from `carry_in` and out to `carry_out` (which may
    be the same tensor)."""
    d = _desc_from(k, key_scale, keys_prepared, qk_rmsnorm)
    B, H, T, S, D = k.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need(t, n, k.shape, k.dtype)
    _need(beta, "beta", (B, H, T, S), torch.float32)
    _need(gamma, "gamma", (B, H, T), torch.float32)
    _need(carry_in, "carry_in", (B, H, D, D), torch.float32)
    _need(carry_out, "carry_out", (B, H, D, D), torch.float32)
    carry_out = _out(carry_out, True, (B, H, D, D), torch.float32, k.device)
    o = _out(o, want_o, k.shape, k.dtype, k.device)
    states_fwd = _out(states_fwd, want_states, (B, H, T, D, D), torch.float32, k.device)
    states_rev = _out(states_rev, want_states, (B, H, T, D, D), torch.float32, k.device)
    ws, nb = _ws(ws, d, 1, k.device)
    _check(lib().gdn_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gamma),
                          _ptr(carry_in), _ptr(carry_out), _ptr(o), _ptr(states_fwd),
                          _ptr(states_rev), _ptr(ws), nb, _stream(stream)), "gdn_step")
    return {"carry_out": carry_out, "o": o, "states_fwd": states_fwd, "states_rev": states_rev}


def gdn_step_noalloc(q, k, v, beta, gamma, carry_in=None, carry_out=None, key_scale=0.0,
                     keys_prepared=False, want_o=True, want_states=False, o=None, states_fwd=None,
                     states_rev=None, stream=None, qk_rmsnorm=False):
    """gdn_step on the library's static device scratch instead of a workspace
    (gdn_step_noalloc): the library allocates nothing. Outputs that are not
    given are allocated here by torch, so a caller that must not allocate
    passes every wanted output."""
    d = _desc_from(k, key_scale, keys_prepared, qk_rmsnorm)
    B, H, T, S, D = k.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need(t, n, k.shape, k.dtype)
    _need(beta, "beta", (B, H, T, S), torch.float32)
    _need(gamma, "gamma", (B, H, T), torch.float32)
    _need(carry_in, "carry_in", (B, H, D, D), torch.float32)
    _need(carry_out, "carry_out", (B, H, D, D), torch.float32)
    carry_out = _out(carry_out, True, (B, H, D, D), torch.float32, k.device)
    o = _out(o, want_o, k.shape, k.dtype, k.device)
    states_fwd = _out(states_fwd, want_states, (B, H, T, D, D), torch.float32, k.device)
    states_rev = _out(states_rev, want_states, (B, H, T, D, D), torch.float32, k.device)
    _check(lib().gdn_step_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                  _ptr(gamma), _ptr(carry_in), _ptr(carry_out), _ptr(o),
                                  _ptr(states_fwd), _ptr(states_rev), _stream(stream)),
           "gdn_step_noalloc")
    return {"carry_out": carry_out, "o": o, "states_fwd": states_fwd, "states_rev": states_rev}


def gdn_compose(k, v, beta, gamma, chunk_offsets, s0=None, key_scale=0.0, keys_prepared=False,
                want_C=True, want_H=True, want_s_start=True, C=None, Hc=None, s_start=None,
                ws=None, stream=None, qk_rmsnorm=False):
    d = _desc_from(k, key_scale, keys_prepared, qk_rmsnorm)
    B, H, T, S, D = k.shape
    P = len(chunk_offsets) - 1
    offs = (ctypes.c_int32 * (P + 1))(*[int(x) for x in chunk_offsets])
    _need(beta, "beta", (B, H, T, S), torch.float32)
    _need(gamma, "gamma", (B, H, T), torch.float32)
    _need(s0, "s0", (B, H, D, D), torch.float32)
    C = _out(C, want_C, (B, H, P, D, D), torch.float32, k.device)
    Hc = _out(Hc, want_H, (B, H, P, D, D), torch.float32, k.device)
    s_start = _out(s_start, want_s_start, (B, H, P, D, D), torch.float32, k.device)
    ws, nb = _ws(ws, d, max(P, 1), k.device)
    _check(lib().gdn_compose(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(beta), _ptr(gamma), offs, P,
                             _ptr(C), _ptr(Hc), _ptr(s0), _ptr(s_start), _ptr(ws), nb,
                             _stream(stream)), "gdn_compose")
    return {"C": C, "Hc": Hc, "s_start": s_start}


def gdn_bwd_workspace_bytes(desc: gdn_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_bwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "gdn_bwd_workspace_bytes")
    return int(n.value)


def gdn_scan_bwd(q, k, v, beta, gamma, states, d_o, s0=None, ds_final=None, key_scale=0.0,
                 keys_prepared=False, want=("dq", "dk", "dv", "dbeta", "dgamma", "ds0"),
                 out=None, ws=None, stream=None, qk_rmsnorm=False, reuse_fwd_terms=False):
    """Gradients of the causal frame scan; `states` are the forward's
    per-frame states. Returns a dict with the requested gradients.
    reuse_fwd_terms: `ws` is the workspace the forward call used (sized for
    both calls, untouched since), and A_t is read from it (GDN_REUSE_FWD_TERMS)."""
    if reuse_fwd_terms and ws is None:
        raise ValueError("reuse_fwd_terms needs the forward call's workspace as ws")
    d = _desc_from(k, key_scale, keys_prepared, qk_rmsnorm, reuse_fwd_terms)
    B, H, T, S, D = k.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (d_o, "d_o")):
        _need(t, n, k.shape, k.dtype)
    _need(beta, "beta", (B, H, T, S), torch.float32)
    _need(gamma, "gamma", (B, H, T), torch.float32)
    _need(states, "states", (B, H, T, D, D), torch.float32)
    _need(s0, "s0", (B, H, D, D), torch.float32)
    _need(ds_final, "ds_final", (B, H, D, D), torch.float32)
    shapes = {"dq": (k.shape, k.dtype), "dk": (k.shape, k.dtype), "dv": (k.shape, k.dtype),
              "dbeta": ((B, H, T, S), torch.float32), "dgamma": ((B, H, T), torch.float32),
              "ds0": ((B, H, D, D), torch.float32)}
    out = dict(out or {})
    for n, (shp, dt) in shapes.items():
        _need(out.get(n), n, shp, dt)
        out[n] = _out(out.get(n), n in want, shp, dt, k.device)
    if ws is None:
        ws = torch.empty(max(gdn_bwd_workspace_bytes(d), 1), dtype=torch.uint8, device=k.device)
    nb = ws.numel() * ws.element_size()
    _check(lib().gdn_scan_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gamma),
                              _ptr(s0), _ptr(states), _ptr(d_o), _ptr(ds_final), _ptr(out["dq"]),
                              _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
                              _ptr(out["dgamma"]), _ptr(out["ds0"]), _ptr(ws), nb, _stream(stream)),
           "gdn_scan_bwd")
    return out


def gdn_bidir_bwd_workspace_bytes(desc: gdn_desc, chunk_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_bidir_bwd_workspace_bytes(ctypes.byref(desc), int(chunk_len), ctypes.byref(n)),
           "gdn_bidir_bwd_workspace_bytes")
    return int(n.value)


def gdn_scan_bidir_chunked_bwd(q, k, v, beta, gamma, chunk_len, states_fwd, states_rev, d_o,
                               s0=None, ds_final=None, key_scale=0.0, keys_prepared=False,
                               want=("dq", "dk", "dv", "dbeta", "dgamma", "ds0"), out=None,
                               ws=None, stream=None, qk_rmsnorm=False, reuse_fwd_terms=False):
    """Gradients of the chunk-causal bidirectional scan; `states_fwd` and
    `states_rev` are the forward call's states. Returns a dict with the
    requested gradients. reuse_fwd_terms as in gdn_scan_bwd."""
    if reuse_fwd_terms and ws is None:
        raise ValueError("reuse_fwd_terms needs the forward call's workspace as ws")
    d = _desc_from(k, key_scale, keys_prepared, qk_rmsnorm, reuse_fwd_terms)
    B, H, T, S, D = k.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (d_o, "d_o")):
        _need(t, n, k.shape, k.dtype)
    _need(beta, "beta", (B, H, T, S), torch.float32)
    _need(gamma, "gamma", (B, H, T), torch.float32)
    _need(states_fwd, "states_fwd", (B, H, T, D, D), torch.float32)
    _need(states_rev, "states_rev", (B, H, T, D, D), torch.float32)
    _need(s0, "s0", (B, H, D, D), torch.float32)
    _need(ds_final, "ds_final", (B, H, D, D), torch.float32)
    shapes = {"dq": (k.shape, k.dtype), "dk": (k.shape, k.dtype), "dv": (k.shape, k.dtype),
              "dbeta": ((B, H, T, S), torch.float32), "dgamma": ((B, H, T), torch.float32),
              "ds0": ((B, H, D, D), torch.float32)}
    out = dict(out or {})
    for n, (shp, dt) in shapes.items():
        _need(out.get(n), n, shp, dt)
        out[n] = _out(out.get(n), n in want, shp, dt, k.device)
    if ws is None:
        ws = torch.empty(max(gdn_bidir_bwd_workspace_bytes(d, chunk_len), 1), dtype=torch.uint8,
                         device=k.device)
    nb = ws.numel() * ws.element_size()
    _check(lib().gdn_scan_bidir_chunked_bwd(
        ctypes.byref(d), int(chunk_len), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gamma),
        _ptr(s0), _ptr(states_fwd), _ptr(states_rev), _ptr(d_o), _ptr(ds_final), _ptr(out["dq"]),
        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dgamma"]),
        _ptr(out["ds0"]), _ptr(ws), nb, _stream(stream)), "gdn_scan_bidir_chunked_bwd")
    return out


def gdn_readout(q, states, states_add=None, o=None, qk_rmsnorm=False, stream=None):
    d = _desc_from(q, 0.0, False, qk_rmsnorm)
    B, H, T, S, D = q.shape
    _need(q, "q", q.shape, q.dtype)
    _need(states, "states", (B, H, T, D, D), torch.float32)
    _need(states_add, "states_add", (B, H, T, D, D), torch.float32)
    o = _out(o, True, q.shape, q.dtype, q.device)
    _need(o, "o", q.shape, q.dtype)
    _check(lib().gdn_readout(ctypes.byref(d), _ptr(q), _ptr(states), _ptr(states_add), _ptr(o),
                             _stream(stream)), "gdn_readout")
    return o


_hip = None
HIP_EVENT_RELEASE_TO_DEVICE = 0x40000000  # hipEventReleaseToDevice


def _hip_runtime() -> ctypes.CDLL:
    """The HIP runtime already loaded by torch (same soname as libgdn needs),
    for creating and reading the trace events."""
    global _hip
    if _hip is None:
        torch.cuda.init()
        h = ctypes.CDLL("libamdhip64.so.7")
        h.hipEventCreateWithFlags.restype = ctypes.c_int
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventElapsedTime.restype = ctypes.c_int
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        h.hipEventDestroy.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip = h
    return _hip


class PhaseTrace:
    """Per-phase device times of the library calls made on this thread.

    Inside ``with PhaseTrace(capacity) as tr:`` every call records HIP events
    on its stream at its start and after each launch group (gdn_trace_set).
    After a synchronisation, ``tr.calls()`` returns one dict per call:
    ``{"total": ms, <phase name>: ms, ...}``, the device time from the call's
    first event to its last and of each phase. The events are created here
    with a device-scope release (hipEventReleaseToDevice): recording them
    writes nothing back to the host, so they barely disturb the timed work."""

    def __init__(self, capacity: int, flags: int = HIP_EVENT_RELEASE_TO_DEVICE):
        h = _hip_runtime()
        self._ev = (ctypes.c_void_p * capacity)()
        for i in range(capacity):
            e = ctypes.c_void_p()
            if h.hipEventCreateWithFlags(ctypes.byref(e), flags) != 0:
                self.close()
                raise RuntimeError("hipEventCreateWithFlags failed")
            self._ev[i] = e.value
        self._ph = (ctypes.c_int32 * capacity)()
        self._t = gdn_trace(self._ev, self._ph, capacity, 0)

    def close(self) -> None:
        if _hip is not None and getattr(self, "_ev", None) is not None:
            for e in self._ev:
                if e:
                    _hip.hipEventDestroy(e)
            self._ev = None

    def __del__(self):
        self.close()

    def reset(self) -> None:
        self._t.count = 0

    def __enter__(self):
        _check(lib().gdn_trace_set(ctypes.byref(self._t)), "gdn_trace_set")
        return self

    def __exit__(self, *exc):
        lib().gdn_trace_set(None)
        return False

    @property
    def count(self) -> int:
        return int(self._t.count)

    def full(self) -> bool:
        return self._t.count >= self._t.capacity

    def _ms(self, i: int, j: int) -> float:
        out = ctypes.c_float(0.0)
        if _hip.hipEventElapsedTime(ctypes.byref(out), self._ev[i], self._ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed (events not complete?)")
        return float(out.value)

    def calls(self) -> list[dict]:
        out, cur, first = [], None, None
        for i in range(self._t.count):
            ph = PHASES.get(int(self._ph[i]), "other")
            if ph == "call_begin":
                if cur is not None:
                    cur["total"] = self._ms(first, i - 1)
                    out.append(cur)
                cur, first = {}, i
            elif cur is not None:
                cur[ph] = cur.get(ph, 0.0) + self._ms(i - 1, i)
        if cur is not None:
            cur["total"] = self._ms(first, self._t.count - 1)
            out.append(cur)
        return out
