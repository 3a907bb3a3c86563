"""Thin ctypes binding over ``libkdaconv.so`` (argument marshalling only).

The functions carry the C-ABI names of ``include/kdaconv.h``.  Every step of
the computation runs in the library's HIP kernels; PyTorch only provides
device memory and the current stream.  If the library is not built the
binding raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkdaconv.so")

KDA_F32 = 0
KDA_BF16 = 1

KDA_OK = 0
KDA_ERR_INVALID_ARG = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_WORKSPACE = -3
KDA_ERR_HIP = -4

KDA_MAX_SEQS = 64   # streams of one variable-length batch

EXPORTED_SYMBOLS = ("kda_conv_forward", "kda_conv_forward_stream", "kda_forward_workspace_size", "kda_forward",
                    "kda_forward_chunks", "kda_forward_scan", "kda_forward_varlen_workspace_size",
                    "kda_forward_varlen", "kda_conv_forward_varlen", "mla_attention_forward",
                    "kda_backward_workspace_size", "kda_backward", "kda_conv_backward", "kda_status_string",
                    "kda_forward_noalloc", "mla_latent_forward", "kda_conv_kda_forward_workspace_size",
                    "kda_conv_kda_forward")
KDA_NOALLOC_SCRATCH_BYTES = 64 << 20


class KdaStreamDesc(ctypes.Structure):
    _fields_ = [("n_text", ctypes.c_int32), ("grid_t", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("k_text", ctypes.c_int32), ("k_vis", ctypes.c_int32),
                ("causal_t", ctypes.c_int32)]


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%d)" % (fn, kda_status_string(status), status))
        self.status = status


_lib = None


def load_library():
    """Load the built library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkdaconv.so is not built (expected at %s); run "
                           "python -m linear_attention_sequence_modality_amd.build first" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    desc_p = ctypes.POINTER(KdaStreamDesc)
    lib.kda_conv_forward.restype = i32
    lib.kda_conv_forward.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp,
                                     ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, vp]
    lib.kda_conv_forward_stream.restype = i32
    lib.kda_conv_forward_stream.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp,
                                            ctypes.POINTER(vp), i32, ctypes.POINTER(vp),
                                            ctypes.POINTER(vp), vp, vp, vp, vp]
    lib.kda_forward_workspace_size.restype = ctypes.c_size_t
    lib.kda_forward_workspace_size.argtypes = [desc_p, i32, i32, i32, i32, i32]
    lib.kda_forward.restype = i32
    lib.kda_forward.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                vp, ctypes.c_size_t, vp]
    lib.kda_forward_noalloc.restype = i32
    lib.kda_forward_noalloc.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_forward_chunks.restype = i32
    lib.kda_forward_chunks.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
    lib.kda_forward_scan.restype = i32
    lib.kda_forward_scan.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
    lib.kda_forward_varlen_workspace_size.restype = ctypes.c_size_t
    lib.kda_forward_varlen_workspace_size.argtypes = [desc_p, i32, i32, i32, i32, i32]
    lib.kda_forward_varlen.restype = i32
    lib.kda_forward_varlen.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, ctypes.c_size_t, vp]
    lib.kda_conv_forward_varlen.restype = i32
    lib.kda_conv_forward_varlen.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp,
                                            ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, vp]
    lib.kda_backward_workspace_size.restype = ctypes.c_size_t
    lib.kda_backward_workspace_size.argtypes = [desc_p, i32, i32, i32, i32, i32]
    lib.kda_backward.restype = i32
    lib.kda_backward.argtypes = [desc_p, i32, i32, i32, i32, i32] + [vp] * 15 + [ctypes.c_size_t, vp]
    lib.kda_conv_backward.restype = i32
    lib.kda_conv_backward.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp, ctypes.POINTER(vp),
                                      ctypes.POINTER(vp), vp, vp, vp, vp, vp, vp, ctypes.POINTER(vp),
                                      ctypes.POINTER(vp), vp]
    lib.mla_attention_forward.restype = i32
    lib.mla_attention_forward.argtypes = [i32] * 7 + [vp] * 5 + [ctypes.c_float, vp, vp]
    lib.kda_conv_kda_forward_workspace_size.restype = ctypes.c_size_t
    lib.kda_conv_kda_forward_workspace_size.argtypes = [desc_p, i32, i32, i32, i32, i32]
    lib.kda_conv_kda_forward.restype = i32
    lib.kda_conv_kda_forward.argtypes = [desc_p, i32, i32, i32, i32, i32, vp, vp, vp, ctypes.POINTER(vp),
                                         ctypes.POINTER(vp), vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.mla_latent_forward.restype = i32
    lib.mla_latent_forward.argtypes = [ctypes.c_int64] + [i32] * 7 + [vp] * 10
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i32]
    _lib = lib
    return lib


def make_desc(n_text: int, grid: Sequence[int], causal_t: int = 0, k_text: int = 4,
              k_vis: int = 3) -> KdaStreamDesc:
    gt, gh, gw = (int(x) for x in grid)
    return KdaStreamDesc(int(n_text), gt, gh, gw, int(k_text), int(k_vis), int(causal_t))


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return KDA_F32
    if dt == torch.bfloat16:
        return KDA_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % dt)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _torch_stream(stream, device) -> Optional["torch.cuda.Stream"]:
    if stream is None or isinstance(stream, torch.cuda.Stream):
        return stream
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.ExternalStream(handle, device=device)


def _hand_over(stream, device, *tensors):
    """Tensors a wrapper allocated (on the current stream) and handed to kernels enqueued on
    ``stream``: when that is another stream, tell the caching allocator, so that their memory
    is not given to a new allocation before that stream's work on them is done."""
    s = _torch_stream(stream, device)
    if s is None or s.cuda_stream == torch.cuda.current_stream(device).cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def _check(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must have dtype %s" % (name, dtype))


def kda_forward_workspace_size(desc: KdaStreamDesc, B: int, H: int, dk: int, dv: int,
                               dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(load_library().kda_forward_workspace_size(ctypes.byref(desc), B, H, dk, dv, code))


def kda_conv_kda_forward_workspace_size(desc: KdaStreamDesc, B: int, H: int, dk: int, dv: int,
                                        dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(load_library().kda_conv_kda_forward_workspace_size(ctypes.byref(desc), B, H, dk, dv, code))


def kda_conv_kda_forward(desc: KdaStreamDesc, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         w_text: Sequence[torch.Tensor], w_vis: Sequence[torch.Tensor],
                         alpha: torch.Tensor, beta: torch.Tensor,
                         initial_state: Optional[torch.Tensor] = None,
                         final_state: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Conv + KDA in one call, the conv formed inside the chunk transform (q', k', v' are
    never written); q, k, v are the conv inputs.  Returns o [B,T,H,dv] (final_state filled
    in place if given)."""
    lib = load_library()
    dt = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta")):
        _check(t, nm, dt)
    for i in range(3):
        _check(w_text[i], "w_text[%d]" % i, dt)
        _check(w_vis[i], "w_vis[%d]" % i, dt)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _check(t, nm, torch.float32)
    made_o, made_ws = o is None, workspace is None
    o = torch.empty_like(v) if o is None else o
    _check(o, "o", dt)
    need = kda_conv_kda_forward_workspace_size(desc, B, H, dk, dv, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _hand_over(stream, q.device, o if made_o else None, workspace if made_ws else None)
    wt = (ctypes.c_void_p * 3)(*[w.data_ptr() for w in w_text])
    wv = (ctypes.c_void_p * 3)(*[w.data_ptr() for w in w_vis])
    rc = lib.kda_conv_kda_forward(ctypes.byref(desc), B, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v),
                                  wt, wv, _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(final_state),
                                  _ptr(o), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_conv_kda_forward", rc)
    return o


def supports(dtype, dk: int, dv: int) -> bool:
    """Whether the library runs KDA for this dtype and head size (its workspace query is nonzero)."""
    return kda_forward_workspace_size(make_desc(1, (0, 0, 0)), 1, 1, dk, dv, dtype) > 0


def kda_conv_forward(desc: KdaStreamDesc, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     w_text: Sequence[torch.Tensor], w_vis: Sequence[torch.Tensor],
                     q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                     v_out: Optional[torch.Tensor] = None, stream=None,
                     history: Optional[Sequence[torch.Tensor]] = None
                     ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Modality-aware depthwise short conv of q [B,T,H,dk], k [B,T,H,dk], v [B,T,H,dv].

    ``history`` (time-causal segments, kda_conv_forward_stream): the conv inputs
    (q, k, v) of the latent slices just before this segment, each
    [B, n_hist * h * w, H, d] with n_hist in {1, 2}.
    """
    lib = load_library()
    dt = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm, dt)
    for i in range(3):
        _check(w_text[i], "w_text[%d]" % i, dt)
        _check(w_vis[i], "w_vis[%d]" % i, dt)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    made = [t is None for t in (q_out, k_out, v_out)]
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    v_out = torch.empty_like(v) if v_out is None else v_out
    _hand_over(stream, q.device, *[t for t, m in zip((q_out, k_out, v_out), made) if m])
    wt = (ctypes.c_void_p * 3)(*[w.data_ptr() for w in w_text])
    wv = (ctypes.c_void_p * 3)(*[w.data_ptr() for w in w_vis])
    if history is None:
        rc = lib.kda_conv_forward(ctypes.byref(desc), B, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k),
                                  _ptr(v), wt, wv, _ptr(q_out), _ptr(k_out), _ptr(v_out),
                                  _stream(stream))
        if rc != KDA_OK:
            raise KdaError("kda_conv_forward", rc)
        return q_out, k_out, v_out
    for i, t in enumerate(history):
        _check(t, "history[%d]" % i, dt)
    slice_tokens = desc.grid_h * desc.grid_w
    n_hist = history[0].shape[1] // slice_tokens if slice_tokens else 0
    if any(t.shape[1] != n_hist * slice_tokens or t.shape[0] != B for t in history):
        raise ValueError("history tensors must be [B, n_hist * h * w, H, d]")
    hs = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in history])
    rc = lib.kda_conv_forward_stream(ctypes.byref(desc), B, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k),
                                     _ptr(v), hs, n_hist, wt, wv, _ptr(q_out), _ptr(k_out), _ptr(v_out),
                                     _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_conv_forward_stream", rc)
    return q_out, k_out, v_out


def kda_forward(desc: KdaStreamDesc, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                alpha: torch.Tensor, beta: torch.Tensor,
                initial_state: Optional[torch.Tensor] = None,
                final_state: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """KDA gated delta-rule scan; returns o [B,T,H,dv] (final_state filled in place if given)."""
    lib = load_library()
    dt = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta")):
        _check(t, nm, dt)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _check(t, nm, torch.float32)
    made_o, made_ws = o is None, workspace is None
    o = torch.empty_like(v) if o is None else o
    _check(o, "o", dt)
    need = kda_forward_workspace_size(desc, B, H, dk, dv, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _hand_over(stream, q.device, o if made_o else None, workspace if made_ws else None)
    rc = lib.kda_forward(ctypes.byref(desc), B, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k),
                         _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(final_state),
                         _ptr(o), _ptr(workspace), workspace.numel() * workspace.element_size(),
                         _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_forward", rc)
    return o


def kda_forward_noalloc(desc: KdaStreamDesc, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        alpha: torch.Tensor, beta: torch.Tensor,
                        initial_state: Optional[torch.Tensor] = None,
                        final_state: Optional[torch.Tensor] = None, o: torch.Tensor = None,
                        stream=None) -> torch.Tensor:
    """kda_forward with the workspace in the library's own device array: the call allocates
    nothing, so ``o`` (and ``final_state`` if wanted) must be passed in."""
    lib = load_library()
    dt = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta")):
        _check(t, nm, dt)
    if o is None:
        raise ValueError("kda_forward_noalloc allocates nothing: pass o")
    _check(o, "o", dt)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _check(t, nm, torch.float32)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    rc = lib.kda_forward_noalloc(ctypes.byref(desc), B, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(final_state), _ptr(o),
                                 _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_forward_noalloc", rc)
    return o


def kda_forward_chunks(desc: KdaStreamDesc, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       alpha: torch.Tensor, beta: torch.Tensor, workspace: torch.Tensor,
                       stream=None) -> torch.Tensor:
    """First kernel of kda_forward: every chunk's UT/WY transform into ``workspace``."""
    lib = load_library()
    dt = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta")):
        _check(t, nm, dt)
    _check(workspace, "workspace")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    rc = lib.kda_forward_chunks(ctypes.byref(desc), B, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(alpha), _ptr(beta), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_forward_chunks", rc)
    return workspace


def kda_forward_scan(desc: KdaStreamDesc, B: int, H: int, dk: int, dv: int, dtype: torch.dtype,
                     workspace: torch.Tensor, o: torch.Tensor,
                     initial_state: Optional[torch.Tensor] = None,
                     final_state: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Second kernel of kda_forward: the ordered state pass writing ``o``."""
    lib = load_library()
    _check(workspace, "workspace")
    _check(o, "o", dtype)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _check(t, nm, torch.float32)
    rc = lib.kda_forward_scan(ctypes.byref(desc), B, H, dk, dv, _dtype_code(dtype),
                              _ptr(initial_state), _ptr(final_state), _ptr(o), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_forward_scan", rc)
    return o


def _desc_array(descs: Sequence[KdaStreamDesc]):
    arr = (KdaStreamDesc * max(len(descs), 1))()
    for i, d in enumerate(descs):
        arr[i] = d
    return arr


def kda_forward_varlen_workspace_size(descs: Sequence[KdaStreamDesc], H: int, dk: int, dv: int,
                                      dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(load_library().kda_forward_varlen_workspace_size(_desc_array(descs), len(descs), H, dk, dv,
                                                                code))


def kda_forward_varlen(descs: Sequence[KdaStreamDesc], q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       alpha: torch.Tensor, beta: torch.Tensor,
                       initial_state: Optional[torch.Tensor] = None,
                       final_state: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """KDA over a variable-length batch: stream i of ``descs`` at its tokens of the packed
    token axis of q [sum T_i, H, dk] (a leading axis of size 1 is allowed); states are
    [len(descs), H, dk, dv].  Returns o shaped like v."""
    lib = load_library()
    dt = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta")):
        _check(t, nm, dt)
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    total = sum(d.n_text + d.grid_t * d.grid_h * d.grid_w for d in descs)
    if q.numel() != total * H * dk or v.numel() != total * H * dv or beta.numel() != total * H:
        raise ValueError("q, k, v, alpha, beta must hold the %d tokens of the streams" % total)
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _check(t, nm, torch.float32)
    made_o, made_ws = o is None, workspace is None
    o = torch.empty_like(v) if o is None else o
    _check(o, "o", dt)
    need = kda_forward_varlen_workspace_size(descs, H, dk, dv, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _hand_over(stream, q.device, o if made_o else None, workspace if made_ws else None)
    rc = lib.kda_forward_varlen(_desc_array(descs), len(descs), H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(final_state),
                                _ptr(o), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_forward_varlen", rc)
    return o


def kda_conv_forward_varlen(descs: Sequence[KdaStreamDesc], q: torch.Tensor, k: torch.Tensor,
                            v: torch.Tensor, w_text: Sequence[torch.Tensor], w_vis: Sequence[torch.Tensor],
                            q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                            v_out: Optional[torch.Tensor] = None, stream=None
                            ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The short conv over a variable-length batch packed along the token axis."""
    lib = load_library()
    dt = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm, dt)
    for i in range(3):
        _check(w_text[i], "w_text[%d]" % i, dt)
        _check(w_vis[i], "w_vis[%d]" % i, dt)
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    total = sum(d.n_text + d.grid_t * d.grid_h * d.grid_w for d in descs)
    if q.numel() != total * H * dk or k.numel() != total * H * dk or v.numel() != total * H * dv:
        raise ValueError("q, k, v must hold the %d tokens of the streams" % total)
    made = [t is None for t in (q_out, k_out, v_out)]
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    v_out = torch.empty_like(v) if v_out is None else v_out
    _hand_over(stream, q.device, *[t for t, m in zip((q_out, k_out, v_out), made) if m])
    wt = (ctypes.c_void_p * 3)(*[w.data_ptr() for w in w_text])
    wv = (ctypes.c_void_p * 3)(*[w.data_ptr() for w in w_vis])
    rc = lib.kda_conv_forward_varlen(_desc_array(descs), len(descs), H, dk, dv, _dtype_code(dt), _ptr(q),
                                     _ptr(k), _ptr(v), wt, wv, _ptr(q_out), _ptr(k_out), _ptr(v_out),
                                     _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_conv_forward_varlen", rc)
    return q_out, k_out, v_out


def kda_backward_workspace_size(desc: KdaStreamDesc, B: int, H: int, dk: int, dv: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(load_library().kda_backward_workspace_size(ctypes.byref(desc), B, H, dk, dv, code))


def kda_backward(desc: KdaStreamDesc, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 alpha: torch.Tensor, beta: torch.Tensor, d_o: torch.Tensor,
                 initial_state: Optional[torch.Tensor] = None, d_final_state: Optional[torch.Tensor] = None,
                 want_d_initial_state: bool = True, workspace: Optional[torch.Tensor] = None,
                 stream=None) -> dict:
    """Gradients of the KDA scan: returns dict dq, dk, dv, dalpha, dbeta (stream dtype) and
    d_initial_state (fp32, or None)."""
    lib = load_library()
    dt = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta"), (d_o, "d_o")):
        _check(t, nm, dt)
    for t, nm in ((initial_state, "initial_state"), (d_final_state, "d_final_state")):
        if t is not None:
            _check(t, nm, torch.float32)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dalpha": torch.empty_like(alpha), "dbeta": torch.empty_like(beta),
           "d_initial_state": (torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device)
                               if want_d_initial_state else None)}
    need = kda_backward_workspace_size(desc, B, H, dk, dv, dt)
    made_ws = workspace is None
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _hand_over(stream, q.device, *out.values(), workspace if made_ws else None)
    rc = lib.kda_backward(ctypes.byref(desc), B, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v),
                          _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(d_o), _ptr(d_final_state),
                          _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]),
                          _ptr(out["dbeta"]), _ptr(out["d_initial_state"]), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_backward", rc)
    return out


def kda_conv_backward(desc: KdaStreamDesc, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      w_text: Sequence[torch.Tensor], w_vis: Sequence[torch.Tensor],
                      d_q_out: torch.Tensor, d_k_out: torch.Tensor, d_v_out: torch.Tensor,
                      stream=None) -> dict:
    """Backward of kda_conv_forward: returns dict dq, dk, dv (stream dtype) and
    dw_text, dw_vis (tuples of fp32 [H*d, 4] / [H*d, 27] per q, k, v)."""
    lib = load_library()
    dt = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (d_q_out, "d_q_out"), (d_k_out, "d_k_out"), (d_v_out, "d_v_out")):
        _check(t, nm, dt)
    for i in range(3):
        _check(w_text[i], "w_text[%d]" % i, dt)
        _check(w_vis[i], "w_vis[%d]" % i, dt)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dw_text": tuple(torch.empty(w.shape, dtype=torch.float32, device=q.device) for w in w_text),
           "dw_vis": tuple(torch.empty(w.shape, dtype=torch.float32, device=q.device) for w in w_vis)}
    _hand_over(stream, q.device, out["dq"], out["dk"], out["dv"], *out["dw_text"], *out["dw_vis"])
    arr = lambda ts: (ctypes.c_void_p * 3)(*[t.data_ptr() for t in ts])
    rc = lib.kda_conv_backward(ctypes.byref(desc), B, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v),
                               arr(w_text), arr(w_vis), _ptr(d_q_out), _ptr(d_k_out), _ptr(d_v_out),
                               _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), arr(out["dw_text"]),
                               arr(out["dw_vis"]), _stream(stream))
    if rc != KDA_OK:
        raise KdaError("kda_conv_backward", rc)
    return out


def mla_attention_forward(q_nope: torch.Tensor, q_dir: torch.Tensor, k_nope: torch.Tensor,
                          k_dir: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                          o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """MLA attention core: q_nope, k_nope [B,T,H,d_nope]; q_dir [B,T,H,d_dir]; k_dir [B,T,d_dir]
    (shared by the heads); v [B,T,H,dv].  Returns o shaped like v.  ``scale`` defaults to
    1/sqrt(d_nope + d_dir)."""
    lib = load_library()
    dt = q_nope.dtype
    for t, nm in ((q_nope, "q_nope"), (q_dir, "q_dir"), (k_nope, "k_nope"), (k_dir, "k_dir"), (v, "v")):
        _check(t, nm, dt)
    B, T, H, dn = q_nope.shape
    dr, dv = q_dir.shape[-1], v.shape[-1]
    if (tuple(q_dir.shape) != (B, T, H, dr) or tuple(k_nope.shape) != (B, T, H, dn)
            or tuple(k_dir.shape) != (B, T, dr) or tuple(v.shape[:3]) != (B, T, H)):
        raise ValueError("q_nope/k_nope [B,T,H,dn], q_dir [B,T,H,dr], k_dir [B,T,dr], v [B,T,H,dv] expected")
    scale = 1.0 / float(dn + dr) ** 0.5 if scale is None else float(scale)
    made_o = o is None
    o = torch.empty_like(v) if o is None else o
    _check(o, "o", dt)
    _hand_over(stream, q_nope.device, o if made_o else None)
    rc = lib.mla_attention_forward(B, T, H, dn, dr, dv, _dtype_code(dt), _ptr(q_nope), _ptr(q_dir), _ptr(k_nope),
                                   _ptr(k_dir), _ptr(v), ctypes.c_float(scale), _ptr(o), _stream(stream))
    if rc != KDA_OK:
        raise KdaError("mla_attention_forward", rc)
    return o


def mla_latent_forward(x: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor, w_uk: torch.Tensor,
                       w_uv: torch.Tensor, H: int, outputs: Optional[Sequence[torch.Tensor]] = None,
                       stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """MLA latent projections of hidden states x [..., d_model] with linear-layer weights
    w_dkv [d_c, d_model], w_kr [d_dir, d_model], w_uk [H*d_nope, d_c], w_uv [H*dv, d_c].
    Returns (c [..., d_c], k_dir [..., d_dir], k_nope [..., H, d_nope], v [..., H, dv])."""
    lib = load_library()
    dt = x.dtype
    for t, nm in ((x, "x"), (w_dkv, "w_dkv"), (w_kr, "w_kr"), (w_uk, "w_uk"), (w_uv, "w_uv")):
        _check(t, nm, dt)
    d_model = x.shape[-1]
    lead = tuple(x.shape[:-1])
    rows = x.numel() // d_model if d_model else 0
    d_c, d_dir = w_dkv.shape[0], w_kr.shape[0]
    if (tuple(w_dkv.shape) != (d_c, d_model) or tuple(w_kr.shape) != (d_dir, d_model)
            or w_uk.shape[1] != d_c or w_uv.shape[1] != d_c or w_uk.shape[0] % H or w_uv.shape[0] % H):
        raise ValueError("w_dkv [d_c, d_model], w_kr [d_dir, d_model], w_uk [H*d_nope, d_c], "
                         "w_uv [H*dv, d_c] expected")
    d_nope, dv = w_uk.shape[0] // H, w_uv.shape[0] // H
    shapes = (lead + (d_c,), lead + (d_dir,), lead + (H, d_nope), lead + (H, dv))
    if outputs is None:
        outs = [torch.empty(sh, dtype=dt, device=x.device) for sh in shapes]
        _hand_over(stream, x.device, *outs)
    else:
        outs = list(outputs)
        for t, sh, nm in zip(outs, shapes, ("c", "k_dir", "k_nope", "v")):
            _check(t, nm, dt)
            if tuple(t.shape) != sh:
                raise ValueError("%s must have shape %s" % (nm, sh))
    rc = lib.mla_latent_forward(rows, d_model, d_c, d_dir, H, d_nope, dv, _dtype_code(dt), _ptr(x), _ptr(w_dkv),
                                _ptr(w_kr), _ptr(w_uk), _ptr(w_uv), *[_ptr(t) for t in outs], _stream(stream))
    if rc != KDA_OK:
        raise KdaError("mla_latent_forward", rc)
    return tuple(outs)


def mla_layer_forward(x: torch.Tensor, q_nope: torch.Tensor, q_dir: torch.Tensor, weights: dict,
                      scale: Optional[float] = None, stream=None) -> Tuple[torch.Tensor, tuple]:
    """The MLA token mixer from hidden states: latent projections (mla_latent_forward) then
    attention (mla_attention_forward).  x [B,T,d_model]; q_nope [B,T,H,d_nope]; q_dir
    [B,T,H,d_dir]; weights w_dkv, w_kr, w_uk, w_uv.  Returns (o, (c, k_dir, k_nope, v))."""
    H = q_nope.shape[2]
    lat = mla_latent_forward(x, weights["w_dkv"], weights["w_kr"], weights["w_uk"], weights["w_uv"], H,
                             stream=stream)
    c, k_dir, k_nope, v = lat
    o = mla_attention_forward(q_nope, q_dir, k_nope, k_dir, v, scale=scale, stream=stream)
    return o, lat


def conv_kda_forward(desc: KdaStreamDesc, inp: dict, initial_state=None, final_state=None,
                     workspace=None, stream=None):
    """The measured path: kda_conv_forward then kda_forward on one stream.

    ``inp`` holds device tensors q, k, v, alpha, beta, w_text_{q,k,v}, w_vis_{q,k,v}.
    Returns (q', k', v', o).
    """
    qc, kc, vc = kda_conv_forward(desc, inp["q"], inp["k"], inp["v"],
                                  (inp["w_text_q"], inp["w_text_k"], inp["w_text_v"]),
                                  (inp["w_vis_q"], inp["w_vis_k"], inp["w_vis_v"]), stream=stream)
    o = kda_forward(desc, qc, kc, vc, inp["alpha"], inp["beta"], initial_state, final_state,
                    workspace=workspace, stream=stream)
    return qc, kc, vc, o
