"""ctypes binding of libvda.so (Video Delta Attention forward on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libvda.so.  The functions mirror the C ABI in include/vda.h and
have the same names; tensors are torch tensors on the GPU (their data_ptr() is
passed), and the stream defaults to torch's current stream.  There is no CPU
fallback: when the library is missing or no GPU is present these functions
raise.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvda.so")

VDA_OK = 0
VDA_ERR_INVALID_ARG = -1
VDA_ERR_BAD_DTYPE = -2
VDA_ERR_WORKSPACE_TOO_SMALL = -3
VDA_ERR_MISALIGNED = -4
VDA_ERR_HIP = -5
VDA_ERR_SCRATCH_TOO_SMALL = -6
VDA_ERR_NOT_SPD = -7
VDA_NOALLOC_MAX_BYTES = 64 << 20  # the fixed scratch of vda_forward_noalloc
VDA_DTYPE_F32 = 0
VDA_DTYPE_BF16 = 1

EXPORTED = ("vda_workspace_bytes", "vda_check_desc", "vda_forward", "vda_forward_noalloc",
            "vda_forward_timed",
            "vda_forward_decay", "vda_debug_stats", "vda_debug_solve", "vda_debug_frame_maps",
            "vda_debug_chunks",
            "vda_debug_chunks_decay", "vda_debug_states", "vda_debug_states_decay",
            "vda_prep", "vda_prep_check_desc", "vda_status_string")


class VdaDesc(ctypes.Structure):
    """vda_desc_t of include/vda.h."""
    _fields_ = [
        ("units", ctypes.c_int32), ("frames", ctypes.c_int32), ("tokens", ctypes.c_int32),
        ("text_tokens", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("chunk", ctypes.c_int32), ("radius", ctypes.c_int32), ("rms_eps", ctypes.c_float),
        ("seed_mode", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("anchors", ctypes.c_int32), ("rule", ctypes.c_int32),
        ("fp32_products", ctypes.c_int32), ("solver", ctypes.c_int32),
        ("q_heads", ctypes.c_int32), ("q_l2_eps", ctypes.c_float),
    ]

    @property
    def n_chunks(self):
        return -(-self.frames // self.chunk) if self.frames > 0 else 0


class VdaPrepDesc(ctypes.Structure):
    """vda_prep_desc_t of include/vda.h."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("frames", ctypes.c_int32),
        ("height", ctypes.c_int32), ("width", ctypes.c_int32), ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32), ("eps", ctypes.c_float), ("dtype", ctypes.c_int32),
    ]


class VdaError(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, vda_status_string(status), status))


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libvda.so (once).  Raises when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libvda.so is not built (%s); run `python -m "
                           "frame_wise_delta_gram_amd.build`" % path)
    try:  # bind to the HIP runtime torch already uses (one runtime per process)
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(VdaDesc)
    lib.vda_workspace_bytes.argtypes = [D]
    lib.vda_workspace_bytes.restype = ctypes.c_size_t
    lib.vda_check_desc.argtypes = [D]
    lib.vda_check_desc.restype = ctypes.c_int
    lib.vda_forward.argtypes = [D] + [P] * 11 + [ctypes.c_size_t, P]
    lib.vda_forward.restype = ctypes.c_int
    lib.vda_forward_noalloc.argtypes = [D] + [P] * 10 + [P]
    lib.vda_forward_noalloc.restype = ctypes.c_int
    lib.vda_forward_timed.argtypes = [D] + [P] * 12 + [ctypes.c_size_t, P,
                                                      ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.vda_forward_timed.restype = ctypes.c_int
    lib.vda_forward_decay.argtypes = [D] + [P] * 12 + [ctypes.c_size_t, P]
    lib.vda_forward_decay.restype = ctypes.c_int
    lib.vda_debug_chunks_decay.argtypes = [D] + [P] * 12 + [ctypes.c_size_t, P]
    lib.vda_debug_chunks_decay.restype = ctypes.c_int
    lib.vda_debug_states_decay.argtypes = [D] + [P] * 10 + [ctypes.c_size_t, P]
    lib.vda_debug_states_decay.restype = ctypes.c_int
    lib.vda_debug_stats.argtypes = [D] + [P] * 9 + [ctypes.c_size_t, P]
    lib.vda_debug_stats.restype = ctypes.c_int
    lib.vda_debug_solve.argtypes = [D] + [P] * 9 + [ctypes.c_size_t, P]
    lib.vda_debug_solve.restype = ctypes.c_int
    lib.vda_debug_frame_maps.argtypes = [D] + [P] * 10 + [ctypes.c_size_t, P]
    lib.vda_debug_frame_maps.restype = ctypes.c_int
    lib.vda_debug_chunks.argtypes = [D] + [P] * 10 + [ctypes.c_size_t, P]
    lib.vda_debug_chunks.restype = ctypes.c_int
    lib.vda_debug_states.argtypes = [D] + [P] * 9 + [ctypes.c_size_t, P]
    lib.vda_debug_states.restype = ctypes.c_int
    DP = ctypes.POINTER(VdaPrepDesc)
    lib.vda_prep_check_desc.argtypes = [DP]
    lib.vda_prep_check_desc.restype = ctypes.c_int
    lib.vda_prep.argtypes = [DP] + [P] * 10 + [P]
    lib.vda_prep.restype = ctypes.c_int
    lib.vda_status_string.argtypes = [ctypes.c_int]
    lib.vda_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def vda_status_string(status: int) -> str:
    return load_library().vda_status_string(int(status)).decode()


def make_desc(units, frames, tokens, text_tokens, d_k, d_v, chunk=5, radius=1, rms_eps=1e-6,
              seed_mode=0, dtype=VDA_DTYPE_BF16, anchors=0, rule=0, fp32_products=0,
              solver=0, q_heads=0, q_l2_eps=0.0) -> VdaDesc:
    return VdaDesc(units, frames, tokens, text_tokens, d_k, d_v, chunk, radius, rms_eps,
                   seed_mode, dtype, dtype, int(anchors), int(rule), int(fp32_products),
                   int(solver), int(q_heads), float(q_l2_eps))


def vda_workspace_bytes(desc: VdaDesc) -> int:
    return int(load_library().vda_workspace_bytes(ctypes.byref(desc)))


def vda_check_desc(desc: VdaDesc) -> int:
    return int(load_library().vda_check_desc(ctypes.byref(desc)))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr() if x.numel() > 0 else None


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, fn):
    if status != VDA_OK:
        raise VdaError(status, fn)


def vda_forward(desc, q, k, v, beta, gate, text_k, text_v, text_beta, rms_weight, out,
                workspace, workspace_bytes=None, stream=None):
    """C vda_forward: enqueue the forward pass on `stream` (torch's current by default)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().vda_forward(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gate), _ptr(text_k),
        _ptr(text_v), _ptr(text_beta), _ptr(rms_weight), _ptr(out), _ptr(workspace),
        workspace_bytes, _stream(stream))
    _check(st, "vda_forward")


def vda_forward_noalloc(desc, q, k, v, beta, gate, text_k, text_v, text_beta, rms_weight, out,
                        stream=None):
    """C vda_forward_noalloc: vda_forward in the library's fixed per-GPU scratch
    (no workspace argument, nothing allocated; problems whose workspace exceeds
    VDA_NOALLOC_MAX_BYTES are refused)."""
    st = load_library().vda_forward_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gate), _ptr(text_k),
        _ptr(text_v), _ptr(text_beta), _ptr(rms_weight), _ptr(out), _stream(stream))
    _check(st, "vda_forward_noalloc")


def vda_forward_timed(desc, q, k, v, beta, alpha, gate, text_k, text_v, text_beta, rms_weight,
                      out, workspace, stage_events, workspace_bytes=None, stream=None):
    """C vda_forward_timed: as vda_forward (alpha None) or vda_forward_decay,
    recording the six caller-created hipEvent_t handles (ints) in
    ``stage_events`` at the stage boundaries (None or 0 skips a boundary)."""
    ev = (ctypes.c_void_p * 6)(*[int(e) if e else None for e in stage_events])
    st = load_library().vda_forward_timed(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(gate),
        _ptr(text_k), _ptr(text_v), _ptr(text_beta), _ptr(rms_weight), _ptr(out),
        _ptr(workspace), _ws_bytes(workspace, workspace_bytes), _stream(stream), ev,
        len(stage_events))
    _check(st, "vda_forward_timed")


def vda_forward_decay(desc, q, k, v, beta, alpha, gate, text_k, text_v, text_beta, rms_weight,
                      out, workspace, workspace_bytes=None, stream=None):
    """C vda_forward_decay: vda_forward with channel-wise decay gates alpha
    [units, F, d_k] (float32)."""
    st = load_library().vda_forward_decay(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(gate),
        _ptr(text_k), _ptr(text_v), _ptr(text_beta), _ptr(rms_weight), _ptr(out),
        _ptr(workspace), _ws_bytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "vda_forward_decay")


def _ws_bytes(workspace, workspace_bytes):
    if workspace_bytes is not None:
        return workspace_bytes
    return workspace.numel() * workspace.element_size() if workspace is not None else 0


def vda_debug_stats(desc, k, v, beta, text_k, text_v, text_beta, A_out, B_out, workspace,
                    workspace_bytes=None, stream=None):
    st = load_library().vda_debug_stats(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(beta), _ptr(text_k), _ptr(text_v),
        _ptr(text_beta), _ptr(A_out), _ptr(B_out), _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "vda_debug_stats")


def vda_debug_solve(desc, k, v, beta, text_k, text_v, text_beta, M_out, seed_out, workspace,
                    workspace_bytes=None, stream=None):
    st = load_library().vda_debug_solve(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(beta), _ptr(text_k), _ptr(text_v),
        _ptr(text_beta), _ptr(M_out), _ptr(seed_out), _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "vda_debug_solve")


def vda_debug_frame_maps(desc, k, v, beta, text_k, text_v, text_beta, M_out, J_out, not_spd,
                         workspace, workspace_bytes=None, stream=None):
    """C vda_debug_frame_maps: per-frame M_t and J_t = B_t M_t; not_spd (an int32
    GPU tensor of one element, or None) receives VDA_ERR_NOT_SPD when a pivot of
    some I + A_t is not positive."""
    st = load_library().vda_debug_frame_maps(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(beta), _ptr(text_k), _ptr(text_v),
        _ptr(text_beta), _ptr(M_out), _ptr(J_out), _ptr(not_spd), _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "vda_debug_frame_maps")


def vda_debug_chunks(desc, k, v, beta, text_k, text_v, text_beta, Mc_out, Jf_out, Jr_out,
                     workspace, workspace_bytes=None, stream=None):
    st = load_library().vda_debug_chunks(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(beta), _ptr(text_k), _ptr(text_v),
        _ptr(text_beta), _ptr(Mc_out), _ptr(Jf_out), _ptr(Jr_out), _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "vda_debug_chunks")


def vda_debug_states(desc, k, v, beta, text_k, text_v, text_beta, P_out, R_out, workspace,
                     workspace_bytes=None, stream=None):
    st = load_library().vda_debug_states(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(beta), _ptr(text_k), _ptr(text_v),
        _ptr(text_beta), _ptr(P_out), _ptr(R_out), _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "vda_debug_states")


def vda_debug_chunks_decay(desc, k, v, beta, alpha, text_k, text_v, text_beta, Mc_out, Mr_t_out,
                           Jf_out, Jr_out, workspace, workspace_bytes=None, stream=None):
    st = load_library().vda_debug_chunks_decay(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(text_k),
        _ptr(text_v), _ptr(text_beta), _ptr(Mc_out), _ptr(Mr_t_out), _ptr(Jf_out), _ptr(Jr_out),
        _ptr(workspace), _ws_bytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "vda_debug_chunks_decay")


def vda_debug_states_decay(desc, k, v, beta, alpha, text_k, text_v, text_beta, P_out, R_out,
                           workspace, workspace_bytes=None, stream=None):
    st = load_library().vda_debug_states_decay(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(text_k),
        _ptr(text_v), _ptr(text_beta), _ptr(P_out), _ptr(R_out), _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "vda_debug_states_decay")


def make_prep_desc(batch, heads, frames, height, width, d_k, d_v, eps=1e-6,
                   dtype=VDA_DTYPE_BF16) -> VdaPrepDesc:
    return VdaPrepDesc(batch, heads, frames, height, width, d_k, d_v, eps, dtype)


def vda_prep_check_desc(desc: VdaPrepDesc) -> int:
    return int(load_library().vda_prep_check_desc(ctypes.byref(desc)))


def vda_prep(desc, q, k, v, wk_s, wk_t, wv_s, wv_t, q_out, k_out, v_out, stream=None):
    """C vda_prep: the feature map from projection outputs to prepared features
    (q and q_out both None: K' and V' only, the query map left to the readout)."""
    st = load_library().vda_prep(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(wk_s), _ptr(wk_t), _ptr(wv_s),
        _ptr(wv_t), _ptr(q_out), _ptr(k_out), _ptr(v_out), _stream(stream))
    _check(st, "vda_prep")


# ----------------------------------------------------------------------------- torch helpers
def desc_from_tensors(q, k, v, text_k, chunk=5, radius=1, eps=1e-6, seed_mode=0,
                      anchors=False, rule=0, fp32_products=0, solver=0, q_heads=0,
                      q_l2_eps=0.0) -> VdaDesc:
    """Descriptor from tensor shapes: q/k [units, F, U, d_k], v [units, F, U, d_v],
    text_k [units, T, d_k]."""
    import torch
    units, F, U, dk = k.shape
    dv = v.shape[-1]
    if text_k is not None and (not isinstance(text_k, torch.Tensor) or text_k.dim() != 3):
        raise TypeError("text_k: expected a 3-d torch tensor [units, T, d_k] or None")
    T = text_k.shape[1] if text_k is not None else 0
    if k.dtype == torch.bfloat16:
        dt = VDA_DTYPE_BF16
    elif k.dtype == torch.float32:
        dt = VDA_DTYPE_F32
    else:
        raise TypeError("features must be bfloat16 or float32, got %s" % k.dtype)
    return make_desc(units, F, U, T, dk, dv, chunk, radius, eps, seed_mode, dt, anchors, rule,
                     fp32_products, solver, q_heads, q_l2_eps)


def _check_tensor(name, x, dtype, shape, device=None):
    """Raise TypeError / ValueError unless x is a torch tensor of this dtype and
    shape that is contiguous and on the GPU (on `device` when given); empty
    tensors are accepted wherever they live (no pointer of theirs is used)."""
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s: expected a torch tensor, got %s" % (name, type(x).__name__))
    if x.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, x.dtype))
    if tuple(x.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(x.shape)))
    if x.numel() > 0:
        if not x.is_cuda or not x.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
        if device is not None and x.device != device:
            raise ValueError("%s is on %s, the features on %s" % (name, x.device, device))


def forward(q, k, v, beta, gate, text_k, text_v, text_beta, rms_weight, chunk=5, radius=1,
            eps=1e-6, seed_mode=0, out=None, workspace=None, stream=None, alpha=None,
            anchors=False, rule=0, fp32_products=0, solver=0, q_heads=0, q_l2_eps=0.0):
    """VDA forward on torch GPU tensors; allocates `out` and the workspace when absent.

    Shapes: q, k [units, F, U, d_k]; v, gate [units, F, U, d_v]; beta [units, F, U]
    (float32); text_k [units, T, d_k]; text_v [units, T, d_v]; text_beta
    [units, T] (float32), all three None for no text (T = 0); rms_weight [d_v]
    (float32); alpha (optional decay gates) [units, F, d_k] (float32); anchors:
    boundary anchors (frames 0 and F - 1 out of the linear states, their rows
    zero); rule: 0 the frame-wise delta rule, 1 / 2 the batched comparison rules
    (no decay); fp32_products: composition and scan on fp32 MFMA for bf16
    features; solver: 0 symmetric Gauss-Jordan, 1 blocked Cholesky; q_heads = H > 1:
    q in the projection layout [units / H, F, U, H, d_k] (heads interleaved per
    token); q_l2_eps > 0: each query row L2-normalised inside the readout (the
    feature map's query map).  A caller-supplied `out` must be [units, F, U, d_v] in the
    features' dtype, a caller-supplied workspace a contiguous uint8 tensor on the
    features' GPU.  Every tensor is checked (dtype, shape, device, contiguity)
    before anything is enqueued: a mismatch raises TypeError or ValueError.
    Returns out [units, F, U, d_v] in the features' dtype.
    """
    import torch
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise TypeError("k: expected a 4-d torch tensor [units, F, U, d_k]")
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise TypeError("v: expected a 4-d torch tensor [units, F, U, d_v]")
    if (text_k is None) != (text_v is None) or (text_k is None) != (text_beta is None):
        raise ValueError("text_k, text_v and text_beta are given together or all None")
    desc = desc_from_tensors(q, k, v, text_k, chunk, radius, eps, seed_mode, anchors, rule,
                             fp32_products, solver, q_heads, q_l2_eps)
    units, F, U, dk = k.shape
    dv = v.shape[-1]
    T = desc.text_tokens
    fdt = k.dtype
    dev = k.device
    H = int(q_heads) if int(q_heads) > 1 else 1
    if units % H:
        raise ValueError("q_heads = %d does not divide units = %d" % (H, units))
    qshape = (units, F, U, dk) if H == 1 else (units // H, F, U, H, dk)
    checks = [("k", k, fdt, (units, F, U, dk)), ("q", q, fdt, qshape),
              ("v", v, fdt, (units, F, U, dv)), ("gate", gate, fdt, (units, F, U, dv)),
              ("beta", beta, torch.float32, (units, F, U))]
    if text_k is not None:
        checks += [("text_k", text_k, fdt, (units, T, dk)), ("text_v", text_v, fdt, (units, T, dv)),
                   ("text_beta", text_beta, torch.float32, (units, T))]
    if alpha is not None:
        checks.append(("alpha", alpha, torch.float32, (units, F, dk)))
    if out is not None:
        checks.append(("out", out, fdt, (units, F, U, dv)))
    for name, x, dt, shp in checks:
        _check_tensor(name, x, dt, shp, dev)
    # the RMSNorm weight is read only when there are rows to write
    _check_tensor("rms_weight", rms_weight if units * F * U > 0 else rms_weight[:0],
                  torch.float32, (dv,) if units * F * U > 0 else (0,), dev)
    nbytes = vda_workspace_bytes(desc)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8:
            raise TypeError("workspace: expected a torch.uint8 tensor")
        if nbytes > 0 and (not workspace.is_cuda or workspace.device != dev
                           or not workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    if out is None:
        out = torch.empty((units, F, U, dv), dtype=fdt, device=dev)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)  # empty: NULL
    if alpha is None:
        vda_forward(desc, q, k, v, beta, gate, text_k, text_v, text_beta, rms_weight, out,
                    workspace, stream=stream)
    else:
        vda_forward_decay(desc, q, k, v, beta, alpha, gate, text_k, text_v, text_beta,
                          rms_weight, out, workspace, stream=stream)
    return out
