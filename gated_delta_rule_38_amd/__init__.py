"""libkda: the Kimi Delta Attention (KDA) gated delta-rule recurrence on MI355X.

A thin Python binding over the C ABI in ``include/kda.h``.  It only checks
and marshals arguments: torch supplies device memory, output allocation and
the current stream; every step of the computation runs in the HIP kernels of
``libkda.so``.  There is no fallback: if the library is missing or was built
for another GPU, the calls fail.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["kda_chunk_fwd", "kda_chunk_fwd_gated", "kda_chunk_fwd_fused",
           "kda_chunk_fwd_noalloc", "KDA_NOALLOC_MAX_SEQS", "kda_gdn2_chunk_fwd",
           "kda_gdn2_recurrent_step", "kda_recurrent_step",
           "kda_recurrent_step_gated", "kda_recurrent_step_fused", "kda_backward",
           "kda_backward_workspace_size", "kda_chunk_fwd_workspace_size",
           "kda_chunk_fwd_split_workspace_size", "kda_status_string", "kda_version",
           "KDAError", "LIB_PATH", "load_library"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1
# forget-gate granularity (kda_gate): alpha per key channel (KDA), one alpha
# per token and head (Gated DeltaNet), or none (DeltaNet, alpha = 1)
KDA_GATE_CHANNEL = 0
KDA_GATE_HEAD = 1
KDA_GATE_NONE = 2
_GATES = {"channel": KDA_GATE_CHANNEL, "head": KDA_GATE_HEAD, "none": KDA_GATE_NONE}
# in-kernel input preparation (kda_fuse_flag)
KDA_FUSE_GATE_LOGITS = 1
KDA_FUSE_BETA_LOGITS = 2
KDA_FUSE_QK_L2NORM = 4
# packed sequences kda_chunk_fwd_noalloc accepts (its fixed device scratch)
KDA_NOALLOC_MAX_SEQS = 65536
_STATUS = {0: "KDA_SUCCESS", 1: "KDA_ERROR_INVALID_VALUE", 2: "KDA_ERROR_NOT_SUPPORTED",
           3: "KDA_ERROR_MISALIGNED", 4: "KDA_ERROR_INSUFFICIENT_WORKSPACE", 5: "KDA_ERROR_HIP"}

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: %s" % (where, kda_status_string(status)))


def load_library():
    """Load libkda.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkda.so not found at %s; build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')" % LIB_PATH)
        _lib = _bind_signatures(ctypes.CDLL(LIB_PATH))
    return _lib


def _bind_signatures(lib):
    """Argument and result types of every entry point of kda.h on ``lib``."""
    vp, fp = ctypes.c_void_p, ctypes.c_void_p
    ip = ctypes.POINTER(ctypes.c_int)
    i, f, sz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.kda_chunk_fwd.restype = i
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, i, i, i, i, i, i,
                                  vp, ip, i, f, i, vp, sz, vp]
    lib.kda_chunk_fwd_gated.restype = i
    lib.kda_chunk_fwd_gated.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, i, i, i, i, i, i, i,
                                        vp, ip, i, f, i, vp, sz, vp]
    lib.kda_chunk_fwd_noalloc.restype = i
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, i, i, i, i, i, i,
                                          vp, ip, i, f, i, vp]
    lib.kda_gdn2_chunk_fwd.restype = i
    lib.kda_gdn2_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, fp, i, i, i, i, i, i,
                                       vp, ip, i, f, i, vp, sz, vp]
    lib.kda_gdn2_recurrent_step.restype = i
    lib.kda_gdn2_recurrent_step.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, i, i, i, i, i, f,
                                            vp]
    lib.kda_recurrent_step.restype = i
    lib.kda_recurrent_step.argtypes = [vp, vp, vp, fp, fp, fp, vp, i, i, i, i, i, f, vp]
    lib.kda_recurrent_step_gated.restype = i
    lib.kda_recurrent_step_gated.argtypes = [vp, vp, vp, fp, fp, fp, vp, i, i, i, i, i, i,
                                             f, vp]
    u = ctypes.c_uint
    lib.kda_chunk_fwd_fused.restype = i
    lib.kda_chunk_fwd_fused.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, i, i, i, i, i, i, i,
                                        u, vp, ip, i, f, i, vp, sz, vp]
    lib.kda_recurrent_step_fused.restype = i
    lib.kda_recurrent_step_fused.argtypes = [vp, vp, vp, vp, fp, fp, vp, i, i, i, i, i, i,
                                             u, f, vp]
    lib.kda_backward.restype = i
    lib.kda_backward.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp, fp, fp, fp, fp, fp,
                                 i, i, i, i, i, i, vp, ip, i, f, vp, sz, vp]
    lib.kda_backward_workspace_size.restype = sz
    lib.kda_backward_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.kda_chunk_fwd_split_workspace_size.restype = sz
    lib.kda_chunk_fwd_split_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i]
    lib.kda_version.restype = i
    lib.kda_version.argtypes = []
    return lib


def kda_status_string(status):
    if _lib is None and not os.path.exists(LIB_PATH):
        return _STATUS.get(int(status), "unknown status")
    return load_library().kda_status_string(int(status)).decode()


def kda_version():
    return load_library().kda_version()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def kda_chunk_fwd_workspace_size(B, T, H, dk, dv, num_seqs, dtype=torch.bfloat16):
    code = KDA_DTYPE_BF16 if dtype == torch.bfloat16 else KDA_DTYPE_F32
    return int(load_library().kda_chunk_fwd_workspace_size(B, T, H, dk, dv, num_seqs, code))


def kda_chunk_fwd_split_workspace_size(B, T, H, dk, dv, dtype=torch.bfloat16):
    """Workspace bytes with which a dense call runs in two time segments (0: the
    shape does not qualify)."""
    code = KDA_DTYPE_BF16 if dtype == torch.bfloat16 else KDA_DTYPE_F32
    return int(load_library().kda_chunk_fwd_split_workspace_size(B, T, H, dk, dv, code))


def _gate_code(gate):
    if isinstance(gate, str):
        if gate not in _GATES:
            raise ValueError("gate must be one of %s, got %r" % (sorted(_GATES), gate))
        return _GATES[gate]
    return int(gate)


def _check_alpha(alpha, gate, lead, dk, dev, dtype=torch.float32):
    """alpha for a gate code: [*lead, dk] per channel, [*lead] per head, None."""
    if gate == KDA_GATE_NONE:
        if alpha is not None:
            raise ValueError("alpha must be None without a forget gate")
    elif gate == KDA_GATE_HEAD:
        _check(alpha, "alpha", dtype, dev, tuple(lead))
    else:
        _check(alpha, "alpha", dtype, dev, tuple(lead) + (dk,))


def _fuse_flags(gate_logits, beta_logits, qk_l2norm):
    return ((KDA_FUSE_GATE_LOGITS if gate_logits else 0) |
            (KDA_FUSE_BETA_LOGITS if beta_logits else 0) |
            (KDA_FUSE_QK_L2NORM if qk_l2norm else 0))


def kda_chunk_fwd(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None,
                  cu_seqlens_host=None, scale=None, output_final_state=True,
                  final_state=None, o=None, chunk_size=64, workspace=None, split=True):
    """Chunk-wise KDA forward.

    q, k: [B, T, H, dk]; v: [B, T, H, dv] (bf16 or fp32, same dtype);
    alpha: [B, T, H, dk] fp32; beta: [B, T, H] fp32;
    initial_state: [B or N, H, dk, dv] fp32 or None (zero start).
    Varlen: B == 1 and cu_seqlens (int32 device tensor of N+1 offsets) with
    its host copy cu_seqlens_host (list or CPU tensor; derived with a copy if
    omitted).  final_state may be passed (e.g. initial_state itself for an
    in-place update); o may be passed as a preallocated output, and
    workspace as a uint8 device tensor of at least
    kda_chunk_fwd_workspace_size() bytes (else one is allocated per call).
    With split (the default), a dense call allocates the workspace of the
    two-segment path when the shape qualifies
    (kda_chunk_fwd_split_workspace_size); split=False keeps the single pass
    (a passed workspace is then announced with its minimum size only).
    Returns (o, final_state or None).
    """
    return _chunk_fwd(q, k, v, alpha, beta, initial_state, cu_seqlens, cu_seqlens_host, scale,
                      output_final_state, final_state, o, chunk_size, workspace, None,
                      split=split)


def kda_chunk_fwd_gated(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None,
                        cu_seqlens_host=None, scale=None, output_final_state=True,
                        final_state=None, o=None, chunk_size=64, workspace=None,
                        gate="channel", split=True):
    """kda_chunk_fwd with the forget gate's granularity chosen by ``gate``:
    "channel" (alpha [B, T, H, dk], KDA), "head" (alpha [B, T, H], Gated
    DeltaNet) or "none" (alpha None, DeltaNet)."""
    return _chunk_fwd(q, k, v, alpha, beta, initial_state, cu_seqlens, cu_seqlens_host, scale,
                      output_final_state, final_state, o, chunk_size, workspace, _gate_code(gate),
                      split=split)


def kda_chunk_fwd_fused(q, k, v, gate, beta, initial_state=None, cu_seqlens=None,
                        cu_seqlens_host=None, scale=None, output_final_state=True,
                        final_state=None, o=None, chunk_size=64, workspace=None,
                        gate_kind="channel", gate_logits=True, beta_logits=True,
                        qk_l2norm=True, split=True):
    """kda_chunk_fwd_gated with the inputs prepared in the kernel: ``gate``
    holds logits (dtype of q, alpha = sigmoid) when gate_logits, else float32
    alpha; ``beta`` holds logits (beta = sigmoid) when beta_logits; q and k
    are L2-normalised per token and head when qk_l2norm."""
    return _chunk_fwd(q, k, v, gate, beta, initial_state, cu_seqlens, cu_seqlens_host, scale,
                      output_final_state, final_state, o, chunk_size, workspace,
                      _gate_code(gate_kind), _fuse_flags(gate_logits, beta_logits, qk_l2norm),
                      split=split)


def _chunk_fwd(q, k, v, alpha, beta, initial_state, cu_seqlens, cu_seqlens_host, scale,
               output_final_state, final_state, o, chunk_size, workspace, gate, flags=None,
               split=True):
    lib = load_library()
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _check(q, "q", dt, dev)
    _check(k, "k", dt, dev, (B, T, H, dk))
    _check(v, "v", dt, dev, (B, T, H, dv))
    _check_alpha(alpha, KDA_GATE_CHANNEL if gate is None else gate, (B, T, H), dk, dev,
                 dt if (flags or 0) & KDA_FUSE_GATE_LOGITS else torch.float32)
    _check(beta, "beta", torch.float32, dev, (B, T, H))
    num_seqs = 0
    cu_dev = None
    cu_host_arr = None
    if cu_seqlens is not None or cu_seqlens_host is not None:
        if cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.to("cpu")
        host = [int(x) for x in (cu_seqlens_host.tolist() if isinstance(cu_seqlens_host, torch.Tensor)
                                 else cu_seqlens_host)]
        if cu_seqlens is None:
            cu_seqlens = torch.tensor(host, dtype=torch.int32, device=dev)
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev, (len(host),))
        num_seqs = len(host) - 1
        cu_dev = cu_seqlens
        cu_host_arr = (ctypes.c_int * len(host))(*host)
    nstates = num_seqs if num_seqs > 0 else B
    sshape = (nstates, H, dk, dv)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.float32, dev, sshape)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _check(o, "o", dt, dev, (B, T, H, dv))
    if final_state is None and output_final_state:
        final_state = torch.empty(sshape, dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", torch.float32, dev, sshape)
    ws_bytes = int(lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, num_seqs, code))
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < ws_bytes:
            raise ValueError("workspace holds %d bytes, the call needs %d" % (workspace.numel(), ws_bytes))
        ws = workspace
        ws_bytes = workspace.numel() if split else ws_bytes
    else:
        if split and num_seqs == 0:
            ws_bytes = max(ws_bytes, int(lib.kda_chunk_fwd_split_workspace_size(B, T, H, dk, dv,
                                                                                code)))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    common = (float(scale) if scale is not None else 0.0, int(chunk_size), _ptr(ws), ws_bytes,
              _stream(dev))
    if flags is not None:
        st = lib.kda_chunk_fwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(initial_state), _ptr(o), _ptr(final_state),
                                     B, T, H, dk, dv, code, gate, flags, _ptr(cu_dev),
                                     cu_host_arr, num_seqs, *common)
    elif gate is None:
        st = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(initial_state), _ptr(o), _ptr(final_state),
                               B, T, H, dk, dv, code, _ptr(cu_dev), cu_host_arr, num_seqs,
                               *common)
    else:
        st = lib.kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(initial_state), _ptr(o), _ptr(final_state),
                                     B, T, H, dk, dv, code, gate, _ptr(cu_dev), cu_host_arr,
                                     num_seqs, *common)
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd_fused" if flags is not None else
                       "kda_chunk_fwd" if gate is None else "kda_chunk_fwd_gated")
    return o, final_state


def kda_chunk_fwd_noalloc(q, k, v, alpha, beta, initial_state, o, final_state=None,
                          cu_seqlens=None, cu_seqlens_host=None, scale=None, chunk_size=64):
    """kda_chunk_fwd through the entry point that allocates nothing: the caller
    passes every output (o, and final_state unless the state is not wanted)
    and, for packed sequences, both the int32 device tensor cu_seqlens and its
    host copy.  Nothing is allocated on the device, here or in the library.
    Returns (o, final_state)."""
    lib = load_library()
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _check(q, "q", dt, dev)
    _check(k, "k", dt, dev, (B, T, H, dk))
    _check(v, "v", dt, dev, (B, T, H, dv))
    _check(alpha, "alpha", torch.float32, dev, (B, T, H, dk))
    _check(beta, "beta", torch.float32, dev, (B, T, H))
    _check(o, "o", dt, dev, (B, T, H, dv))
    num_seqs, cu_host_arr = 0, None
    if (cu_seqlens is None) != (cu_seqlens_host is None):
        raise ValueError("packed sequences need both cu_seqlens and cu_seqlens_host")
    if cu_seqlens is not None:
        host = [int(x) for x in (cu_seqlens_host.tolist() if isinstance(cu_seqlens_host, torch.Tensor)
                                 else cu_seqlens_host)]
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev, (len(host),))
        num_seqs = len(host) - 1
        cu_host_arr = (ctypes.c_int * len(host))(*host)
    sshape = (num_seqs if num_seqs > 0 else B, H, dk, dv)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.float32, dev, sshape)
    if final_state is not None:
        _check(final_state, "final_state", torch.float32, dev, sshape)
    st = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                   _ptr(initial_state), _ptr(o), _ptr(final_state), B, T, H, dk,
                                   dv, code, _ptr(cu_seqlens), cu_host_arr, num_seqs,
                                   float(scale) if scale is not None else 0.0, int(chunk_size),
                                   _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd_noalloc")
    return o, final_state


def _cu(cu_seqlens, cu_seqlens_host, dev):
    """(num_seqs, device tensor, host int array) of optional packed-sequence offsets."""
    if cu_seqlens is None and cu_seqlens_host is None:
        return 0, None, None
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.to("cpu")
    host = [int(x) for x in (cu_seqlens_host.tolist() if isinstance(cu_seqlens_host, torch.Tensor)
                             else cu_seqlens_host)]
    if cu_seqlens is None:
        cu_seqlens = torch.tensor(host, dtype=torch.int32, device=dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev, (len(host),))
    return len(host) - 1, cu_seqlens, (ctypes.c_int * len(host))(*host)


def kda_gdn2_chunk_fwd(q, k, v, alpha, erase, write, initial_state=None, cu_seqlens=None,
                       cu_seqlens_host=None, scale=None, output_final_state=True,
                       final_state=None, o=None, chunk_size=64, workspace=None):
    """Chunk-wise Gated DeltaNet-2 forward: q, k [B, T, H, dk] and v [B, T, H, dv]
    bf16; alpha (or None: no forget gate), erase and write [B, T, H, dk] fp32;
    initial_state [B or N, H, dk, dv] fp32 or None; varlen and outputs as for
    kda_chunk_fwd.  Returns (o, final_state or None)."""
    lib = load_library()
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _check(q, "q", dt, dev)
    _check(k, "k", dt, dev, (B, T, H, dk))
    _check(v, "v", dt, dev, (B, T, H, dv))
    if alpha is not None:
        _check(alpha, "alpha", torch.float32, dev, (B, T, H, dk))
    _check(erase, "erase", torch.float32, dev, (B, T, H, dk))
    _check(write, "write", torch.float32, dev, (B, T, H, dk))
    num_seqs, cu_dev, cu_host = _cu(cu_seqlens, cu_seqlens_host, dev)
    sshape = (num_seqs if num_seqs > 0 else B, H, dk, dv)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.float32, dev, sshape)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _check(o, "o", dt, dev, (B, T, H, dv))
    if final_state is None and output_final_state:
        final_state = torch.empty(sshape, dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", torch.float32, dev, sshape)
    ws_bytes = int(lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, num_seqs, code))
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < ws_bytes:
            raise ValueError("workspace holds %d bytes, the call needs %d" % (workspace.numel(), ws_bytes))
        ws, ws_bytes = workspace, workspace.numel()
    else:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = lib.kda_gdn2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase), _ptr(write),
                                _ptr(initial_state), _ptr(o), _ptr(final_state), B, T, H, dk, dv,
                                code, _ptr(cu_dev), cu_host, num_seqs,
                                float(scale) if scale is not None else 0.0, int(chunk_size),
                                _ptr(ws), ws_bytes, _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_gdn2_chunk_fwd")
    return o, final_state


def kda_gdn2_recurrent_step(q, k, v, alpha, erase, write, state, scale=None, o=None):
    """One Gated DeltaNet-2 decode step; ``state`` [N, H, dk, dv] fp32 is updated
    in place.  q, k [N, H, dk]; v [N, H, dv]; alpha (or None), erase, write
    [N, H, dk] fp32.  Returns o [N, H, dv]."""
    lib = load_library()
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    _check(q, "q", dt, dev)
    _check(k, "k", dt, dev, (N, H, dk))
    _check(v, "v", dt, dev, (N, H, dv))
    if alpha is not None:
        _check(alpha, "alpha", torch.float32, dev, (N, H, dk))
    _check(erase, "erase", torch.float32, dev, (N, H, dk))
    _check(write, "write", torch.float32, dev, (N, H, dk))
    _check(state, "state", torch.float32, dev, (N, H, dk, dv))
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _check(o, "o", dt, dev, (N, H, dv))
    st = lib.kda_gdn2_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase),
                                     _ptr(write), _ptr(state), _ptr(o), N, H, dk, dv, code,
                                     float(scale) if scale is not None else 0.0, _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_gdn2_recurrent_step")
    return o


def kda_backward_workspace_size(B, T, H, dk, dv, num_seqs, dtype=torch.bfloat16):
    code = KDA_DTYPE_BF16 if dtype == torch.bfloat16 else KDA_DTYPE_F32
    return int(load_library().kda_backward_workspace_size(B, T, H, dk, dv, num_seqs, code))


def kda_backward(q, k, v, alpha, beta, initial_state, dout, dfinal_state=None,
                 cu_seqlens=None, cu_seqlens_host=None, scale=None, workspace=None, out=None):
    """Gradients of kda_chunk_fwd (per-channel gate): dout [B, T, H, dv] in the
    dtype of q, dfinal_state [B or N, H, dk, dv] float32 or None.  Returns
    float32 (dq, dk, dv, dalpha, dbeta, dinitial_state), written into ``out``
    (a tuple of those six tensors, contiguous, float32) when given."""
    lib = load_library()
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _check(q, "q", dt, dev)
    _check(k, "k", dt, dev, (B, T, H, dk))
    _check(v, "v", dt, dev, (B, T, H, dv))
    _check(alpha, "alpha", torch.float32, dev, (B, T, H, dk))
    _check(beta, "beta", torch.float32, dev, (B, T, H))
    _check(dout, "dout", dt, dev, (B, T, H, dv))
    num_seqs, cu_dev, cu_host_arr = 0, None, None
    if cu_seqlens is not None or cu_seqlens_host is not None:
        if cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.to("cpu")
        host = [int(x) for x in (cu_seqlens_host.tolist() if isinstance(cu_seqlens_host, torch.Tensor)
                                 else cu_seqlens_host)]
        if cu_seqlens is None:
            cu_seqlens = torch.tensor(host, dtype=torch.int32, device=dev)
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev, (len(host),))
        num_seqs = len(host) - 1
        cu_dev = cu_seqlens
        cu_host_arr = (ctypes.c_int * len(host))(*host)
    nstates = num_seqs if num_seqs > 0 else B
    sshape = (nstates, H, dk, dv)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.float32, dev, sshape)
    if dfinal_state is not None:
        _check(dfinal_state, "dfinal_state", torch.float32, dev, sshape)
    f32 = dict(dtype=torch.float32, device=dev)
    shapes = ((B, T, H, dk), (B, T, H, dk), (B, T, H, dv), (B, T, H, dk), (B, T, H), sshape)
    if out is not None:
        g = tuple(out)
        names = ("dq", "dk", "dv", "dalpha", "dbeta", "dinitial_state")
        if len(g) != 6:
            raise ValueError("out holds %d tensors, kda_backward writes 6" % len(g))
        for x, n, shp in zip(g, names, shapes):
            _check(x, n, torch.float32, dev, shp)
    else:
        g = tuple(torch.empty(shp, **f32) for shp in shapes)
    ws_bytes = int(lib.kda_backward_workspace_size(B, T, H, dk, dv, num_seqs, code))
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < ws_bytes:
            raise ValueError("workspace holds %d bytes, the call needs %d" % (workspace.numel(), ws_bytes))
        ws, ws_bytes = workspace, workspace.numel()
    else:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = lib.kda_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state),
                          _ptr(dout), _ptr(dfinal_state), *[_ptr(x) for x in g],
                          B, T, H, dk, dv, code, _ptr(cu_dev), cu_host_arr, num_seqs,
                          float(scale) if scale is not None else 0.0, _ptr(ws), ws_bytes,
                          _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_backward")
    return g


def kda_recurrent_step(q, k, v, alpha, beta, state, scale=None, o=None):
    """One decode step; ``state`` [N, H, dk, dv] fp32 is updated in place.
    q, k: [N, H, dk]; v: [N, H, dv]; alpha: [N, H, dk] fp32; beta: [N, H] fp32.
    Returns o [N, H, dv]."""
    return _recurrent_step(q, k, v, alpha, beta, state, scale, o, None)


def kda_recurrent_step_gated(q, k, v, alpha, beta, state, scale=None, o=None, gate="channel"):
    """kda_recurrent_step with the forget gate's granularity chosen by ``gate``:
    "channel" (alpha [N, H, dk]), "head" (alpha [N, H]) or "none" (alpha None)."""
    return _recurrent_step(q, k, v, alpha, beta, state, scale, o, _gate_code(gate))


def kda_recurrent_step_fused(q, k, v, gate, beta, state, scale=None, o=None, gate_kind="channel",
                             gate_logits=True, beta_logits=True, qk_l2norm=True):
    """kda_recurrent_step_gated with the inputs prepared in the kernel (flags as
    for kda_chunk_fwd_fused)."""
    return _recurrent_step(q, k, v, gate, beta, state, scale, o, _gate_code(gate_kind),
                           _fuse_flags(gate_logits, beta_logits, qk_l2norm))


def _recurrent_step(q, k, v, alpha, beta, state, scale, o, gate, flags=None):
    lib = load_library()
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    _check(q, "q", dt, dev)
    _check(k, "k", dt, dev, (N, H, dk))
    _check(v, "v", dt, dev, (N, H, dv))
    _check_alpha(alpha, KDA_GATE_CHANNEL if gate is None else gate, (N, H), dk, dev,
                 dt if (flags or 0) & KDA_FUSE_GATE_LOGITS else torch.float32)
    _check(beta, "beta", torch.float32, dev, (N, H))
    _check(state, "state", torch.float32, dev, (N, H, dk, dv))
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _check(o, "o", dt, dev, (N, H, dv))
    sc = float(scale) if scale is not None else 0.0
    if flags is not None:
        st = lib.kda_recurrent_step_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                          _ptr(state), _ptr(o), N, H, dk, dv, code, gate, flags,
                                          sc, _stream(dev))
    elif gate is None:
        st = lib.kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(state), _ptr(o), N, H, dk, dv, code, sc, _stream(dev))
    else:
        st = lib.kda_recurrent_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                          _ptr(state), _ptr(o), N, H, dk, dv, code, gate, sc,
                                          _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_recurrent_step_fused" if flags is not None else
                       "kda_recurrent_step" if gate is None else "kda_recurrent_step_gated")
    return o
