"""MI355X (gfx950) lightning attention: causal decayed linear attention.

Thin ctypes binding over liblightning_attn.so (C ABI in include/lightning_attn.h).
This layer only checks and marshals arguments: every step of the computation
runs in the library's HIP kernels.  torch supplies device memory and the
current stream.  If the library has not been built the calls raise; there is
no CPU fallback.

    out = fwd(q, k, v, decay, kv_in=None, kv_out=None, block=64)
    o   = decode_step(q, k, v, decay, kv_in, kv_out)
    dq, dk, dv, dkv_in = bwd(q, k, v, decay, dout)
    out, kv_out = lightning_attn(q, k, v, decay, kv_in)   # differentiable (autograd)

block 64 is the tuned path; 128 and 256 give the same result up to rounding
through a general, slower kernel.
"""
import contextlib
import ctypes
import os

import torch

__all__ = [
    "LIB_PATH",
    "LightningAttnError",
    "load",
    "LA_FLAG_EXACT",
    "LA_FLAG_SILU_QKV",
    "fwd",
    "fwd_noalloc",
    "fwd_fused",
    "NOALLOC_SCRATCH_BYTES",
    "fwd_slots",
    "bwd",
    "lightning_attn",
    "decode_step",
    "decode_slots",
    "decode_fused",
    "decode_layers",
    "norm_gate",
    "silu_",
    "workspace_bytes",
    "lib_bwd_workspace_bytes",
    "chunk_for",
    "warm_chunk_for",
    "runtime_version",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblightning_attn.so")

LA_DTYPE_BF16 = 0
LA_DTYPE_F32 = 1
LA_FLAG_EXACT = 1
LA_FLAG_SILU_QKV = 2
NOALLOC_SCRATCH_BYTES = 96 * 1024 * 1024  # LA_NOALLOC_SCRATCH_BYTES
_DT = {torch.bfloat16: LA_DTYPE_BF16, torch.float32: LA_DTYPE_F32}

_lib = None


class LightningAttnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, _strerror(status), status))


def load():
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "liblightning_attn.so is not built (%s); run "
            "`python -m long_context_decayed_amd.build`" % LIB_PATH
        )
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    fwd_args = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64]
    for name in ("lightning_attn_fwd", "lightning_attn_fwd_f32", "lightning_attn_fwd_bf16_f32out"):
        fn = getattr(lib, name)
        fn.restype = I
        fn.argtypes = fwd_args + [P]
    lib.lightning_attn_fwd_ex.restype = I
    lib.lightning_attn_fwd_ex.argtypes = fwd_args + [I, I, I64, I64, ctypes.c_uint, P, SZ, P, P, P]
    lib.lightning_attn_fwd_fused.restype = I
    lib.lightning_attn_fwd_fused.argtypes = [P] * 5 + [ctypes.c_float, P, P, P, P, I64, I64, I64, I64, I, I64, I64,
                                                       ctypes.c_uint, P, SZ, P, P, P]
    lib.lightning_attn_fwd_noalloc.restype = I
    lib.lightning_attn_fwd_noalloc.argtypes = [P] * 7 + [I64, I64, I64, I64, I, I, I64, I64, ctypes.c_uint, P]
    lib.lightning_attn_fwd_chunk.restype = I64
    lib.lightning_attn_fwd_chunk.argtypes = [I64, I64, I64, I64, I64]
    lib.lightning_attn_fwd_warm_chunk.restype = I64
    lib.lightning_attn_fwd_warm_chunk.argtypes = [I64, I64, I64, I64, I64, I64]
    lib.lightning_attn_fwd_workspace_bytes.restype = SZ
    lib.lightning_attn_fwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I64]
    lib.lightning_attn_fwd_workspace_bytes_ex.restype = SZ
    lib.lightning_attn_fwd_workspace_bytes_ex.argtypes = [I64, I64, I64, I64, I64, I64]
    lib.lightning_attn_decode_step.restype = I
    lib.lightning_attn_decode_step.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, P]
    lib.lightning_attn_decode_fused.restype = I
    lib.lightning_attn_decode_fused.argtypes = [P] * 7 + [I64, I, P, ctypes.c_float, P, I64, I64, I64, P]
    lib.lightning_attn_decode_layers.restype = I
    lib.lightning_attn_decode_layers.argtypes = [P] * 7 + [I64, I64, I64, I64, I64, I, P, ctypes.c_float, P, P]
    lib.lightning_attn_norm_gate.restype = I
    lib.lightning_attn_norm_gate.argtypes = [P, I, P, P, ctypes.c_float, P, I64, I64, I64, I64, P]
    lib.lightning_attn_silu.restype = I
    lib.lightning_attn_silu.argtypes = [P, I64, P]
    lib.lightning_attn_fwd_slots.restype = I
    lib.lightning_attn_fwd_slots.argtypes = [P] * 7 + [I64, I64, I64, I64, I64, I64, I, I, ctypes.c_uint, P]
    lib.lightning_attn_bwd.restype = I
    lib.lightning_attn_bwd.argtypes = [P] * 11 + [I64, I64, I64, I64, I, I, ctypes.c_uint, P, SZ, P]
    lib.lightning_attn_bwd_workspace_bytes.restype = SZ
    lib.lightning_attn_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64]
    lib.lightning_attn_decode_slots.restype = I
    lib.lightning_attn_decode_slots.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, P]
    lib.lightning_attn_strerror.restype = ctypes.c_char_p
    lib.lightning_attn_strerror.argtypes = [I]
    lib.lightning_attn_runtime_version.restype = I
    lib.lightning_attn_runtime_version.argtypes = [ctypes.POINTER(ctypes.c_int)]
    _lib = lib
    return lib


def _strerror(status):
    try:
        return load().lightning_attn_strerror(int(status)).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return "status %d" % status


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _device_of(name, t):
    """The device of the tensor that anchors a call (every other tensor of the
    call must be on it)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    return t.device


def _current(device):
    """Makes the call's device the current one for the library call (a no-op
    when it already is)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif stream.device != device:
        raise ValueError("stream is on %s, the tensors on %s" % (stream.device, device))
    return ctypes.c_void_p(stream.cuda_stream)


def _check_dev(name, t, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, the call's tensors on %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def chunk_for(B, H, N, block=64, chunk=0):
    """Chunk length the library uses (chunk=0: its default)."""
    return int(load().lightning_attn_fwd_chunk(B, H, N, block, chunk))


def warm_chunk_for(B, H, N, block=64, chunk=0, warm_chunk=0):
    """Warm-start chunk length the library uses (0s: its defaults)."""
    return int(load().lightning_attn_fwd_warm_chunk(B, H, N, block, chunk, warm_chunk))


def lib_bwd_workspace_bytes(B, H, N, d):
    return int(load().lightning_attn_bwd_workspace_bytes(B, H, N, d))


def workspace_bytes(B, H, N, d, block=64, chunk=0):
    return int(load().lightning_attn_fwd_workspace_bytes_ex(B, H, N, d, block, chunk))


def _fwd_flags(exact, silu):
    return (LA_FLAG_EXACT if exact else 0) | (LA_FLAG_SILU_QKV if silu else 0)


def fwd(q, k, v, decay, kv_in=None, kv_out=None, block=64, out=None, out_dtype=None, chunk=0,
        workspace=None, events=None, exact=False, silu=False, warm_chunk=0, stream=None):
    """Prefill.  q, k, v: [B, H, N, d] bf16 or fp32 device tensors; decay: fp32 [H];
    kv_in / kv_out: fp32 [B, H, d, d] or None.  Returns out [B, H, N, d] in
    out_dtype (default: the input dtype).

    workspace: a uint8 device tensor of at least workspace_bytes(...) bytes;
    None allocates one from torch's caching allocator.  events: optional pair
    of hipEvent_t handles (ints) recorded around the kernel that writes every
    output row.  exact: every head by the exact chunked path (no warm start).
    silu: q, k, v are pre-activations; SiLU is applied inside the kernels as
    their tiles load (bf16, block 64), q, k, v themselves are not changed.
    warm_chunk: chunk of the warm-start pass (0: the library's default,
    warm_chunk_for)."""
    lib = load()
    dev = _device_of("q", q)
    if q.dtype not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype, (B, H, N, d), device=dev)
    _check_dev("decay", decay, torch.float32, (H,), device=dev)
    for name, t in (("kv_in", kv_in), ("kv_out", kv_out)):
        if t is not None:
            _check_dev(name, t, torch.float32, (B, H, d, d), device=dev)
    odt = out_dtype if out_dtype is not None else (out.dtype if out is not None else q.dtype)
    if odt not in _DT:
        raise TypeError("out dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((B, H, N, d), device=q.device, dtype=odt)
    _check_dev("out", out, odt, (B, H, N, d), device=dev)
    need = int(lib.lightning_attn_fwd_workspace_bytes_ex(B, H, N, d, block, chunk))
    if need == 0:
        raise LightningAttnError(1, "lightning_attn_fwd_workspace_bytes_ex")
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    _check_dev("workspace", workspace, torch.uint8, device=dev)
    e0, e1 = (None, None) if events is None else (ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    with _current(dev):
        rc = lib.lightning_attn_fwd_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(out), _ptr(kv_in), _ptr(kv_out),
            B, H, N, d, block, _DT[q.dtype], _DT[odt], chunk, warm_chunk, _fwd_flags(exact, silu),
            _ptr(workspace), workspace.numel(), e0, e1, _stream(stream, dev),
        )
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_fwd_ex")
    return out


def fwd_fused(q, k, v, decay, gamma=None, gate=None, eps=1e-5, kv_in=None, kv_out=None, out=None,
              out_dtype=torch.bfloat16, chunk=0, warm_chunk=0, workspace=None, events=None, exact=False, silu=False,
              stream=None):
    """Prefill with the per-head RMSNorm (gamma fp32 [H, d]) and the sigmoid
    gate (gate bf16 [B, H, N, d]) applied in the kernels that write the output
    rows: out = o / sqrt(mean(o^2) + eps) * gamma[h] * sigmoid(gate).  q, k, v
    bf16 [B, H, N, d] (pre-activations with silu=True); block 64; the rest as
    fwd.  Returns out [B, H, N, d] in out_dtype."""
    lib = load()
    dev = _device_of("q", q)
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, torch.bfloat16, (B, H, N, d), device=dev)
    _check_dev("decay", decay, torch.float32, (H,), device=dev)
    if gamma is not None:
        _check_dev("gamma", gamma, torch.float32, (H, d), device=dev)
    if gate is not None:
        _check_dev("gate", gate, torch.bfloat16, (B, H, N, d), device=dev)
    for name, t in (("kv_in", kv_in), ("kv_out", kv_out)):
        if t is not None:
            _check_dev(name, t, torch.float32, (B, H, d, d), device=dev)
    if out is None:
        out = torch.empty((B, H, N, d), device=q.device, dtype=out_dtype)
    _check_dev("out", out, out_dtype, (B, H, N, d), device=dev)
    need = int(lib.lightning_attn_fwd_workspace_bytes_ex(B, H, N, d, 64, chunk))
    if need == 0:
        raise LightningAttnError(1, "lightning_attn_fwd_workspace_bytes_ex")
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    _check_dev("workspace", workspace, torch.uint8, device=dev)
    e0, e1 = (None, None) if events is None else (ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    with _current(dev):
        rc = lib.lightning_attn_fwd_fused(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(gamma), float(eps), _ptr(gate), _ptr(out), _ptr(kv_in),
            _ptr(kv_out), B, H, N, d, _DT[out_dtype], chunk, warm_chunk, _fwd_flags(exact, silu), _ptr(workspace),
            workspace.numel(), e0, e1, _stream(stream, dev),
        )
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_fwd_fused")
    return out


def fwd_noalloc(q, k, v, decay, out, kv_in=None, kv_out=None, chunk=0, warm_chunk=0, exact=False, silu=False,
                stream=None):
    """Prefill at block 64 that allocates nothing: the library keeps its
    workspace in a device array of NOALLOC_SCRATCH_BYTES per GPU (calls that
    overlap on one GPU race).  out is the caller's [B, H, N, d] tensor (bf16 or
    fp32); the rest as fwd.  chunk 0: the default chunk doubled until the chunk
    states fit the array.  Returns out."""
    lib = load()
    dev = _device_of("q", q)
    if q.dtype not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype, (B, H, N, d), device=dev)
    _check_dev("decay", decay, torch.float32, (H,), device=dev)
    for name, t in (("kv_in", kv_in), ("kv_out", kv_out)):
        if t is not None:
            _check_dev(name, t, torch.float32, (B, H, d, d), device=dev)
    if not isinstance(out, torch.Tensor) or out.dtype not in _DT:
        raise TypeError("out must be a bfloat16 or float32 tensor")
    _check_dev("out", out, out.dtype, (B, H, N, d), device=dev)
    with _current(dev):
        rc = lib.lightning_attn_fwd_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(out), _ptr(kv_in), _ptr(kv_out), B, H, N, d, _DT[q.dtype],
            _DT[out.dtype], chunk, warm_chunk, _fwd_flags(exact, silu), _stream(stream, dev),
        )
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_fwd_noalloc")
    return out


def decode_step(q, k, v, decay, kv_in=None, kv_out=None, out=None, stream=None):
    """One decode step.  q, k, v: [B, H, d] bf16; decay fp32 [H]; kv_in / kv_out:
    fp32 [B, H, d, d] (may be the same tensor).  Returns o [B, H, d] bf16."""
    lib = load()
    dev = _device_of("q", q)
    B, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, torch.bfloat16, (B, H, d), device=dev)
    _check_dev("decay", decay, torch.float32, (H,), device=dev)
    for name, t in (("kv_in", kv_in), ("kv_out", kv_out)):
        if t is not None:
            _check_dev(name, t, torch.float32, (B, H, d, d), device=dev)
    if out is None:
        out = torch.empty((B, H, d), device=q.device, dtype=torch.bfloat16)
    _check_dev("out", out, torch.bfloat16, (B, H, d), device=dev)
    with _current(dev):
        rc = lib.lightning_attn_decode_step(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(out), _ptr(kv_in), _ptr(kv_out), B, H, d, _stream(stream, dev)
        )
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_decode_step")
    return out


def fwd_slots(q, k, v, decay, states, slots, block=64, out=None, out_dtype=None, exact=False, silu=False,
              stream=None):
    """Prefill into a state pool.  q, k, v: [B, H, N, d]; states: fp32
    [num_slots, H, d, d], read and written in place for the rows' slots;
    slots: int32 [B] on the device (out of range: zero start, no write-back).
    Returns out [B, H, N, d] in out_dtype (default: the input dtype)."""
    lib = load()
    dev = _device_of("q", q)
    B, H, N, d = q.shape
    if q.dtype not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype, (B, H, N, d), device=dev)
    _check_dev("decay", decay, torch.float32, (H,), device=dev)
    if states.dim() != 4:
        raise ValueError("states must be [num_slots, H, d, d]")
    _check_dev("states", states, torch.float32, (states.shape[0], H, d, d), device=dev)
    _check_dev("slots", slots, torch.int32, (B,), device=dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H, N, d), device=q.device, dtype=out_dtype)
    _check_dev("out", out, out_dtype, (B, H, N, d), device=dev)
    with _current(dev):
        rc = lib.lightning_attn_fwd_slots(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(out), _ptr(states), _ptr(slots), B, H, N, d,
            states.shape[0], block, _DT[q.dtype], _DT[out_dtype], _fwd_flags(exact, silu), _stream(stream, dev)
        )
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_fwd_slots")
    return out


def bwd(q, k, v, decay, dout, kv_in=None, dkv_out=None, out_dtype=None, dkv_in=False, workspace=None,
        exact=False, stream=None):
    """Backward pass.  q, k, v, dout: [B, H, N, d] device tensors, all bf16 or all
    fp32; decay fp32 [H]; kv_in: the forward's initial state, dkv_out:
    dL/d(kv_out), fp32 [B, H, d, d] or None.  Returns (dq, dk, dv, dkv_in) with
    dq, dk, dv in out_dtype (default: the input dtype); dkv_in is an fp32
    tensor when asked for (True, or a tensor to write into), else None."""
    lib = load()
    dev = _device_of("q", q)
    B, H, N, d = q.shape
    if q.dtype not in _DT:
        raise TypeError("q must be bfloat16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_dev(name, t, q.dtype, (B, H, N, d), device=dev)
    _check_dev("decay", decay, torch.float32, (H,), device=dev)
    for name, t in (("kv_in", kv_in), ("dkv_out", dkv_out)):
        if t is not None:
            _check_dev(name, t, torch.float32, (B, H, d, d), device=dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    code = _DT[out_dtype]
    dq, dk, dv = (torch.empty((B, H, N, d), device=q.device, dtype=out_dtype) for _ in range(3))
    if dkv_in is True:
        dkv_in = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32)
    elif dkv_in is False:
        dkv_in = None
    if dkv_in is not None:
        _check_dev("dkv_in", dkv_in, torch.float32, (B, H, d, d), device=dev)
    need = lib_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    _check_dev("workspace", workspace, torch.uint8, device=dev)
    with _current(dev):
        rc = lib.lightning_attn_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(dout), _ptr(kv_in), _ptr(dkv_out), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(dkv_in), B, H, N, d, _DT[q.dtype], code, LA_FLAG_EXACT if exact else 0, _ptr(workspace),
            workspace.numel(), _stream(stream, dev)
        )
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_bwd")
    return dq, dk, dv, dkv_in


class _LightningAttnFunction(torch.autograd.Function):
    """fwd in the forward, bwd in the backward: the same library calls, with
    the tensors autograd hands over."""

    @staticmethod
    def forward(ctx, q, k, v, decay, kv_in, block):
        B, H, N, d = q.shape
        kv_out = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32)
        out = fwd(q, k, v, decay, kv_in=kv_in, kv_out=kv_out, block=block)
        ctx.save_for_backward(q, k, v, decay, kv_in)
        return out, kv_out

    @staticmethod
    def backward(ctx, dout, dkv_out):
        q, k, v, decay, kv_in = ctx.saved_tensors
        want_dkv_in = kv_in is not None and ctx.needs_input_grad[4]
        dq, dk, dv, dkv_in = bwd(q, k, v, decay, dout.contiguous(), kv_in=kv_in,
                                 dkv_out=None if dkv_out is None else dkv_out.contiguous(), dkv_in=want_dkv_in)
        return dq, dk, dv, None, dkv_in, None


def lightning_attn(q, k, v, decay, kv_in=None, block=64):
    """The prefill as a differentiable op: returns (out, kv_out) like fwd with
    kv_out given, and gradients for q, k, v and kv_in through bwd (out's and
    kv_out's gradients both enter).  decay gets no gradient.  q, k, v: bf16 or
    fp32 [B, H, N, d] on one device; kv_in fp32 [B, H, d, d] or None."""
    return _LightningAttnFunction.apply(q, k, v, decay, kv_in, block)


def decode_slots(q, k, v, decay, states, slots, out=None, stream=None):
    """Decode step over a state pool.  q, k, v: [B, H, d] bf16; decay fp32 [H];
    states: fp32 [num_slots, H, d, d], updated in place for the rows' slots;
    slots: int32 [B] on the device (out of range = idle row, zero output).
    Returns o [B, H, d] bf16."""
    lib = load()
    dev = _device_of("q", q)
    B, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, torch.bfloat16, (B, H, d), device=dev)
    _check_dev("decay", decay, torch.float32, (H,), device=dev)
    if states.dim() != 4:
        raise ValueError("states must be [num_slots, H, d, d]")
    _check_dev("states", states, torch.float32, (states.shape[0], H, d, d), device=dev)
    _check_dev("slots", slots, torch.int32, (B,), device=dev)
    if out is None:
        out = torch.empty((B, H, d), device=q.device, dtype=torch.bfloat16)
    _check_dev("out", out, torch.bfloat16, (B, H, d), device=dev)
    with _current(dev):
        rc = lib.lightning_attn_decode_slots(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(out), _ptr(states), _ptr(slots), B, H, d, states.shape[0],
            _stream(stream, dev)
        )
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_decode_slots")
    return out


def decode_fused(q, k, v, decay, states, slots=None, silu=True, gamma=None, gate=None, eps=1e-5, out=None,
                 stream=None):
    """Decode step with SiLU on q, k, v (silu=True), per-head RMSNorm of o
    (gamma fp32 [H, d]) and o * sigmoid(gate) (gate bf16 [B, H, d]) fused.
    states: fp32 [num_slots, H, d, d] in place; slots: int32 [B] or None
    (row b uses state row b).  Returns o [B, H, d] bf16."""
    lib = load()
    dev = _device_of("q", q)
    B, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, torch.bfloat16, (B, H, d), device=dev)
    _check_dev("decay", decay, torch.float32, (H,), device=dev)
    if states.dim() != 4:
        raise ValueError("states must be [num_slots, H, d, d]")
    _check_dev("states", states, torch.float32, (states.shape[0], H, d, d), device=dev)
    if slots is not None:
        _check_dev("slots", slots, torch.int32, (B,), device=dev)
    if gamma is not None:
        _check_dev("gamma", gamma, torch.float32, (H, d), device=dev)
    if gate is not None:
        _check_dev("gate", gate, torch.bfloat16, (B, H, d), device=dev)
    if out is None:
        out = torch.empty((B, H, d), device=q.device, dtype=torch.bfloat16)
    _check_dev("out", out, torch.bfloat16, (B, H, d), device=dev)
    with _current(dev):
        rc = lib.lightning_attn_decode_fused(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(out), _ptr(states), _ptr(slots), states.shape[0],
            1 if silu else 0, _ptr(gamma), float(eps), _ptr(gate), B, H, d, _stream(stream, dev)
        )
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_decode_fused")
    return out


def decode_layers(q, k, v, decay, states, slots=None, silu=False, gamma=None, gate=None, eps=1e-5, out=None,
                  stream=None):
    """One decode step of several layers in one launch.  q, k, v: bf16
    [L, B, H, d]; decay fp32 [L, H]; states fp32 [L, num_slots, H, d, d],
    updated in place; slots int32 [L, B] on the device (out of range = idle
    row) or None (row b uses slot b); silu / gamma fp32 [L, H, d] / gate bf16
    [L, B, H, d] as decode_fused.  Returns o [L, B, H, d] bf16."""
    lib = load()
    dev = _device_of("q", q)
    L, B, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, torch.bfloat16, (L, B, H, d), device=dev)
    _check_dev("decay", decay, torch.float32, (L, H), device=dev)
    if states.dim() != 5:
        raise ValueError("states must be [L, num_slots, H, d, d]")
    _check_dev("states", states, torch.float32, (L, states.shape[1], H, d, d), device=dev)
    if slots is not None:
        _check_dev("slots", slots, torch.int32, (L, B), device=dev)
    if gamma is not None:
        _check_dev("gamma", gamma, torch.float32, (L, H, d), device=dev)
    if gate is not None:
        _check_dev("gate", gate, torch.bfloat16, (L, B, H, d), device=dev)
    if out is None:
        out = torch.empty((L, B, H, d), device=q.device, dtype=torch.bfloat16)
    _check_dev("out", out, torch.bfloat16, (L, B, H, d), device=dev)
    with _current(dev):
        rc = lib.lightning_attn_decode_layers(
            _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(out), _ptr(states), _ptr(slots), L, B, H, d, states.shape[1],
            1 if silu else 0, _ptr(gamma), float(eps), _ptr(gate), _stream(stream, dev)
        )
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_decode_layers")
    return out


def norm_gate(o, gamma=None, gate=None, eps=1e-5, out=None, stream=None):
    """Per-head RMSNorm (gamma fp32 [H, d]) and sigmoid gate (gate bf16, o's
    shape) of a prefill output o [B, H, N, d] (bf16 or fp32), into bf16 out
    (o itself allowed when o is bf16)."""
    lib = load()
    dev = _device_of("o", o)
    if o.dtype not in _DT:
        raise TypeError("o must be bfloat16 or float32")
    B, H, N, d = o.shape
    _check_dev("o", o, None, (B, H, N, d), device=dev)
    if gamma is not None:
        _check_dev("gamma", gamma, torch.float32, (H, d), device=dev)
    if gate is not None:
        _check_dev("gate", gate, torch.bfloat16, (B, H, N, d), device=dev)
    if out is None:
        out = torch.empty((B, H, N, d), device=o.device, dtype=torch.bfloat16)
    _check_dev("out", out, torch.bfloat16, (B, H, N, d), device=dev)
    with _current(dev):
        rc = lib.lightning_attn_norm_gate(_ptr(o), _DT[o.dtype], _ptr(gate), _ptr(gamma), float(eps), _ptr(out),
                                          B, H, N, d, _stream(stream, dev))
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_norm_gate")
    return out


def silu_(x, stream=None):
    """x <- SiLU(x) in place (bf16 device tensor); returns x."""
    lib = load()
    dev = _device_of("x", x)
    _check_dev("x", x, torch.bfloat16, device=dev)
    with _current(dev):
        rc = lib.lightning_attn_silu(_ptr(x), x.numel(), _stream(stream, dev))
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_silu")
    return x


def runtime_version():
    v = ctypes.c_int(0)
    rc = load().lightning_attn_runtime_version(ctypes.byref(v))
    if rc != 0:
        raise LightningAttnError(rc, "lightning_attn_runtime_version")
    return v.value
