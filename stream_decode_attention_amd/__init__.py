"""Python binding of libdecattn (split-KV decode attention for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libdecattn.so, reached through its C ABI (include/decattn.h) with
ctypes. PyTorch supplies device memory and the current stream. If the library
has not been built, every call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "DecattnError", "load_library", "abi_version", "status_str", "default_chunk",
    "workspace_bytes", "decode_attn", "decode_attn_noalloc", "NOALLOC_SCRATCH_BYTES", "chunk_attn", "attn_partial", "attn_merge",
    "probe_read", "probe_copy", "rope_kv_write", "RopeParams", "prefill_attn",
    "gemv_bf16", "gemv_int8", "quantize_rows_int8", "spec_accept", "spec_accept_workspace_bytes",
    "OUT_BF16", "OUT_F32", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdecattn.so")
OUT_BF16, OUT_F32 = 0, 1
NOALLOC_SCRATCH_BYTES = 8 << 20     # DECATTN_NOALLOC_SCRATCH_BYTES of include/decattn.h
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}

_lib: Optional[ctypes.CDLL] = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class RopeParams(ctypes.Structure):
    """decattn_rope: the rotary frequencies of a model (include/decattn.h)."""
    _fields_ = [("theta", ctypes.c_double), ("pairing", ctypes.c_int), ("llama3_scaling", ctypes.c_int),
                ("factor", ctypes.c_double), ("low_freq_factor", ctypes.c_double),
                ("high_freq_factor", ctypes.c_double), ("original_max_position", ctypes.c_double)]


_SIGNATURES = {
    "decattn_abi_version": ([], _i),
    "decattn_status_str": ([_i], ctypes.c_char_p),
    "decattn_default_chunk": ([_i] * 6, _i),
    "decattn_workspace_bytes": ([_i] * 7, _sz),
    "decode_attn": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _i, _vp, _sz, _i, _vp], _i),
    "decode_attn_noalloc": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _i, _i, _vp], _i),
    "chunk_attn": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _i, _vp, _sz, _i, _vp], _i),
    "attn_partial": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _i, _vp], _i),
    "prefill_attn": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _i, _vp], _i),
    "gemv_bf16": ([_vp, _vp, _i, _i, _i, _vp, _i, _vp], _i),
    "gemv_int8": ([_vp, _vp, _vp, _i, _i, _i, _vp, _i, _vp], _i),
    "quantize_rows_int8": ([_vp, _i, _i, _vp, _vp, _vp], _i),
    "attn_merge": ([_vp, _i, _i, _i, _i, _i, _i, _i, _vp, _i, _vp, _sz, _i, _vp], _i),
    "rope_kv_write": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.POINTER(RopeParams), _vp, _vp, _vp,
                       _vp], _i),
    "spec_accept_workspace_bytes": ([_i, _i, _i], _sz),
    "spec_accept": ([_vp, _vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp], _i),
    "decattn_probe_read": ([_vp, _sz, _vp, _vp], _i),
    "decattn_probe_copy": ([_vp, _vp, _sz, _vp], _i),
}


class DecattnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_str(status)} (status {status})")
        self.status = status


def load_library() -> ctypes.CDLL:
    """The loaded libdecattn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m stream_decode_attention_amd.build` "
                "(or __graft_entry__.build()); there is no non-HIP fallback")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def abi_version() -> int:
    return load_library().decattn_abi_version()


def status_str(status: int) -> str:
    try:
        return load_library().decattn_status_str(status).decode()
    except Exception:
        return _STATUS.get(status, "unknown status")


def default_chunk(B: int, T: int, Hq: int, Hkv: int, D: int, S_max: int) -> int:
    return load_library().decattn_default_chunk(B, T, Hq, Hkv, D, S_max)


def workspace_bytes(B: int, T: int, Hq: int, Hkv: int, D: int, S_max: int, chunk: int = 0) -> int:
    return load_library().decattn_workspace_bytes(B, T, Hq, Hkv, D, S_max, chunk)


def _check(fn: str, status: int):
    if status != 0:
        raise DecattnError(fn, status)


def _ptr(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream, dev) -> int:
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, int):
        return stream
    if stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    return stream.cuda_stream


class _on_device:
    """Checks that every tensor argument sits on one device and makes that
    device the current one for the library call (the library launches on, and
    sizes its grids for, the current device)."""

    def __init__(self, *tensors):
        dev = None
        for t in tensors:
            if t is None:
                continue
            if not isinstance(t, torch.Tensor) or not t.is_cuda:
                raise ValueError("every tensor argument must be a device tensor")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"tensor arguments on {dev} and {t.device}: all must be on one device")
        self.index = dev.index if dev is not None and dev.index is not None else None
        self.prev = None

    def __enter__(self):
        if self.index is not None:
            cur = torch.cuda.current_device()
            if cur != self.index:
                self.prev = cur
                torch.cuda.set_device(self.index)
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)
        return False


def _out_dtype(out: torch.Tensor) -> int:
    if out.dtype == torch.float32:
        return OUT_F32
    if out.dtype in _BF16:
        return OUT_BF16
    raise TypeError(f"out has dtype {out.dtype}; expected float32 or bfloat16")


def decode_attn(q, k_cache, v_cache, seq_lens, scale: float, out, workspace, chunk: int = 0,
                stream=None):
    """out[b,h] = softmax(scale q[b,h].K[b,h//G,:n_b]^T) V[b,h//G,:n_b]; see include/decattn.h.

    q bf16 [B,Hq,D]; caches bf16 [B,Hkv,S_max,D]; seq_lens int32 [B] (device);
    out fp32 or bf16 [B,Hq,D]; workspace uint8 device tensor of at least
    workspace_bytes(B, 1, Hq, Hkv, D, S_max, chunk) bytes.
    """
    B, Hq, D = q.shape
    _, Hkv, S_max, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != (B, Hq, D) \
            or k_cache.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("shape mismatch between q, caches, seq_lens and out")
    with _on_device(q, k_cache, v_cache, seq_lens, out, workspace):
        st = load_library().decode_attn(
            _ptr(q, "q", _BF16), _ptr(k_cache, "k_cache", _BF16), _ptr(v_cache, "v_cache", _BF16),
            _ptr(seq_lens, "seq_lens", (torch.int32,)), B, Hq, Hkv, D, S_max, float(scale),
            _ptr(out, "out", (torch.float32,) + _BF16), _out_dtype(out),
            _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), int(chunk),
            _stream(stream, q.device))
    _check("decode_attn", st)
    return out


def decode_attn_noalloc(q, k_cache, v_cache, seq_lens, scale: float, out, chunk: int = 0, stream=None):
    """decode_attn without a workspace argument: the library keeps the partial
    state in its own static device array (NOALLOC_SCRATCH_BYTES per GPU) and
    allocates nothing. Calls that may overlap on one GPU race; see
    include/decattn.h."""
    B, Hq, D = q.shape
    _, Hkv, S_max, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != (B, Hq, D) \
            or k_cache.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("shape mismatch between q, caches, seq_lens and out")
    with _on_device(q, k_cache, v_cache, seq_lens, out):
        st = load_library().decode_attn_noalloc(
            _ptr(q, "q", _BF16), _ptr(k_cache, "k_cache", _BF16), _ptr(v_cache, "v_cache", _BF16),
            _ptr(seq_lens, "seq_lens", (torch.int32,)), B, Hq, Hkv, D, S_max, float(scale),
            _ptr(out, "out", (torch.float32,) + _BF16), _out_dtype(out), int(chunk),
            _stream(stream, q.device))
    _check("decode_attn_noalloc", st)
    return out


def chunk_attn(q, k_cache, v_cache, ctx_lens, scale: float, out, workspace, chunk: int = 0,
               stream=None):
    """Causal verify attention: q bf16 [B,T,Hq,D]; token i attends keys j < ctx_lens[b]+i+1."""
    B, T, Hq, D = q.shape
    _, Hkv, S_max, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != (B, T, Hq, D) \
            or k_cache.shape[0] != B or tuple(ctx_lens.shape) != (B,):
        raise ValueError("shape mismatch between q, caches, ctx_lens and out")
    with _on_device(q, k_cache, v_cache, ctx_lens, out, workspace):
        st = load_library().chunk_attn(
            _ptr(q, "q", _BF16), _ptr(k_cache, "k_cache", _BF16), _ptr(v_cache, "v_cache", _BF16),
            _ptr(ctx_lens, "ctx_lens", (torch.int32,)), B, T, Hq, Hkv, D, S_max, float(scale),
            _ptr(out, "out", (torch.float32,) + _BF16), _out_dtype(out),
            _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), int(chunk),
            _stream(stream, q.device))
    _check("chunk_attn", st)
    return out


def prefill_attn(q, k_cache, v_cache, ctx_lens, scale: float, out, stream=None):
    """Causal attention of T query tokens on the matrix cores (any T): token i
    attends keys j < ctx_lens[b]+i+1. q bf16 [B,T,Hq,D]; out fp32 or bf16
    [B,T,Hq,D]; no workspace. See include/decattn.h."""
    B, T, Hq, D = q.shape
    _, Hkv, S_max, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != (B, T, Hq, D) \
            or k_cache.shape[0] != B or tuple(ctx_lens.shape) != (B,):
        raise ValueError("shape mismatch between q, caches, ctx_lens and out")
    with _on_device(q, k_cache, v_cache, ctx_lens, out):
        st = load_library().prefill_attn(
            _ptr(q, "q", _BF16), _ptr(k_cache, "k_cache", _BF16), _ptr(v_cache, "v_cache", _BF16),
            _ptr(ctx_lens, "ctx_lens", (torch.int32,)), B, T, Hq, Hkv, D, S_max, float(scale),
            _ptr(out, "out", (torch.float32,) + _BF16), _out_dtype(out), _stream(stream, q.device))
    _check("prefill_attn", st)
    return out


def gemv_bf16(W, x, y, stream=None):
    """y[b, n] = sum_k W[n, k] x[b, k]: W bf16 [N, K], x bf16 [B, K] (B <= 8),
    y fp32 or bf16 [B, N]. See include/decattn.h."""
    N, K = W.shape
    B = x.shape[0]
    if tuple(x.shape) != (B, K) or tuple(y.shape) != (B, N):
        raise ValueError("shape mismatch between W, x and y")
    with _on_device(W, x, y):
        st = load_library().gemv_bf16(_ptr(W, "W", _BF16), _ptr(x, "x", _BF16), B, N, K,
                                      _ptr(y, "y", (torch.float32,) + _BF16), _out_dtype(y), _stream(stream, W.device))
    _check("gemv_bf16", st)
    return y


def gemv_int8(Wq, scale, x, y, stream=None):
    """y[b, n] = scale[n] * sum_k Wq[n, k] x[b, k]: Wq int8 [N, K], scale fp32 [N]."""
    N, K = Wq.shape
    B = x.shape[0]
    if tuple(x.shape) != (B, K) or tuple(y.shape) != (B, N) or tuple(scale.shape) != (N,):
        raise ValueError("shape mismatch between Wq, scale, x and y")
    with _on_device(Wq, scale, x, y):
        st = load_library().gemv_int8(_ptr(Wq, "Wq", (torch.int8,)), _ptr(scale, "scale", (torch.float32,)),
                                      _ptr(x, "x", _BF16), B, N, K, _ptr(y, "y", (torch.float32,) + _BF16),
                                      _out_dtype(y), _stream(stream, Wq.device))
    _check("gemv_int8", st)
    return y


def quantize_rows_int8(W, Wq, scale, stream=None):
    """Per-row symmetric INT8 codes and fp32 scales of bf16 W [N, K]."""
    N, K = W.shape
    if tuple(Wq.shape) != (N, K) or tuple(scale.shape) != (N,):
        raise ValueError("shape mismatch between W, Wq and scale")
    with _on_device(W, Wq, scale):
        st = load_library().quantize_rows_int8(_ptr(W, "W", _BF16), N, K, _ptr(Wq, "Wq", (torch.int8,)),
                                               _ptr(scale, "scale", (torch.float32,)), _stream(stream, W.device))
    _check("quantize_rows_int8", st)


def spec_accept_workspace_bytes(B: int, T: int, V: int) -> int:
    return load_library().spec_accept_workspace_bytes(B, T, V)


def _opt_ptr(t, name, dtypes) -> Optional[int]:
    return None if t is None else _ptr(t, name, dtypes)


def spec_accept(logits, q, drafts, u, r, tau: float, lens, result, workspace, S_max: int, stream=None):
    """Accept/reject of speculative drafts and rollback of ``lens``, on the device.

    logits fp32 [B,T,V]; q fp32 [B,T-1,V] (None when tau == 0); drafts int32
    [B,T-1]; u fp32 [B,T-1] and r fp32 [B] (None when tau == 0); lens int32 [B]
    (read and written); result int32 [B,2] receives (accepted drafts, next
    token); workspace uint8 of at least spec_accept_workspace_bytes(B, T, V).
    See include/decattn.h.
    """
    B, T, V = logits.shape
    G = T - 1
    if tuple(lens.shape) != (B,) or tuple(result.shape) != (B, 2):
        raise ValueError("lens must be [B] and result [B, 2]")
    for name, t, shape in (("q", q, (B, G, V)), ("drafts", drafts, (B, G)), ("u", u, (B, G)), ("r", r, (B,))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    with _on_device(logits, q, drafts, u, r, lens, result, workspace):
        st = load_library().spec_accept(
            _ptr(logits, "logits", (torch.float32,)), _opt_ptr(q, "q", (torch.float32,)),
            _opt_ptr(drafts, "drafts", (torch.int32,)), _opt_ptr(u, "u", (torch.float32,)),
            _opt_ptr(r, "r", (torch.float32,)), float(tau), B, T, V, int(S_max),
            _ptr(lens, "lens", (torch.int32,)), _ptr(result, "result", (torch.int32,)),
            _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream, logits.device))
    _check("spec_accept", st)
    return result


def attn_partial(q, k_cache, v_cache, lens, scale: float, workspace, causal: bool = False,
                 chunk: int = 0, stream=None):
    """First phase only: per-tile partial softmax state into ``workspace``."""
    if q.dim() == 3:
        B, Hq, D = q.shape
        T = 1
    else:
        B, T, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    with _on_device(q, k_cache, v_cache, lens, workspace):
        st = load_library().attn_partial(
            _ptr(q, "q", _BF16), _ptr(k_cache, "k_cache", _BF16), _ptr(v_cache, "v_cache", _BF16),
            _ptr(lens, "lens", (torch.int32,)), B, T, Hq, Hkv, D, S_max, float(scale), int(bool(causal)),
            _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), int(chunk),
            _stream(stream, q.device))
    _check("attn_partial", st)


def attn_merge(lens, out, workspace, *, T: int, Hq: int, Hkv: int, S_max: int, causal: bool = False,
               chunk: int = 0, stream=None):
    """Second phase only: log-sum-exp merge of ``workspace`` into ``out``."""
    B = lens.shape[0]
    D = out.shape[-1]
    with _on_device(lens, out, workspace):
        st = load_library().attn_merge(
            _ptr(lens, "lens", (torch.int32,)), B, T, Hq, Hkv, D, S_max, int(bool(causal)),
            _ptr(out, "out", (torch.float32,) + _BF16), _out_dtype(out),
            _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), int(chunk),
            _stream(stream, out.device))
    _check("attn_merge", st)


_PAIRING = {"half": 0, "adjacent": 1}


def rope_params(theta: float, pairing: str = "half", llama3: Optional[dict] = None) -> RopeParams:
    """Pack the frequency description; ``llama3`` holds factor, low_freq_factor,
    high_freq_factor and original_max_position when that scaling applies."""
    if pairing not in _PAIRING:
        raise ValueError(f"pairing must be one of {sorted(_PAIRING)}")
    r = RopeParams(float(theta), _PAIRING[pairing], 0, 0.0, 0.0, 0.0, 0.0)
    if llama3:
        r.llama3_scaling = 1
        r.factor = float(llama3["factor"])
        r.low_freq_factor = float(llama3["low_freq_factor"])
        r.high_freq_factor = float(llama3["high_freq_factor"])
        r.original_max_position = float(llama3["original_max_position"])
    return r


def rope_kv_write(q_in, k_in, v_in, pos0, q_out, k_cache, v_cache, theta: float, pairing: str = "half",
                  llama3: Optional[dict] = None, stream=None):
    """Rotate the step's new q (into ``q_out``, which may be ``q_in``) and k by
    their positions pos0[b] + i and store k, v into the caches there.

    q_in / q_out bf16 [B,T,Hq,D]; k_in / v_in bf16 [B,T,Hkv,D]; pos0 int32 [B]
    (device); caches bf16 [B,Hkv,S_max,D]. See include/decattn.h.
    """
    B, T, Hq, D = q_in.shape
    _, Hkv, S_max, Dk = k_cache.shape
    if tuple(q_out.shape) != (B, T, Hq, D) or tuple(k_in.shape) != (B, T, Hkv, D) \
            or tuple(v_in.shape) != (B, T, Hkv, D) or Dk != D or k_cache.shape[0] != B \
            or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(pos0.shape) != (B,):
        raise ValueError("shape mismatch between q, k, v, pos0 and the caches")
    params = rope_params(theta, pairing, llama3)
    with _on_device(q_in, k_in, v_in, pos0, q_out, k_cache, v_cache):
        st = load_library().rope_kv_write(
            _ptr(q_in, "q_in", _BF16), _ptr(k_in, "k_in", _BF16), _ptr(v_in, "v_in", _BF16),
            _ptr(pos0, "pos0", (torch.int32,)), B, T, Hq, Hkv, D, S_max, ctypes.byref(params),
            _ptr(q_out, "q_out", _BF16), _ptr(k_cache, "k_cache", _BF16), _ptr(v_cache, "v_cache", _BF16),
            _stream(stream, q_in.device))
    _check("rope_kv_write", st)
    return q_out


def probe_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Stream-read every byte of ``buf`` (16-byte loads); writes at most 4 bytes of ``sink``."""
    with _on_device(buf, sink):
        st = load_library().decattn_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                               sink.data_ptr(), _stream(stream, buf.device))
    _check("decattn_probe_read", st)


def probe_copy(dst: torch.Tensor, src: torch.Tensor, stream=None):
    with _on_device(dst, src):
        st = load_library().decattn_probe_copy(dst.data_ptr(), src.data_ptr(),
                                               src.numel() * src.element_size(), _stream(stream, src.device))
    _check("decattn_probe_copy", st)
