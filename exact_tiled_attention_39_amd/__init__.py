"""Python binding of libfa (exact tiled attention forward for gfx950): argument marshalling only.

Every step of the computation runs in the HIP kernels of ``libfa.so``; this module converts
torch tensors to the C-ABI's pointers, sizes and strides, allocates outputs on request, and
raises ``FaError`` on any non-OK status. There is no fallback: if the library is not built the
import of the binding functions raises.

The C entry points (include/fa.h) are mirrored with the same names:
``fa_fwd``, ``fa_check_args``, ``fa_splitkv_plan``, ``fa_fwd_splitkv``,
``fa_fwd_splitkv_noalloc``, ``fa_bwd``,
``fa_bwd_check_args``, ``fa_status_string``, ``fa_abi_version``, ``fa_params_size``,
``fa_bwd_params_size``. ``attention`` allocates O and LSE and calls ``fa_fwd``;
``attention_splitkv`` allocates O, LSE and the split workspace and calls ``fa_fwd_splitkv``;
``attention_fp8`` runs ``fa_fwd`` on E4M3 inputs with their descales;
``attention_backward`` allocates dQ, dK, dV and the delta workspace and calls ``fa_bwd``.
"""
from __future__ import annotations

import ctypes
import math
import pathlib
from typing import Optional, Tuple

import torch  # loaded first: libfa then binds to the HIP runtime torch already loaded

LIB_PATH = pathlib.Path(__file__).resolve().with_name("libfa.so")

FA_F16, FA_BF16, FA_E4M3 = 0, 1, 2
(FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_GQA,
 FA_ERR_VARLEN, FA_ERR_ABI, FA_ERR_LAUNCH, FA_ERR_SCRATCH) = range(10)
FA_ABI_VERSION = 8
FA_MAX_SPLITS = 256
FA_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024

_I64x3 = ctypes.c_int64 * 3


class FaFwdParams(ctypes.Structure):
    """Mirror of ``fa_fwd_params`` in include/fa.h (same field order and types)."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("num_seqs", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("q_stride", _I64x3),
        ("k_stride", _I64x3),
        ("v_stride", _I64x3),
        ("o_stride", _I64x3),
        ("seqlen_k", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("rope_cos", ctypes.c_void_p),
        ("rope_sin", ctypes.c_void_p),
        ("rope_rows", ctypes.c_int32),
        ("rope_interleaved", ctypes.c_int32),
        ("k_rot", ctypes.c_void_p),
        ("k_rot_stride", _I64x3),
        ("q_descale", ctypes.c_void_p),
        ("k_descale", ctypes.c_void_p),
        ("v_descale", ctypes.c_void_p),
    ]

    def __init__(self, **kw):
        super().__init__(struct_size=ctypes.sizeof(FaFwdParams), **kw)


class FaBwdParams(ctypes.Structure):
    """Mirror of ``fa_bwd_params`` in include/fa.h (same field order and types)."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("dout", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("delta", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("num_seqs", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("q_stride", _I64x3),
        ("k_stride", _I64x3),
        ("v_stride", _I64x3),
        ("o_stride", _I64x3),
        ("do_stride", _I64x3),
        ("dq_stride", _I64x3),
        ("dk_stride", _I64x3),
        ("dv_stride", _I64x3),
    ]

    def __init__(self, **kw):
        super().__init__(struct_size=ctypes.sizeof(FaBwdParams), **kw)


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libfa status {status}: {message}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads libfa.so once and checks that its ABI matches this binding."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = pathlib.Path(path) if path else LIB_PATH
    if not p.exists():
        raise ImportError(f"{p} is not built; run `python -m exact_tiled_attention_39_amd.build` "
                          "(libfa has no fallback path)")
    lib = ctypes.CDLL(str(p))
    lib.fa_abi_version.restype = ctypes.c_int32
    lib.fa_abi_version.argtypes = []
    lib.fa_params_size.restype = ctypes.c_uint32
    lib.fa_params_size.argtypes = []
    lib.fa_check_args.restype = ctypes.c_int32
    lib.fa_check_args.argtypes = [ctypes.POINTER(FaFwdParams)]
    lib.fa_fwd.restype = ctypes.c_int32
    lib.fa_fwd.argtypes = [ctypes.POINTER(FaFwdParams), ctypes.c_void_p]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [ctypes.c_int32]
    lib.fa_splitkv_plan.restype = ctypes.c_int32
    lib.fa_splitkv_plan.argtypes = [ctypes.POINTER(FaFwdParams), ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_uint64)]
    lib.fa_fwd_splitkv.restype = ctypes.c_int32
    lib.fa_fwd_splitkv.argtypes = [ctypes.POINTER(FaFwdParams), ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_uint64, ctypes.c_void_p]
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int32
    lib.fa_fwd_splitkv_noalloc.argtypes = [ctypes.POINTER(FaFwdParams), ctypes.c_int32,
                                           ctypes.c_void_p]
    lib.fa_bwd_params_size.restype = ctypes.c_uint32
    lib.fa_bwd_params_size.argtypes = []
    lib.fa_bwd_check_args.restype = ctypes.c_int32
    lib.fa_bwd_check_args.argtypes = [ctypes.POINTER(FaBwdParams)]
    lib.fa_bwd.restype = ctypes.c_int32
    lib.fa_bwd.argtypes = [ctypes.POINTER(FaBwdParams), ctypes.c_void_p]
    if lib.fa_abi_version() != FA_ABI_VERSION:
        raise ImportError(f"libfa ABI {lib.fa_abi_version()} != binding ABI {FA_ABI_VERSION}")
    if lib.fa_params_size() != ctypes.sizeof(FaFwdParams):
        raise ImportError("fa_fwd_params layout differs between libfa and the binding")
    if lib.fa_bwd_params_size() != ctypes.sizeof(FaBwdParams):
        raise ImportError("fa_bwd_params layout differs between libfa and the binding")
    if path is None:
        _lib = lib
    return lib


def fa_abi_version() -> int:
    return int(load_library().fa_abi_version())


def fa_params_size() -> int:
    return int(load_library().fa_params_size())


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_check_args(params: FaFwdParams) -> int:
    """Host-only validation of a filled FaFwdParams; returns the fa_status code."""
    return int(load_library().fa_check_args(ctypes.byref(params)))


def fa_bwd_params_size() -> int:
    return int(load_library().fa_bwd_params_size())


def fa_bwd_check_args(params: FaBwdParams) -> int:
    """Host-only validation of a filled FaBwdParams; returns the fa_status code."""
    return int(load_library().fa_bwd_check_args(ctypes.byref(params)))


_DTYPES = {torch.float16: FA_F16, torch.bfloat16: FA_BF16}
_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _strides(t: torch.Tensor):
    if t.numel() == 0:  # no element is addressed: report the contiguous layout
        return _I64x3(t.shape[1] * t.shape[2] * t.shape[3], t.shape[2] * t.shape[3], t.shape[3])
    s = t.stride()
    return _I64x3(s[0], s[1], s[2])


def make_params(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                lse: torch.Tensor, scale: float, causal: bool,
                cu_seqlens: Optional[torch.Tensor], max_seqlen: Optional[int],
                cu_seqlens_k: Optional[torch.Tensor] = None,
                rope_cos: Optional[torch.Tensor] = None, rope_sin: Optional[torch.Tensor] = None,
                rope_interleaved: bool = False,
                k_rot: Optional[torch.Tensor] = None) -> FaFwdParams:
    """Fills FaFwdParams from [B, H, N, d] tensors (strides in elements); K and V may have
    their own token count. RoPE: contiguous fp32 tables [positions, d/2], and k_rot (shaped
    like k) to receive the rotated keys, or None when k already holds rotated keys."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or o.dim() != 4:
        raise ValueError("q, k, v and o must be 4-D [batch, heads, tokens, head_dim]")
    fp8 = q.dtype in _FP8_DTYPES
    if fp8:
        if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != torch.bfloat16:
            raise ValueError("FP8 attention takes E4M3 q, k, v (uint8 codes or "
                             "torch.float8_e4m3fn) and a bfloat16 o")
    elif q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise ValueError("q, k, v and o must share one dtype: float16 or bfloat16")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [batch, heads_q, tokens]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.stride(3) != 1 and t.shape[3] > 1 and t.numel() > 0:
            raise ValueError(f"{name}: the head_dim dimension must be contiguous")
    b, hq, n, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (b, hkv, nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [batch, heads_kv, key tokens, head_dim] matching q")
    if tuple(o.shape) != tuple(q.shape) or tuple(lse.shape) != (b, hq, n):
        raise ValueError("o must match q and lse must be [batch, heads_q, tokens]")
    p = FaFwdParams(
        dtype=FA_E4M3 if fp8 else _DTYPES[q.dtype], q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(),
        o=o.data_ptr(), lse=lse.data_ptr(), batch=b, heads_q=hq, heads_kv=hkv, seqlen=n,
        seqlen_k=nk, head_dim=d, causal=int(bool(causal)), scale=float(scale),
        q_stride=_strides(q), k_stride=_strides(k), v_stride=_strides(v), o_stride=_strides(o))
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor")
        if cu_seqlens.device != q.device:
            raise ValueError("cu_seqlens must live on the same device as q")
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens")
        p.cu_seqlens = cu_seqlens.data_ptr()
        p.num_seqs = cu_seqlens.numel() - 1
        p.max_seqlen = int(max_seqlen)
    if cu_seqlens_k is not None:
        if cu_seqlens is None:
            raise ValueError("cu_seqlens_k needs cu_seqlens")
        if (cu_seqlens_k.dtype != torch.int32 or cu_seqlens_k.dim() != 1
                or cu_seqlens_k.numel() != cu_seqlens.numel()):
            raise ValueError("cu_seqlens_k must be a 1-D int32 tensor shaped like cu_seqlens")
        if cu_seqlens_k.device != q.device:
            raise ValueError("cu_seqlens_k must live on the same device as q")
        p.cu_seqlens_k = cu_seqlens_k.data_ptr()
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("rope_cos and rope_sin go together")
    if rope_cos is not None:
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            if (t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != d // 2
                    or not t.is_contiguous() or t.device != q.device):
                raise ValueError(f"{name} must be a contiguous float32 [positions, head_dim/2] "
                                 "tensor on the device of q")
        if rope_sin.shape != rope_cos.shape:
            raise ValueError("rope_cos and rope_sin must have one shape")
        p.rope_cos, p.rope_sin = rope_cos.data_ptr(), rope_sin.data_ptr()
        p.rope_rows = rope_cos.shape[0]
        p.rope_interleaved = int(bool(rope_interleaved))
        if k_rot is not None:
            if (k_rot.shape != k.shape or k_rot.dtype != k.dtype or k_rot.device != q.device
                    or (k_rot.stride(3) != 1 and k_rot.numel() > 0)):
                raise ValueError("k_rot must be shaped like k, on its device, with head_dim "
                                 "contiguous")
            p.k_rot = k_rot.data_ptr()
            p.k_rot_stride = _strides(k_rot)
    elif k_rot is not None:
        raise ValueError("k_rot needs the RoPE tables")
    return p


def set_descales(p: FaFwdParams, q: torch.Tensor, k: torch.Tensor,
                 q_descale: Optional[torch.Tensor], k_descale: Optional[torch.Tensor],
                 v_descale: Optional[torch.Tensor]) -> None:
    """FP8 descales: contiguous float32 [batch, heads_q] for q, [batch, heads_kv] for k and v."""
    for name, t, heads in (("q_descale", q_descale, q.shape[1]), ("k_descale", k_descale, k.shape[1]),
                           ("v_descale", v_descale, k.shape[1])):
        if t is None:
            continue
        if (t.dtype != torch.float32 or tuple(t.shape) != (q.shape[0], heads)
                or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous float32 [batch, heads] tensor on the "
                             "device of q")
        setattr(p, name, t.data_ptr())


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
           lse: torch.Tensor, *, scale: float, causal: bool = False,
           cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
           stream: Optional[torch.cuda.Stream] = None,
           cu_seqlens_k: Optional[torch.Tensor] = None,
           rope_cos: Optional[torch.Tensor] = None, rope_sin: Optional[torch.Tensor] = None,
           rope_interleaved: bool = False, k_rot: Optional[torch.Tensor] = None,
           q_descale: Optional[torch.Tensor] = None, k_descale: Optional[torch.Tensor] = None,
           v_descale: Optional[torch.Tensor] = None) -> None:
    """Enqueues the forward pass writing o and lse, on `stream` (default: torch's current);
    with RoPE tables also the rotated keys into k_rot (None: k is already rotated). E4M3 q, k,
    v (FP8) take per-(batch, head) descales and write a bfloat16 o."""
    lib = load_library()
    for t in (q, k, v, o, lse):
        if not t.is_cuda:
            raise ValueError("libfa runs on the GPU: all tensors must be on a HIP device")
    p = make_params(q, k, v, o, lse, scale, causal, cu_seqlens, max_seqlen, cu_seqlens_k,
                    rope_cos, rope_sin, rope_interleaved, k_rot)
    set_descales(p, q, k, q_descale, k_descale, v_descale)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = int(lib.fa_fwd(ctypes.byref(p), ctypes.c_void_p(s.cuda_stream)))
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))


def _rope_keys_out(k: torch.Tensor, rope_cos, keys_rotated: bool):
    """The buffer the rotated keys go to: None without RoPE or when k is already rotated."""
    if rope_cos is None or keys_rotated:
        return None
    return torch.empty(k.shape, dtype=k.dtype, device=k.device)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
              scale: Optional[float] = None, causal: bool = False,
              cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
              cu_seqlens_k: Optional[torch.Tensor] = None,
              rope_cos: Optional[torch.Tensor] = None, rope_sin: Optional[torch.Tensor] = None,
              rope_interleaved: bool = False, keys_rotated: bool = False,
              return_k_rot: bool = False):
    """softmax(scale * Q K^T) V and its per-row log-sum-exp, for [B, H, N, d] tensors.

    scale defaults to 1/sqrt(d). K and V may hold more (or fewer) tokens than Q: the queries
    are then the last positions of the keys, which is what causal masking measures from. With
    cu_seqlens (int32 prefix sums, batch 1) sequences are packed along the token axis and
    attend only within themselves (keys per cu_seqlens_k when packed differently); max_seqlen,
    if omitted, is read from cu_seqlens with a device-to-host copy. With RoPE tables (fp32
    [positions, d/2] cos and sin) Q and K are rotated by their positions first; keys_rotated
    says K already holds rotated keys, and return_k_rot also returns the rotated keys.
    """
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if cu_seqlens is not None and max_seqlen is None:
        lens = (cu_seqlens[1:] - cu_seqlens[:-1]).cpu()
        max_seqlen = int(lens.max()) if lens.numel() else 0
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    k_rot = _rope_keys_out(k, rope_cos, keys_rotated)
    fa_fwd(q, k, v, o, lse, scale=scale, causal=causal, cu_seqlens=cu_seqlens,
           max_seqlen=max_seqlen, cu_seqlens_k=cu_seqlens_k, rope_cos=rope_cos,
           rope_sin=rope_sin, rope_interleaved=rope_interleaved, k_rot=k_rot)
    return (o, lse, k_rot) if return_k_rot else (o, lse)


def fa_splitkv_plan(params: FaFwdParams, num_splits: int = 0) -> Tuple[int, int]:
    """Host-only: (resolved split count, workspace bytes) for fa_fwd_splitkv; raises FaError."""
    splits = ctypes.c_int32(0)
    nbytes = ctypes.c_uint64(0)
    st = int(load_library().fa_splitkv_plan(ctypes.byref(params), int(num_splits),
                                            ctypes.byref(splits), ctypes.byref(nbytes)))
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))
    return int(splits.value), int(nbytes.value)


def fa_fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                   lse: torch.Tensor, workspace: Optional[torch.Tensor], *, scale: float,
                   causal: bool = False, num_splits: int = 0,
                   cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                   stream: Optional[torch.cuda.Stream] = None,
                   cu_seqlens_k: Optional[torch.Tensor] = None,
                   rope_cos: Optional[torch.Tensor] = None,
                   rope_sin: Optional[torch.Tensor] = None, rope_interleaved: bool = False,
                   k_rot: Optional[torch.Tensor] = None) -> None:
    """Enqueues the split-KV forward writing o and lse; `workspace` is a device tensor of at
    least fa_splitkv_plan's byte count (None when that is 0)."""
    lib = load_library()
    for t in (q, k, v, o, lse) + ((workspace,) if workspace is not None else ()):
        if not t.is_cuda:
            raise ValueError("libfa runs on the GPU: all tensors must be on a HIP device")
    p = make_params(q, k, v, o, lse, scale, causal, cu_seqlens, max_seqlen, cu_seqlens_k,
                    rope_cos, rope_sin, rope_interleaved, k_rot)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = int(lib.fa_fwd_splitkv(ctypes.byref(p), int(num_splits), ctypes.c_void_p(ws_ptr),
                                    ctypes.c_uint64(ws_bytes), ctypes.c_void_p(s.cuda_stream)))
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))


def fa_fwd_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                           lse: torch.Tensor, *, scale: float, causal: bool = False,
                           num_splits: int = 0, cu_seqlens: Optional[torch.Tensor] = None,
                           max_seqlen: Optional[int] = None,
                           stream: Optional[torch.cuda.Stream] = None,
                           cu_seqlens_k: Optional[torch.Tensor] = None,
                           rope_cos: Optional[torch.Tensor] = None,
                           rope_sin: Optional[torch.Tensor] = None,
                           rope_interleaved: bool = False,
                           k_rot: Optional[torch.Tensor] = None) -> None:
    """Enqueues the split-KV forward writing o and lse, with the split partials in the
    library's static per-GPU scratch instead of a workspace (nothing is allocated)."""
    lib = load_library()
    for t in (q, k, v, o, lse):
        if not t.is_cuda:
            raise ValueError("libfa runs on the GPU: all tensors must be on a HIP device")
    p = make_params(q, k, v, o, lse, scale, causal, cu_seqlens, max_seqlen, cu_seqlens_k,
                    rope_cos, rope_sin, rope_interleaved, k_rot)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = int(lib.fa_fwd_splitkv_noalloc(ctypes.byref(p), int(num_splits),
                                            ctypes.c_void_p(s.cuda_stream)))
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))


def attention_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                      scale: Optional[float] = None, causal: bool = False, num_splits: int = 0,
                      cu_seqlens: Optional[torch.Tensor] = None,
                      max_seqlen: Optional[int] = None,
                      cu_seqlens_k: Optional[torch.Tensor] = None,
                      rope_cos: Optional[torch.Tensor] = None,
                      rope_sin: Optional[torch.Tensor] = None, rope_interleaved: bool = False,
                      keys_rotated: bool = False, return_k_rot: bool = False):
    """``attention`` computed by the split-KV kernels (meant for a few queries per sequence
    against many keys); allocates O, LSE and the workspace."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if cu_seqlens is not None and max_seqlen is None:
        lens = (cu_seqlens[1:] - cu_seqlens[:-1]).cpu()
        max_seqlen = int(lens.max()) if lens.numel() else 0
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    k_rot = _rope_keys_out(k, rope_cos, keys_rotated)
    p = make_params(q, k, v, o, lse, scale, causal, cu_seqlens, max_seqlen, cu_seqlens_k,
                    rope_cos, rope_sin, rope_interleaved, k_rot)
    _, nbytes = fa_splitkv_plan(p, num_splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    fa_fwd_splitkv(q, k, v, o, lse, ws, scale=scale, causal=causal, num_splits=num_splits,
                   cu_seqlens=cu_seqlens, max_seqlen=max_seqlen, cu_seqlens_k=cu_seqlens_k,
                   rope_cos=rope_cos, rope_sin=rope_sin, rope_interleaved=rope_interleaved,
                   k_rot=k_rot)
    return (o, lse, k_rot) if return_k_rot else (o, lse)


def attention_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  q_descale: Optional[torch.Tensor] = None,
                  k_descale: Optional[torch.Tensor] = None,
                  v_descale: Optional[torch.Tensor] = None, *, scale: Optional[float] = None,
                  causal: bool = False, cu_seqlens: Optional[torch.Tensor] = None,
                  max_seqlen: Optional[int] = None,
                  cu_seqlens_k: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention on E4M3 q, k, v ([B, H, N, d] codes, uint8 or float8_e4m3fn) standing for
    codes times their per-(batch, head) descales; returns bfloat16 O and fp32 LSE."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if cu_seqlens is not None and max_seqlen is None:
        lens = (cu_seqlens[1:] - cu_seqlens[:-1]).cpu()
        max_seqlen = int(lens.max()) if lens.numel() else 0
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale=scale, causal=causal, cu_seqlens=cu_seqlens,
           max_seqlen=max_seqlen, cu_seqlens_k=cu_seqlens_k, q_descale=q_descale,
           k_descale=k_descale, v_descale=v_descale)
    return o, lse


def make_bwd_params(q, k, v, o, dout, lse, dq, dk, dv, delta, scale: float, causal: bool,
                    cu_seqlens: Optional[torch.Tensor], max_seqlen: Optional[int]) -> FaBwdParams:
    """Fills FaBwdParams from [B, H, N, d] tensors (strides in elements)."""
    ts = dict(q=q, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv)
    for name, t in ts.items():
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, heads, tokens, head_dim]")
        if t.dtype != q.dtype or q.dtype not in _DTYPES:
            raise ValueError("q, k, v, o, dout, dq, dk, dv must share one dtype: fp16 or bf16")
        if t.stride(3) != 1 and t.shape[3] > 1 and t.numel() > 0:
            raise ValueError(f"{name}: the head_dim dimension must be contiguous")
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    for name in ("k", "v", "dk", "dv"):
        if tuple(ts[name].shape) != (b, hkv, n, d):
            raise ValueError(f"{name} must be [batch, heads_kv, tokens, head_dim] matching q")
    for name in ("o", "dout", "dq"):
        if tuple(ts[name].shape) != tuple(q.shape):
            raise ValueError(f"{name} must match q")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (b, hq, n):
        raise ValueError("lse must be a contiguous float32 tensor [batch, heads_q, tokens]")
    if (delta.dtype != torch.float32 or not delta.is_contiguous()
            or tuple(delta.shape) != (2, b, hq, n)):
        raise ValueError("delta must be a contiguous float32 workspace [2, batch, heads_q, tokens]")
    p = FaBwdParams(
        dtype=_DTYPES[q.dtype], q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), o=o.data_ptr(),
        dout=dout.data_ptr(), lse=lse.data_ptr(), delta=delta.data_ptr(), dq=dq.data_ptr(),
        dk=dk.data_ptr(), dv=dv.data_ptr(), batch=b, heads_q=hq, heads_kv=hkv, seqlen=n,
        head_dim=d, causal=int(bool(causal)), scale=float(scale),
        q_stride=_strides(q), k_stride=_strides(k), v_stride=_strides(v), o_stride=_strides(o),
        do_stride=_strides(dout), dq_stride=_strides(dq), dk_stride=_strides(dk),
        dv_stride=_strides(dv))
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor")
        if cu_seqlens.device != q.device:
            raise ValueError("cu_seqlens must live on the same device as q")
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens")
        p.cu_seqlens = cu_seqlens.data_ptr()
        p.num_seqs = cu_seqlens.numel() - 1
        p.max_seqlen = int(max_seqlen)
    return p


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, *, scale: float, causal: bool = False,
           cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
           stream: Optional[torch.cuda.Stream] = None) -> None:
    """Enqueues the backward pass writing delta, dq, dk and dv (default: torch's stream)."""
    lib = load_library()
    for t in (q, k, v, o, dout, lse, dq, dk, dv, delta):
        if not t.is_cuda:
            raise ValueError("libfa runs on the GPU: all tensors must be on a HIP device")
    p = make_bwd_params(q, k, v, o, dout, lse, dq, dk, dv, delta, scale, causal, cu_seqlens,
                        max_seqlen)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = int(lib.fa_bwd(ctypes.byref(p), ctypes.c_void_p(s.cuda_stream)))
    if st != FA_OK:
        raise FaError(st, fa_status_string(st))


def attention_backward(q, k, v, o, lse, dout, *, scale: Optional[float] = None,
                       causal: bool = False, cu_seqlens: Optional[torch.Tensor] = None,
                       max_seqlen: Optional[int] = None):
    """(dq, dk, dv) of sum(O * dout) for O, lse = attention(q, k, v, ...) with the same
    arguments. Allocates the gradients and the fp32 delta workspace with torch."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if cu_seqlens is not None and max_seqlen is None:
        lens = (cu_seqlens[1:] - cu_seqlens[:-1]).cpu()
        max_seqlen = int(lens.max()) if lens.numel() else 0
    dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    delta = torch.empty((2, *q.shape[:3]), dtype=torch.float32, device=q.device)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, scale=scale, causal=causal,
           cu_seqlens=cu_seqlens, max_seqlen=max_seqlen)
    return dq, dk, dv


__all__ = [
    "FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_UNSUPPORTED", "FA_ERR_ALIGN", "FA_ERR_GQA",
    "FA_ERR_VARLEN", "FA_ERR_ABI", "FA_ERR_LAUNCH", "FA_F16", "FA_BF16", "FaError",
    "FaFwdParams", "attention", "fa_abi_version", "fa_check_args", "fa_fwd", "fa_params_size",
    "fa_status_string", "load_library", "make_params", "FaBwdParams", "attention_backward",
    "fa_bwd", "fa_bwd_check_args", "fa_bwd_params_size", "make_bwd_params",
]
