"""Python binding of the MSA HIP library (include/msa.h), argument marshalling only.

Every step of the path runs in the HIP kernels of ``libmsa.so``; this module
turns torch tensors into device pointers, element strides and the current HIP
stream, sizes and hands over the workspace, and raises on a non-zero status.
There is no CPU fallback: without the built library every call raises.

Entry points carry the C names:

* ``msa_index_select`` -- frozen lightning-indexer block selection;
* ``msa_attn_fwd``     -- block-sparse GQA attention forward (O, LSE);
* ``msa_attn_bwd``     -- its backward (dQ, dK, dV);
* ``msa_attn_fwd_noalloc`` -- the forward with the library's static scratch (no workspace);
* ``msa_workspace_size``, ``msa_status_string``, ``msa_check_cu_seqlens``.

``MSAAttention`` wraps forward and backward as a ``torch.autograd.Function``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsa.so")

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_UNSUPPORTED = -2
MSA_ERR_WORKSPACE = -3
MSA_ERR_HIP = -4
MSA_SELECT_FORCE_INIT = 1
MSA_ATTN_DENSE = 1
MSA_ATTN_RECOMPUTE = 2
MSA_OP_QKNORM_BWD = 4
MSA_OP_SELECT = 1
MSA_OP_FWD = 2
MSA_OP_BWD = 3
MSA_OP_QSA_FWD = 5
MSA_OP_QSA_BWD = 6
MSA_OP_BWD_QKNORM = 7
MSA_OP_BWD_RECOMPUTE = 8

# Every symbol include/msa.h declares.
EXPORTED = ("msa_workspace_size", "msa_index_select", "msa_index_select_ex", "msa_attn_fwd", "msa_attn_bwd",
            "msa_attn_fwd_ex", "msa_attn_bwd_ex", "msa_attn_fwd_qknorm", "msa_attn_bwd_qknorm",
            "msa_qk_norm_rope_fwd", "msa_qk_norm_rope_bwd", "msa_qsa_attn_fwd", "msa_qsa_attn_bwd",
            "msa_status_string", "msa_check_cu_seqlens", "msa_timing_enable", "msa_timing_collect",
            "msa_version", "msa_attn_fwd_noalloc")
MSA_NOALLOC_SCRATCH_BYTES = 72 << 20


class MsaDims(ctypes.Structure):
    _fields_ = [("total_tokens", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("max_seqlen", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("topk_blocks", ctypes.c_int32)]


class MsaKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_float)]


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    lib.msa_workspace_size.argtypes = [ctypes.POINTER(MsaDims), _I32, ctypes.POINTER(_SZ)]
    lib.msa_workspace_size.restype = _I32
    lib.msa_index_select.argtypes = [ctypes.POINTER(MsaDims), _P, _I64, _I64, _P, _I64, _I64, _P, _P,
                                     _F, _F, _I32, _P, _P, _P, _SZ, _P]
    lib.msa_index_select.restype = _I32
    lib.msa_index_select_ex.argtypes = [ctypes.POINTER(MsaDims), _P, _I64, _I64, _P, _I64, _I64, _P, _P,
                                        _F, _F, _I32, ctypes.c_uint32, _P, _P, _P, _SZ, _P]
    lib.msa_index_select_ex.restype = _I32
    lib.msa_attn_fwd.argtypes = [ctypes.POINTER(MsaDims), _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                 _P, _P, _F, _P, _I64, _I64, _P, _P, _SZ, _P]
    lib.msa_attn_fwd.restype = _I32
    lib.msa_attn_fwd_noalloc.argtypes = [ctypes.POINTER(MsaDims), _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                         _P, _P, _F, _P, _I64, _I64, _P, _P]
    lib.msa_attn_fwd_noalloc.restype = _I32
    lib.msa_attn_bwd.argtypes = [ctypes.POINTER(MsaDims),
                                 _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                 _P, _P, _I64, _I64, _P, _P, _F,
                                 _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _SZ, _P]
    lib.msa_attn_bwd.restype = _I32
    lib.msa_attn_fwd_ex.argtypes = [ctypes.POINTER(MsaDims), _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                    _P, _P, _F, ctypes.c_uint32, _P, _I64, _I64, _P, _P, _SZ, _P]
    lib.msa_attn_fwd_ex.restype = _I32
    lib.msa_attn_bwd_ex.argtypes = [ctypes.POINTER(MsaDims),
                                    _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                    _P, _P, _I64, _I64, _P, _P, _F, ctypes.c_uint32,
                                    _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _SZ, _P]
    lib.msa_attn_bwd_ex.restype = _I32
    lib.msa_attn_fwd_qknorm.argtypes = [ctypes.POINTER(MsaDims), _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                        _P, _P, _F, _F, _I32, _P, _P, _F, ctypes.c_uint32, _P, _I64, _I64, _P, _P,
                                        _SZ, _P]
    lib.msa_attn_fwd_qknorm.restype = _I32
    lib.msa_attn_bwd_qknorm.argtypes = [ctypes.POINTER(MsaDims),
                                        _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _P, _F, _F, _I32,
                                        _P, _I64, _I64, _P, _P, _I64, _I64, _P, _P, _F, ctypes.c_uint32,
                                        _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _P, _P, _SZ, _P]
    lib.msa_attn_bwd_qknorm.restype = _I32
    lib.msa_qsa_attn_fwd.argtypes = lib.msa_attn_fwd.argtypes
    lib.msa_qsa_attn_fwd.restype = _I32
    lib.msa_qsa_attn_bwd.argtypes = lib.msa_attn_bwd.argtypes
    lib.msa_qsa_attn_bwd.restype = _I32
    lib.msa_qk_norm_rope_fwd.argtypes = [ctypes.POINTER(MsaDims), _P, _I64, _I64, _P, _I64, _I64, _P, _P,
                                         _F, _F, _I32, _P, _P, _I64, _I64, _P, _I64, _I64, _P]
    lib.msa_qk_norm_rope_fwd.restype = _I32
    lib.msa_qk_norm_rope_bwd.argtypes = [ctypes.POINTER(MsaDims), _P, _I64, _I64, _P, _I64, _I64, _P, _P,
                                         _F, _F, _I32, _P, _P, _I64, _I64, _P, _I64, _I64,
                                         _P, _I64, _I64, _P, _I64, _I64, _P, _P, _P, _SZ, _P]
    lib.msa_qk_norm_rope_bwd.restype = _I32
    lib.msa_status_string.argtypes = [_I32]
    lib.msa_status_string.restype = ctypes.c_char_p
    lib.msa_check_cu_seqlens.argtypes = [ctypes.POINTER(MsaDims), _P, _P]
    lib.msa_check_cu_seqlens.restype = _I32
    lib.msa_timing_enable.argtypes = [_I32]
    lib.msa_timing_enable.restype = _I32
    lib.msa_timing_collect.argtypes = [ctypes.POINTER(MsaKernelTime), _I32, ctypes.POINTER(_I32)]
    lib.msa_timing_collect.restype = _I32
    lib.msa_version.argtypes = []
    lib.msa_version.restype = _I32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().msa_status_string(int(status)).decode()


msa_status_string = status_string


def make_dims(total_tokens: int, num_seqs: int, max_seqlen: int, num_q_heads: int, num_kv_heads: int,
              head_dim: int = 128, block_size: int = 128, topk_blocks: int = 16) -> MsaDims:
    return MsaDims(int(total_tokens), int(num_seqs), int(max_seqlen), int(num_q_heads), int(num_kv_heads),
                   int(head_dim), int(block_size), int(topk_blocks))


def msa_workspace_size(dims: MsaDims, op: int) -> int:
    n = _SZ(0)
    st = load().msa_workspace_size(ctypes.byref(dims), int(op), ctypes.byref(n))
    if st != MSA_OK:
        raise MsaError(st, "msa_workspace_size")
    return int(n.value)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _bf16_view(t: torch.Tensor, name: str, shape: Optional[Tuple[int, int, int]] = None,
               device: Optional[torch.device] = None) -> Tuple[int, int]:
    if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1 or not t.is_cuda:
        raise ValueError(f"{name}: expected a CUDA bf16 [T, H, D] tensor with a contiguous last dim")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    return t.stride(0), t.stride(1)


# The kernels read the tensors below as plain arrays (no strides), so the
# binding rejects anything else before a launch; a wrong dtype or layout there
# would be read as garbage or, for cu_seqlens, as out-of-range offsets.

def _cu_seqlens(cu: torch.Tensor, device: torch.device) -> torch.Tensor:
    if not isinstance(cu, torch.Tensor) or cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 1:
        raise ValueError("cu_seqlens: expected a 1-D int32 tensor of S+1 offsets")
    if not cu.is_cuda or cu.device != device or not cu.is_contiguous():
        raise ValueError(f"cu_seqlens: expected a contiguous int32 tensor on {device}")
    return cu


def _weight(w: torch.Tensor, name: str, device: torch.device) -> torch.Tensor:
    """A [128] bf16 norm weight; returns it contiguous (the caller keeps the
    result alive until the launch is enqueued)."""
    if not isinstance(w, torch.Tensor) or w.dtype != torch.bfloat16 or w.numel() != 128 or w.dim() != 1:
        raise ValueError(f"{name}: expected a bf16 [128] tensor")
    if not w.is_cuda or w.device != device:
        raise ValueError(f"{name}: expected a tensor on {device}")
    return w.contiguous()


def _int32_rows(b: torch.Tensor, name: str, T: int, H: int, device: torch.device,
                k: Optional[int] = None) -> torch.Tensor:
    if not isinstance(b, torch.Tensor) or b.dtype != torch.int32 or b.dim() != 3:
        raise ValueError(f"{name}: expected an int32 [T, H, K] tensor")
    if b.shape[0] != T or b.shape[1] != H or (k is not None and b.shape[2] != k):
        want = (T, H, k if k is not None else "K")
        raise ValueError(f"{name}: expected shape {want}, got {tuple(b.shape)}")
    if not b.is_cuda or b.device != device or not b.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor on {device}")
    return b


def _lse_rows(t: torch.Tensor, name: str, T: int, Hq: int, device: torch.device) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or tuple(t.shape) != (T, Hq):
        raise ValueError(f"{name}: expected an fp32 [{T}, {Hq}] tensor")
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor on {device}")
    return t



def _workspace(dims: MsaDims, op: int, device, workspace: Optional[torch.Tensor]) -> Tuple[Optional[torch.Tensor], int]:
    need = msa_workspace_size(dims, op)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, workspace.numel()


def _dims_for(cu_seqlens: torch.Tensor, max_seqlen: int, q_heads: int, kv_heads: int, T: int) -> MsaDims:
    return make_dims(T, cu_seqlens.numel() - 1, max_seqlen, q_heads, kv_heads)


def _check(st: int, where: str):
    if st != MSA_OK:
        raise MsaError(st, where)


def msa_index_select(idx_q: torch.Tensor, idx_k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                     cu_seqlens: torch.Tensor, max_seqlen: int, *, eps: float = 1e-6, rope_base: float = 1e7,
                     rope_dims: int = 64, force_init: bool = False, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block ids [T, Hk, 16] (int32, ascending, -1 padded) chosen by the frozen indexer.
    ``force_init`` keeps block 0 in every selection (msa_index_select_ex, MSA_SELECT_FORCE_INIT)."""
    lib = load()
    T, Hk, D = idx_q.shape
    dev = idx_q.device
    sq = _bf16_view(idx_q, "idx_q")
    if idx_k.dim() != 3 or idx_k.shape[0] != T or idx_k.shape[1] not in (1, Hk) or idx_k.shape[2] != D:
        raise ValueError(f"idx_k: expected shape ({T}, {Hk} or 1, {D}), got {tuple(idx_k.shape)}")
    sk = _bf16_view(idx_k, "idx_k", device=dev)
    if idx_k.shape[1] == 1 and Hk > 1:
        sk = (sk[0], 0)
    cu_seqlens = _cu_seqlens(cu_seqlens, dev)
    wq = _weight(w_q, "w_q", dev)
    wk = _weight(w_k, "w_k", dev)
    dims = _dims_for(cu_seqlens, max_seqlen, 16 * Hk, Hk, T)
    if out is None:
        out = torch.empty(T, Hk, 16, dtype=torch.int32, device=dev)
    out = _int32_rows(out, "out", T, Hk, dev, 16)
    ws, nbytes = _workspace(dims, MSA_OP_SELECT, dev, workspace)
    if force_init:
        st = lib.msa_index_select_ex(ctypes.byref(dims), _ptr(idx_q), sq[0], sq[1], _ptr(idx_k), sk[0], sk[1],
                                     _ptr(wq), _ptr(wk), float(eps), float(rope_base), int(rope_dims),
                                     MSA_SELECT_FORCE_INIT, _ptr(cu_seqlens), _ptr(out), _ptr(ws), nbytes,
                                     _stream(idx_q))
        _check(st, "msa_index_select_ex")
    else:
        st = lib.msa_index_select(ctypes.byref(dims), _ptr(idx_q), sq[0], sq[1], _ptr(idx_k), sk[0], sk[1],
                                  _ptr(wq), _ptr(wk), float(eps), float(rope_base), int(rope_dims),
                                  _ptr(cu_seqlens), _ptr(out), _ptr(ws), nbytes, _stream(idx_q))
        _check(st, "msa_index_select")
    return out


def msa_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, blk_idx: Optional[torch.Tensor],
                 cu_seqlens: torch.Tensor, max_seqlen: int, softmax_scale: Optional[float] = None, *,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, dense: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Block-sparse GQA attention forward: returns O [T, Hq, 128] bf16 and LSE [T, Hq] fp32.
    ``dense`` attends to every causal key instead (msa_attn_fwd_ex, MSA_ATTN_DENSE; blk_idx unused)."""
    lib = load()
    T, Hq, D = q.shape
    Hk = k.shape[1]
    dev = q.device
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    sq = _bf16_view(q, "q")
    sk, sv = _bf16_view(k, "k", (T, Hk, D), dev), _bf16_view(v, "v", (T, Hk, D), dev)
    cu_seqlens = _cu_seqlens(cu_seqlens, dev)
    if not dense:
        blk_idx = _int32_rows(blk_idx, "blk_idx", T, Hk, dev, 16)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    so = _bf16_view(out, "out", (T, Hq, D), dev)
    lse = _lse_rows(lse, "lse", T, Hq, dev)
    dims = _dims_for(cu_seqlens, max_seqlen, Hq, Hk, T)
    ws, nbytes = _workspace(dims, MSA_OP_FWD, dev, workspace)
    if dense:
        st = lib.msa_attn_fwd_ex(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1], _ptr(v), sv[0],
                                 sv[1], None, _ptr(cu_seqlens), scale, MSA_ATTN_DENSE, _ptr(out), so[0], so[1],
                                 _ptr(lse), _ptr(ws), nbytes, _stream(q))
        _check(st, "msa_attn_fwd_ex")
    else:
        st = lib.msa_attn_fwd(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1], _ptr(v), sv[0],
                              sv[1], _ptr(blk_idx), _ptr(cu_seqlens), scale, _ptr(out), so[0], so[1], _ptr(lse),
                              _ptr(ws), nbytes, _stream(q))
        _check(st, "msa_attn_fwd")
    return out, lse


def msa_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, blk_idx: torch.Tensor,
                         cu_seqlens: torch.Tensor, max_seqlen: int, softmax_scale: Optional[float] = None, *,
                         out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """msa_attn_fwd with the library's static device scratch instead of a workspace: the library
    allocates nothing (pass ``out`` and ``lse`` to allocate nothing here either).  Calls that overlap
    on one GPU race on that scratch."""
    lib = load()
    T, Hq, D = q.shape
    Hk = k.shape[1]
    dev = q.device
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    sq = _bf16_view(q, "q")
    sk, sv = _bf16_view(k, "k", (T, Hk, D), dev), _bf16_view(v, "v", (T, Hk, D), dev)
    cu_seqlens = _cu_seqlens(cu_seqlens, dev)
    blk_idx = _int32_rows(blk_idx, "blk_idx", T, Hk, dev, 16)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    so = _bf16_view(out, "out", (T, Hq, D), dev)
    lse = _lse_rows(lse, "lse", T, Hq, dev)
    dims = _dims_for(cu_seqlens, max_seqlen, Hq, Hk, T)
    st = lib.msa_attn_fwd_noalloc(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1], _ptr(v), sv[0],
                                  sv[1], _ptr(blk_idx), _ptr(cu_seqlens), scale, _ptr(out), so[0], so[1], _ptr(lse),
                                  _stream(q))
    _check(st, "msa_attn_fwd_noalloc")
    return out, lse


def msa_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                 do: torch.Tensor, blk_idx: Optional[torch.Tensor], cu_seqlens: torch.Tensor, max_seqlen: int,
                 softmax_scale: Optional[float] = None, *, dq: Optional[torch.Tensor] = None,
                 dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None,
                 dense: bool = False, recompute: bool = False) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of msa_attn_fwd: returns dQ, dK, dV (bf16, shaped like q, k, v); ``dense`` as in the forward.
    ``recompute`` (MSA_ATTN_RECOMPUTE): the dQ pass recomputes S and dP instead of reading the dS stored by the
    dK/dV pass; slower, with a workspace smaller by 64 KB per (token, KV head)."""
    lib = load()
    T, Hq, D = q.shape
    Hk = k.shape[1]
    dev = q.device
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if dq is None:
        dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    if dk is None:
        dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    if dv is None:
        dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    qs, ks = (T, Hq, D), (T, Hk, D)
    views = [_bf16_view(t, n, sh, dev) for t, n, sh in ((q, "q", qs), (k, "k", ks), (v, "v", ks), (o, "o", qs),
                                                         (do, "do", qs), (dq, "dq", qs), (dk, "dk", ks),
                                                         (dv, "dv", ks))]
    cu_seqlens = _cu_seqlens(cu_seqlens, dev)
    lse = _lse_rows(lse, "lse", T, Hq, dev)
    if not dense:
        blk_idx = _int32_rows(blk_idx, "blk_idx", T, Hk, dev, 16)
    dims = _dims_for(cu_seqlens, max_seqlen, Hq, Hk, T)
    flags = (MSA_ATTN_DENSE if dense else 0) | (MSA_ATTN_RECOMPUTE if recompute else 0)
    ws, nbytes = _workspace(dims, MSA_OP_BWD_RECOMPUTE if flags else MSA_OP_BWD, dev, workspace)
    (sq, sk, sv, so, sdo, sdq, sdk, sdv) = views
    if flags:
        st = lib.msa_attn_bwd_ex(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1], _ptr(v), sv[0],
                                 sv[1], _ptr(o), so[0], so[1], _ptr(lse), _ptr(do), sdo[0], sdo[1],
                                 None if dense else _ptr(blk_idx), _ptr(cu_seqlens), scale, flags, _ptr(dq), sdq[0],
                                 sdq[1], _ptr(dk), sdk[0], sdk[1], _ptr(dv), sdv[0], sdv[1], _ptr(ws), nbytes,
                                 _stream(q))
        _check(st, "msa_attn_bwd_ex")
    else:
        st = lib.msa_attn_bwd(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1], _ptr(v), sv[0],
                              sv[1], _ptr(o), so[0], so[1], _ptr(lse), _ptr(do), sdo[0], sdo[1], _ptr(blk_idx),
                              _ptr(cu_seqlens), scale, _ptr(dq), sdq[0], sdq[1], _ptr(dk), sdk[0], sdk[1],
                              _ptr(dv), sdv[0], sdv[1], _ptr(ws), nbytes, _stream(q))
        _check(st, "msa_attn_bwd")
    return dq, dk, dv


def msa_attn_fwd_qknorm(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                        blk_idx: Optional[torch.Tensor], cu_seqlens: torch.Tensor, max_seqlen: int,
                        softmax_scale: Optional[float] = None, *, eps: float = 1e-6, rope_base: float = 1e7,
                        rope_dims: int = 64, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None,
                        dense: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """msa_attn_fwd on raw q, k with the attention-side norm + partial RoPE applied inside the kernels."""
    lib = load()
    T, Hq, D = q.shape
    Hk = k.shape[1]
    dev = q.device
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    sq = _bf16_view(q, "q")
    sk, sv = _bf16_view(k, "k", (T, Hk, D), dev), _bf16_view(v, "v", (T, Hk, D), dev)
    cu_seqlens = _cu_seqlens(cu_seqlens, dev)
    wq = _weight(w_q, "w_q", dev)
    wk = _weight(w_k, "w_k", dev)
    if not dense:
        blk_idx = _int32_rows(blk_idx, "blk_idx", T, Hk, dev, 16)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    so = _bf16_view(out, "out", (T, Hq, D), dev)
    lse = _lse_rows(lse, "lse", T, Hq, dev)
    dims = _dims_for(cu_seqlens, max_seqlen, Hq, Hk, T)
    ws, nbytes = _workspace(dims, MSA_OP_FWD, dev, workspace)
    st = lib.msa_attn_fwd_qknorm(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1], _ptr(v), sv[0],
                                 sv[1], _ptr(wq), _ptr(wk), float(eps), float(rope_base),
                                 int(rope_dims), None if dense else _ptr(blk_idx), _ptr(cu_seqlens), scale,
                                 MSA_ATTN_DENSE if dense else 0, _ptr(out), so[0], so[1], _ptr(lse), _ptr(ws), nbytes,
                                 _stream(q))
    _check(st, "msa_attn_fwd_qknorm")
    return out, lse


def msa_attn_bwd_qknorm(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                        o: torch.Tensor, lse: torch.Tensor, do: torch.Tensor, blk_idx: Optional[torch.Tensor],
                        cu_seqlens: torch.Tensor, max_seqlen: int, softmax_scale: Optional[float] = None, *,
                        eps: float = 1e-6, rope_base: float = 1e7, rope_dims: int = 64,
                        workspace: Optional[torch.Tensor] = None, dense: bool = False):
    """Backward of msa_attn_fwd_qknorm: dQ, dK (for the raw q, k), dV (bf16) and dw_q, dw_k (fp32 [128])."""
    lib = load()
    T, Hq, D = q.shape
    Hk = k.shape[1]
    dev = q.device
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    dw_q = torch.empty(128, dtype=torch.float32, device=dev)
    dw_k = torch.empty(128, dtype=torch.float32, device=dev)
    qs, ks = (T, Hq, D), (T, Hk, D)
    views = [_bf16_view(t, n, sh, dev) for t, n, sh in ((q, "q", qs), (k, "k", ks), (v, "v", ks), (o, "o", qs),
                                                         (do, "do", qs), (dq, "dq", qs), (dk, "dk", ks),
                                                         (dv, "dv", ks))]
    (sq, sk, sv, so, sdo, sdq, sdk, sdv) = views
    cu_seqlens = _cu_seqlens(cu_seqlens, dev)
    lse = _lse_rows(lse, "lse", T, Hq, dev)
    wq = _weight(w_q, "w_q", dev)
    wk = _weight(w_k, "w_k", dev)
    if not dense:
        blk_idx = _int32_rows(blk_idx, "blk_idx", T, Hk, dev, 16)
    dims = _dims_for(cu_seqlens, max_seqlen, Hq, Hk, T)
    ws, nbytes = _workspace(dims, MSA_OP_BWD_QKNORM, dev, workspace)
    st = lib.msa_attn_bwd_qknorm(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1], _ptr(v), sv[0],
                                 sv[1], _ptr(wq), _ptr(wk), float(eps), float(rope_base),
                                 int(rope_dims), _ptr(o), so[0], so[1], _ptr(lse), _ptr(do), sdo[0], sdo[1],
                                 None if dense else _ptr(blk_idx), _ptr(cu_seqlens), scale,
                                 MSA_ATTN_DENSE if dense else 0, _ptr(dq), sdq[0], sdq[1], _ptr(dk), sdk[0], sdk[1],
                                 _ptr(dv), sdv[0], sdv[1], _ptr(dw_q), _ptr(dw_k), _ptr(ws), nbytes, _stream(q))
    _check(st, "msa_attn_bwd_qknorm")
    return dq, dk, dv, dw_q, dw_k


def _qsa_dims(cu_seqlens: torch.Tensor, max_seqlen: int, Hq: int, Hk: int, T: int, topk: int) -> MsaDims:
    return make_dims(T, cu_seqlens.numel() - 1, max_seqlen, Hq, Hk, head_dim=256, block_size=4, topk_blocks=topk)


def msa_qsa_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, blk_idx: torch.Tensor,
                     cu_seqlens: torch.Tensor, max_seqlen: int, softmax_scale: Optional[float] = None, *,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Narrow-block (4-token blocks, D 256, 12 q heads per KV head) forward: O [T, Hq, 256], LSE [T, Hq].
    ``blk_idx`` [T, Hk, K] int32 lists sequence-local block ids per query (K <= 1024)."""
    lib = load()
    T, Hq, D = q.shape
    Hk = k.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    sq, sk, sv = _bf16_view(q, "q"), _bf16_view(k, "k"), _bf16_view(v, "v")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty(T, Hq, dtype=torch.float32, device=q.device)
    so = _bf16_view(out, "out", (T, Hq, D), q.device)
    sk, sv = _bf16_view(k, "k", (T, Hk, D), q.device), _bf16_view(v, "v", (T, Hk, D), q.device)
    cu_seqlens = _cu_seqlens(cu_seqlens, q.device)
    lse = _lse_rows(lse, "lse", T, Hq, q.device)
    blk_idx = _int32_rows(blk_idx, "blk_idx", T, Hk, q.device)
    dims = _qsa_dims(cu_seqlens, max_seqlen, Hq, Hk, T, blk_idx.shape[2])
    ws, nbytes = _workspace(dims, MSA_OP_QSA_FWD, q.device, workspace)
    st = lib.msa_qsa_attn_fwd(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1], _ptr(v), sv[0],
                              sv[1], _ptr(blk_idx), _ptr(cu_seqlens), scale, _ptr(out), so[0], so[1], _ptr(lse),
                              _ptr(ws), nbytes, _stream(q))
    _check(st, "msa_qsa_attn_fwd")
    return out, lse


def msa_qsa_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                     do: torch.Tensor, blk_idx: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                     softmax_scale: Optional[float] = None, *, dq: Optional[torch.Tensor] = None,
                     dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of msa_qsa_attn_fwd: returns dQ, dK, dV (bf16, shaped like q, k, v)."""
    lib = load()
    T, Hq, D = q.shape
    Hk = k.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if dq is None:
        dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    if dk is None:
        dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    if dv is None:
        dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    dev = q.device
    qs, ks = (T, Hq, D), (T, Hk, D)
    views = [_bf16_view(t, n, sh, dev) for t, n, sh in ((q, "q", qs), (k, "k", ks), (v, "v", ks), (o, "o", qs),
                                                         (do, "do", qs), (dq, "dq", qs), (dk, "dk", ks),
                                                         (dv, "dv", ks))]
    cu_seqlens = _cu_seqlens(cu_seqlens, dev)
    lse = _lse_rows(lse, "lse", T, Hq, dev)
    blk_idx = _int32_rows(blk_idx, "blk_idx", T, Hk, dev)
    dims = _qsa_dims(cu_seqlens, max_seqlen, Hq, Hk, T, blk_idx.shape[2])
    ws, nbytes = _workspace(dims, MSA_OP_QSA_BWD, q.device, workspace)
    (sq, sk, sv, so, sdo, sdq, sdk, sdv) = views
    st = lib.msa_qsa_attn_bwd(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1], _ptr(v), sv[0],
                              sv[1], _ptr(o), so[0], so[1], _ptr(lse), _ptr(do), sdo[0], sdo[1], _ptr(blk_idx),
                              _ptr(cu_seqlens), scale, _ptr(dq), sdq[0], sdq[1], _ptr(dk), sdk[0], sdk[1],
                              _ptr(dv), sdv[0], sdv[1], _ptr(ws), nbytes, _stream(q))
    _check(st, "msa_qsa_attn_bwd")
    return dq, dk, dv


def msa_qk_norm_rope_fwd(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                         cu_seqlens: torch.Tensor, max_seqlen: int, *, eps: float = 1e-6, rope_base: float = 1e7,
                         rope_dims: int = 64, q_out: Optional[torch.Tensor] = None,
                         k_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention-side per-head gemma norm + partial RoPE of q [T, Hq, 128] and k [T, Hk, 128]."""
    lib = load()
    T, Hq, _ = q.shape
    Hk = k.shape[1]
    if q_out is None:
        q_out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if k_out is None:
        k_out = torch.empty(k.shape, dtype=k.dtype, device=k.device)
    dev = q.device
    D = q.shape[2]
    sq, sk, sqo, sko = (_bf16_view(t, n, sh, dev) for t, n, sh in
                        ((q, "q", (T, Hq, D)), (k, "k", (T, Hk, D)), (q_out, "q_out", (T, Hq, D)),
                         (k_out, "k_out", (T, Hk, D))))
    cu_seqlens = _cu_seqlens(cu_seqlens, dev)
    wq = _weight(w_q, "w_q", dev)
    wk = _weight(w_k, "w_k", dev)
    dims = _dims_for(cu_seqlens, max_seqlen, Hq, Hk, T)
    st = lib.msa_qk_norm_rope_fwd(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1],
                                  _ptr(wq), _ptr(wk), float(eps), float(rope_base),
                                  int(rope_dims), _ptr(cu_seqlens), _ptr(q_out), sqo[0], sqo[1], _ptr(k_out),
                                  sko[0], sko[1], _stream(q))
    _check(st, "msa_qk_norm_rope_fwd")
    return q_out, k_out


def msa_qk_norm_rope_bwd(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                         cu_seqlens: torch.Tensor, max_seqlen: int, dq_hat: torch.Tensor, dk_hat: torch.Tensor, *,
                         eps: float = 1e-6, rope_base: float = 1e7, rope_dims: int = 64,
                         workspace: Optional[torch.Tensor] = None):
    """Backward of msa_qk_norm_rope_fwd: returns dq, dk (bf16) and dw_q, dw_k (fp32 [128])."""
    lib = load()
    T, Hq, _ = q.shape
    Hk = k.shape[1]
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device)
    dw_q = torch.empty(128, dtype=torch.float32, device=q.device)
    dw_k = torch.empty(128, dtype=torch.float32, device=q.device)
    dev = q.device
    D = q.shape[2]
    qs, ks = (T, Hq, D), (T, Hk, D)
    views = [_bf16_view(t, n, sh, dev) for t, n, sh in ((q, "q", qs), (k, "k", ks), (dq_hat, "dq_hat", qs),
                                                         (dk_hat, "dk_hat", ks), (dq, "dq", qs), (dk, "dk", ks))]
    sq, sk, sdqh, sdkh, sdq, sdk = views
    cu_seqlens = _cu_seqlens(cu_seqlens, dev)
    wq = _weight(w_q, "w_q", dev)
    wk = _weight(w_k, "w_k", dev)
    dims = _dims_for(cu_seqlens, max_seqlen, Hq, Hk, T)
    ws, nbytes = _workspace(dims, MSA_OP_QKNORM_BWD, dev, workspace)
    st = lib.msa_qk_norm_rope_bwd(ctypes.byref(dims), _ptr(q), sq[0], sq[1], _ptr(k), sk[0], sk[1],
                                  _ptr(wq), _ptr(wk), float(eps), float(rope_base),
                                  int(rope_dims), _ptr(cu_seqlens), _ptr(dq_hat), sdqh[0], sdqh[1], _ptr(dk_hat),
                                  sdkh[0], sdkh[1], _ptr(dq), sdq[0], sdq[1], _ptr(dk), sdk[0], sdk[1], _ptr(dw_q),
                                  _ptr(dw_k), _ptr(ws), nbytes, _stream(q))
    _check(st, "msa_qk_norm_rope_bwd")
    return dq, dk, dw_q, dw_k


def msa_check_cu_seqlens(cu_seqlens: torch.Tensor, total_tokens: int, max_seqlen: int,
                         num_q_heads: int = 16, num_kv_heads: int = 1) -> int:
    """Debug check of the cu_seqlens contract (synchronizes the stream); returns the status."""
    cu_seqlens = _cu_seqlens(cu_seqlens, cu_seqlens.device)
    dims = make_dims(total_tokens, cu_seqlens.numel() - 1, max_seqlen, num_q_heads, num_kv_heads)
    return int(load().msa_check_cu_seqlens(ctypes.byref(dims), _ptr(cu_seqlens), _stream(cu_seqlens)))


def msa_timing_enable(enable: bool = True) -> None:
    """Bracket every kernel launch with HIP events on its stream (see msa_timing_collect)."""
    _check(load().msa_timing_enable(1 if enable else 0), "msa_timing_enable")


def msa_timing_collect() -> dict:
    """{kernel name: (launches, total ms)} since the previous collect; waits for the events."""
    cap = 64
    arr = (MsaKernelTime * cap)()
    n = _I32(0)
    _check(load().msa_timing_collect(arr, cap, ctypes.byref(n)), "msa_timing_collect")
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(n.value)}


class MSAAttention(torch.autograd.Function):
    """Block-sparse attention with autograd: apply(q, k, v, blk_idx, cu_seqlens, max_seqlen, scale)."""

    @staticmethod
    def forward(ctx, q, k, v, blk_idx, cu_seqlens, max_seqlen, softmax_scale=None):
        o, lse = msa_attn_fwd(q, k, v, blk_idx, cu_seqlens, max_seqlen, softmax_scale)
        ctx.save_for_backward(q, k, v, o, lse, blk_idx, cu_seqlens)
        ctx.max_seqlen = max_seqlen
        ctx.scale = softmax_scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, blk_idx, cu = ctx.saved_tensors
        dq, dk, dv = msa_attn_bwd(q, k, v, o, lse, do.contiguous(), blk_idx, cu, ctx.max_seqlen, ctx.scale)
        return dq, dk, dv, None, None, None, None
