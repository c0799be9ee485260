"""Python binding of libcpattn (ctypes): argument marshalling only.

Each function has the name of the C entry point it calls and performs no
computation of its own: tensors are turned into (pointer, strides), the
current torch stream is passed along, and a non-zero status raises
``CpattnError`` with the library's message. There is no fallback path: if the
shared library is missing, every call raises.

Tensor layouts (torch tensors on the GPU):
  q, k, v, dout          [B, H, T, D]  bf16 or fp32, last dimension contiguous
  o, dq/dk/dv accum.     [B, H, T, D]  fp32
  lse, delta             [B, H, T]     fp32
A position map is a 4-tuple (len, split, d0, d1): local index i sits at global
position i + (d0 if i < split else d1).
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

__all__ = [
    "CpattnError", "lib_path", "load", "cpattn_version", "cpattn_last_error", "cpattn_headtail_shard",
    "cpattn_rope_table", "cpattn_rope_rotate", "cpattn_rope_rotate_grad", "cpattn_block_fwd", "cpattn_lse_merge",
    "cpattn_ring_fwd_workspace_bytes",
    "cpattn_ring_fwd", "cpattn_bwd_preprocess", "cpattn_block_bwd", "cpattn_block_bwd_dkdv", "cpattn_block_bwd_dq",
    "cpattn_step_rows", "cpattn_block_fwd_gqa", "cpattn_block_bwd_gqa", "cpattn_ring_bwd_workspace_bytes",
    "cpattn_ring_bwd", "cpattn_block_fwd_merge", "cpattn_ring_bwd_noalloc", "NOALLOC_MAX_ROWS", "EXPORTS",
    "cpattn_block_bwd_staged_workspace_bytes", "cpattn_block_bwd_staged", "cpattn_ring_bwd_staged_workspace_bytes",
    "cpattn_block_fwd_rotq",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libcpattn.so")

CPATTN_F32, CPATTN_BF16 = 0, 1

EXPORTS = (
    "cpattn_version", "cpattn_last_error", "cpattn_headtail_shard", "cpattn_rope_table", "cpattn_block_fwd",
    "cpattn_lse_merge", "cpattn_ring_fwd_workspace_bytes", "cpattn_ring_fwd", "cpattn_bwd_preprocess",
    "cpattn_block_bwd", "cpattn_block_bwd_dkdv", "cpattn_block_bwd_dq", "cpattn_step_rows", "cpattn_rope_rotate",
    "cpattn_rope_rotate_grad", "cpattn_block_fwd_gqa", "cpattn_block_bwd_gqa", "cpattn_ring_bwd_workspace_bytes",
    "cpattn_ring_bwd", "cpattn_block_fwd_merge", "cpattn_ring_bwd_noalloc", "cpattn_block_bwd_staged_workspace_bytes",
    "cpattn_block_bwd_staged", "cpattn_ring_bwd_staged_workspace_bytes", "cpattn_block_fwd_rotq",
)

NOALLOC_MAX_ROWS = 1 << 20  # CPATTN_NOALLOC_MAX_ROWS: B*H*Tq limit of cpattn_ring_bwd_noalloc


class CpattnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libcpattn error {code}: {msg}")
        self.code = code


class cpattn_posmap(ctypes.Structure):
    _fields_ = [("len", ctypes.c_int64), ("split", ctypes.c_int64), ("d0", ctypes.c_int64), ("d1", ctypes.c_int64)]


class cpattn_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64), ("st", ctypes.c_int64)]


_P = ctypes.POINTER
_i32, _i64, _f32, _f64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
_T, _M = _P(cpattn_tensor), _P(cpattn_posmap)

_SIGS = {
    "cpattn_version": (ctypes.c_int, []),
    "cpattn_last_error": (ctypes.c_char_p, []),
    "cpattn_headtail_shard": (ctypes.c_int, [_i64, _i32, _i32, _M, _P(_i32)]),
    "cpattn_rope_table": (ctypes.c_int, [_f64, _i64, _i64, _vp, _vp]),
    "cpattn_block_fwd": (ctypes.c_int, [_T, _T, _T, _i32, _i64, _i64, _i64, _i64, _i64, _M, _M, _i32, _f32, _vp,
                                        _i64, _i64, _i64, _T, _T, _vp]),
    "cpattn_lse_merge": (ctypes.c_int, [_T, _T, _T, _T, _i64, _i64, _i64, _i64, _i64, _i64, _vp]),
    "cpattn_step_rows": (ctypes.c_int, [_M, _M, _i32, _P(_i64), _P(_i64)]),
    "cpattn_rope_rotate": (ctypes.c_int, [_T, _i32, _i64, _i64, _i64, _i64, _M, _vp, _i64, _T, _vp]),
    "cpattn_rope_rotate_grad": (ctypes.c_int, [_T, _i64, _i64, _i64, _i64, _M, _vp, _i64, _vp]),
    "cpattn_block_fwd_gqa": (ctypes.c_int, [_T, _T, _T, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _M, _M, _i32, _f32,
                                            _vp, _i64, _i64, _i64, _T, _T, _vp]),
    "cpattn_block_bwd_gqa": (ctypes.c_int, [_T, _T, _T, _T, _i32, _T, _T, _T, _T, _T, _i64, _i64, _i64, _i64, _i64,
                                            _i64, _M, _M, _i32, _f32, _i32, _vp]),
    "cpattn_ring_fwd_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, _i64, ctypes.c_int32]),
    "cpattn_ring_fwd": (ctypes.c_int, [_T, _T, _T, _M, _i32, _i32, _M, _i32, _i64, _i64, _i64, _i64, _i64, _i32,
                                       _f32, _vp, _i64, _T, _T, _vp, ctypes.c_size_t, _vp]),
    "cpattn_bwd_preprocess": (ctypes.c_int, [_T, _i32, _T, _T, _i64, _i64, _i64, _i64, _vp]),
    "cpattn_block_bwd": (ctypes.c_int, [_T, _T, _T, _T, _i32, _T, _T, _T, _T, _T, _i64, _i64, _i64, _i64, _i64, _M,
                                        _M, _i32, _f32, _i32, _vp]),
    "cpattn_block_bwd_dkdv": (ctypes.c_int, [_T, _T, _T, _T, _i32, _T, _T, _T, _T, _i64, _i64, _i64, _i64, _i64, _M,
                                             _M, _i32, _f32, _i32, _vp]),
    "cpattn_block_bwd_dq": (ctypes.c_int, [_T, _T, _T, _T, _i32, _T, _T, _T, _i64, _i64, _i64, _i64, _i64, _M, _M,
                                           _i32, _f32, _i32, _vp]),
    "cpattn_block_fwd_merge": (ctypes.c_int, [_T, _T, _T, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _M, _M, _i32,
                                              _f32, _i64, _i64, _T, _T, _vp]),
    "cpattn_block_fwd_rotq": (ctypes.c_int, [_T, _T, _T, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _M, _M, _i32,
                                             _f32, _vp, _i64, _i64, _i64, _i32, _T, _T, _vp]),
    "cpattn_ring_bwd_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "cpattn_ring_bwd_staged_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, _i64]),
    "cpattn_block_bwd_staged_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, _i64]),
    "cpattn_block_bwd_staged": (ctypes.c_int, [_T, _T, _T, _T, _i32, _T, _T, _T, _T, _T, _i64, _i64, _i64, _i64,
                                               _i64, _i64, _M, _M, _i32, _f32, _i32, _vp, ctypes.c_size_t, _vp]),
    "cpattn_ring_bwd": (ctypes.c_int, [_T, _T, _T, _M, _i32, _i32, _M, _i32, _i64, _i64, _i64, _i64, _i64, _i32,
                                       _f32, _T, _T, _T, _T, _T, _T, _i32, _vp, ctypes.c_size_t, _vp]),
    "cpattn_ring_bwd_noalloc": (ctypes.c_int, [_T, _T, _T, _M, _i32, _i32, _M, _i32, _i64, _i64, _i64, _i64, _i64,
                                               _i32, _f32, _T, _T, _T, _T, _T, _T, _i32, _vp]),
}

_lib = None


def load():
    """Load libcpattn.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise CpattnError(-100, f"{lib_path} is missing: build it with context_causal_attention_cpattn_amd/build.py")
        lib = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise CpattnError(status, load().cpattn_last_error().decode())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _tensor(t, ndim: int = 4) -> cpattn_tensor:
    if t.dim() != ndim:
        raise ValueError(f"expected a {ndim}-D tensor, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError("libcpattn takes GPU tensors")
    if ndim == 4 and t.stride(3) != 1 and t.shape[3] > 1:
        raise ValueError("the last dimension must be contiguous")
    s = t.stride()
    return cpattn_tensor(t.data_ptr(), s[0], s[1], s[2])


def _map(m) -> cpattn_posmap:
    if isinstance(m, cpattn_posmap):
        return m
    return cpattn_posmap(*[int(x) for x in m])


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return CPATTN_BF16
    if t.dtype == torch.float32:
        return CPATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _f32():
    import torch
    return torch.float32


def _expect(name: str, t, shape, dtype, like=None):
    """Reject a tensor whose shape, dtype or device does not match what the kernels will
    address: the C ABI sees pointers and strides only and cannot check buffer extents."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name}: on {t.device}, expected {like.device}")


def _inputs(q, k, v, H_kv=None):
    """q [B,H,Tq,D] bf16 or fp32; k, v [B,H_kv,Tk,D] of q's dtype. Returns (B,H,H_kv,Tq,Tk,D)."""
    if q is None or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, H, Tq, D]")
    _dtype(q)
    B, H, Tq, D = q.shape
    if k is None or k.dim() != 4:
        raise ValueError("k must be a 4-D tensor [B, H_kv, Tk, D]")
    Hk, Tk = k.shape[1], k.shape[2]
    if H_kv is not None and Hk != H_kv:
        raise ValueError(f"k has {Hk} heads, expected {H_kv}")
    _expect("k", k, (B, Hk, Tk, D), q.dtype, q)
    _expect("v", v, (B, Hk, Tk, D), q.dtype, q)
    return B, H, Hk, Tq, Tk, D


def _rope_check(rope_table, D, like):
    if rope_table is None:
        return
    if rope_table.dim() != 2 or rope_table.shape[1] != D:
        raise ValueError(f"rope_table: shape {tuple(rope_table.shape)}, expected [rows, {D}]")
    _expect("rope_table", rope_table, rope_table.shape, _f32(), like)
    if not rope_table.is_contiguous():
        raise ValueError("rope_table must be contiguous")


def cpattn_version() -> int:
    return load().cpattn_version()


def cpattn_last_error() -> str:
    return load().cpattn_last_error().decode()


def cpattn_headtail_shard(T: int, ring: int, rank: int):
    """Return ((len, split, d0, d1), positions) of rank ``rank`` (host call)."""
    m = cpattn_posmap()
    n = T // (2 * ring) * 2 if ring > 0 and T > 0 else 0
    pos = (ctypes.c_int32 * max(n, 1))()
    _check(load().cpattn_headtail_shard(T, ring, rank, ctypes.byref(m), pos))
    return (m.len, m.split, m.d0, m.d1), list(pos[: m.len])


def cpattn_rope_table(theta: float, rows: int, D: int, table, stream=None):
    """Fill ``table`` (fp32 GPU tensor of rows*D elements) with (cos, sin) pairs."""
    if table.numel() < rows * D or not table.is_contiguous():
        raise ValueError("table must be a contiguous fp32 tensor of rows*D elements")
    _check(load().cpattn_rope_table(float(theta), rows, D, ctypes.c_void_p(table.data_ptr()), _stream(stream)))


def _rope_args(rope_table):
    if rope_table is None:
        return None, 0
    return ctypes.c_void_p(rope_table.data_ptr()), rope_table.shape[0]


def cpattn_block_fwd(q, k, v, qmap, kmap, o, lse, causal: bool = True, scale: float = 0.0, rope_table=None,
                     row_begin: int = 0, row_end: int | None = None, stream=None):
    """O, LSE of rows [row_begin, row_end) of q against one KV block (rope_table: [rows, D] fp32)."""
    B, H, _, Tq, Tk, D = _inputs(q, k, v, q.shape[1] if q is not None and q.dim() == 4 else None)
    _expect("o", o, (B, H, Tq, D), _f32(), q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    _rope_check(rope_table, D, q)
    rp, rr = _rope_args(rope_table)
    _check(load().cpattn_block_fwd(
        _tensor(q), _tensor(k), _tensor(v), _dtype(q), B, H, Tq, Tk, D, _map(qmap), _map(kmap), int(causal),
        float(scale), rp, rr, row_begin, Tq if row_end is None else row_end, _tensor(o), _tensor(lse, 3),
        _stream(stream)))


def cpattn_lse_merge(o_acc, lse_acc, o_blk, lse_blk, row_begin: int = 0, row_end: int | None = None, stream=None):
    if o_acc is None or o_acc.dim() != 4:
        raise ValueError("o_acc must be a 4-D tensor [B, H, T, D]")
    B, H, T, D = o_acc.shape
    _expect("o_acc", o_acc, (B, H, T, D), _f32())
    _expect("lse_acc", lse_acc, (B, H, T), _f32(), o_acc)
    _expect("o_blk", o_blk, (B, H, T, D), _f32(), o_acc)
    _expect("lse_blk", lse_blk, (B, H, T), _f32(), o_acc)
    _check(load().cpattn_lse_merge(_tensor(o_acc), _tensor(lse_acc, 3), _tensor(o_blk), _tensor(lse_blk, 3), B, H, T,
                                   D, row_begin, T if row_end is None else row_end, _stream(stream)))


def cpattn_step_rows(qmap, kmap, causal: bool = True):
    """(row_begin, visible_keys): local rows [row_begin, len) see keys [0, visible_keys) of the block."""
    rb, nk = ctypes.c_int64(), ctypes.c_int64()
    _check(load().cpattn_step_rows(_map(qmap), _map(kmap), int(causal), ctypes.byref(rb), ctypes.byref(nk)))
    return rb.value, nk.value


def cpattn_ring_fwd_workspace_bytes(B: int, H: int, Tq: int, D: int, Tk: int | None = None, rope: bool = False) -> int:
    return int(load().cpattn_ring_fwd_workspace_bytes(B, H, Tq, Tq if Tk is None else Tk, D, int(bool(rope))))


def cpattn_rope_rotate(x, qmap, rope_table, out=None, stream=None):
    """out (default: x itself) = x rotated row by row at the global positions of ``qmap``."""
    if x is None or x.dim() != 4:
        raise ValueError("x must be a 4-D tensor [B, H, T, D]")
    _dtype(x)
    B, H, T, D = x.shape
    out = x if out is None else out
    _expect("out", out, (B, H, T, D), x.dtype, x)
    if rope_table is None:
        raise ValueError("rope_table is required")
    _rope_check(rope_table, D, x)
    rp, rr = _rope_args(rope_table)
    _check(load().cpattn_rope_rotate(_tensor(x), _dtype(x), B, H, T, D, _map(qmap), rp, rr, _tensor(out),
                                     _stream(stream)))
    return out


def cpattn_rope_rotate_grad(g, qmap, rope_table, stream=None):
    """In place: g (fp32, gradient with respect to rotated rows) <- R(pos)^T g."""
    if g is None or g.dim() != 4:
        raise ValueError("g must be a 4-D tensor [B, H, T, D]")
    B, H, T, D = g.shape
    _expect("g", g, (B, H, T, D), _f32())
    if rope_table is None:
        raise ValueError("rope_table is required")
    _rope_check(rope_table, D, g)
    rp, rr = _rope_args(rope_table)
    _check(load().cpattn_rope_rotate_grad(_tensor(g), B, H, T, D, _map(qmap), rp, rr, _stream(stream)))
    return g


def cpattn_ring_fwd(q, k_blocks: Sequence, v_blocks: Sequence, kmaps: Sequence, rank: int, qmap, o_acc, lse_acc,
                    workspace, causal: bool = True, scale: float = 0.0, rope_table=None, stream=None):
    """Ring forward of rank ``rank``; k_blocks[i]/v_blocks[i]/kmaps[i] belong to rank i."""
    n = len(k_blocks)
    if len(v_blocks) != n or len(kmaps) != n:
        raise ValueError("k_blocks, v_blocks, kmaps must have the same length")
    if n < 1:
        raise ValueError("at least one KV block is needed")
    B, H, _, Tq, Tk, D = _inputs(q, k_blocks[0], v_blocks[0], q.shape[1] if q is not None and q.dim() == 4 else None)
    for i in range(n):
        _expect(f"k_blocks[{i}]", k_blocks[i], (B, H, Tk, D), q.dtype, q)
        _expect(f"v_blocks[{i}]", v_blocks[i], (B, H, Tk, D), q.dtype, q)
    _expect("o_acc", o_acc, (B, H, Tq, D), _f32(), q)
    _expect("lse_acc", lse_acc, (B, H, Tq), _f32(), q)
    _rope_check(rope_table, D, q)
    if workspace is not None and workspace.device != q.device:
        raise ValueError(f"workspace: on {workspace.device}, expected {q.device}")
    ks = (cpattn_tensor * n)(*[_tensor(t) for t in k_blocks])
    vs = (cpattn_tensor * n)(*[_tensor(t) for t in v_blocks])
    ms = (cpattn_posmap * n)(*[_map(m) for m in kmaps])
    rp, rr = _rope_args(rope_table)
    ws = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().cpattn_ring_fwd(_tensor(q), ks, vs, ms, n, rank, _map(qmap), _dtype(q), B, H, Tq, Tk, D,
                                  int(causal), float(scale), rp, rr, _tensor(o_acc), _tensor(lse_acc, 3), ws, wsb,
                                  _stream(stream)))


def cpattn_ring_bwd_workspace_bytes(B: int, H: int, Tq: int) -> int:
    return int(load().cpattn_ring_bwd_workspace_bytes(B, H, Tq))


def cpattn_ring_bwd_staged_workspace_bytes(B: int, H: int, Tq: int, Tk: int, D: int) -> int:
    return int(load().cpattn_ring_bwd_staged_workspace_bytes(B, H, Tq, Tk, D))


def cpattn_ring_bwd(q, k_blocks: Sequence, v_blocks: Sequence, kmaps: Sequence, rank: int, qmap, dout, o, lse, dq_acc,
                    dk_blocks: Sequence, dv_blocks: Sequence, workspace, causal: bool = True, scale: float = 0.0,
                    accumulate: bool = True, stream=None):
    """Ring backward of rank ``rank``: dq_acc gets the local rows' gradient, dk_blocks[i] / dv_blocks[i] this
    rank's contribution to block i's."""
    n = len(k_blocks)
    if len(v_blocks) != n or len(kmaps) != n or len(dk_blocks) != n or len(dv_blocks) != n:
        raise ValueError("k_blocks, v_blocks, kmaps, dk_blocks, dv_blocks must have the same length")
    if n < 1:
        raise ValueError("at least one KV block is needed")
    B, H, _, Tq, Tk, D = _inputs(q, k_blocks[0], v_blocks[0], q.shape[1] if q is not None and q.dim() == 4 else None)
    for i in range(n):
        _expect(f"k_blocks[{i}]", k_blocks[i], (B, H, Tk, D), q.dtype, q)
        _expect(f"v_blocks[{i}]", v_blocks[i], (B, H, Tk, D), q.dtype, q)
        _expect(f"dk_blocks[{i}]", dk_blocks[i], (B, H, Tk, D), _f32(), q)
        _expect(f"dv_blocks[{i}]", dv_blocks[i], (B, H, Tk, D), _f32(), q)
    _expect("dout", dout, (B, H, Tq, D), q.dtype, q)
    _expect("o", o, (B, H, Tq, D), _f32(), q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    _expect("dq_acc", dq_acc, (B, H, Tq, D), _f32(), q)
    if workspace is not None and workspace.device != q.device:
        raise ValueError(f"workspace: on {workspace.device}, expected {q.device}")
    ks = (cpattn_tensor * n)(*[_tensor(t) for t in k_blocks])
    vs = (cpattn_tensor * n)(*[_tensor(t) for t in v_blocks])
    dks = (cpattn_tensor * n)(*[_tensor(t) for t in dk_blocks])
    dvs = (cpattn_tensor * n)(*[_tensor(t) for t in dv_blocks])
    ms = (cpattn_posmap * n)(*[_map(m) for m in kmaps])
    ws = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().cpattn_ring_bwd(_tensor(q), ks, vs, ms, n, rank, _map(qmap), _dtype(q), B, H, Tq, Tk, D,
                                  int(causal), float(scale), _tensor(dout), _tensor(o), _tensor(lse, 3),
                                  _tensor(dq_acc), dks, dvs, int(accumulate), ws, wsb, _stream(stream)))


def cpattn_ring_bwd_noalloc(q, k_blocks: Sequence, v_blocks: Sequence, kmaps: Sequence, rank: int, qmap, dout, o,
                            lse, dq_acc, dk_blocks: Sequence, dv_blocks: Sequence, causal: bool = True,
                            scale: float = 0.0, accumulate: bool = True, stream=None):
    """cpattn_ring_bwd with its fp32 delta in the library's static device array instead of a caller
    workspace (B*H*Tq <= NOALLOC_MAX_ROWS); allocates nothing. Calls that overlap on one GPU race."""
    n = len(k_blocks)
    if len(v_blocks) != n or len(kmaps) != n or len(dk_blocks) != n or len(dv_blocks) != n:
        raise ValueError("k_blocks, v_blocks, kmaps, dk_blocks, dv_blocks must have the same length")
    if n < 1:
        raise ValueError("at least one KV block is needed")
    B, H, _, Tq, Tk, D = _inputs(q, k_blocks[0], v_blocks[0], q.shape[1] if q is not None and q.dim() == 4 else None)
    for i in range(n):
        _expect(f"k_blocks[{i}]", k_blocks[i], (B, H, Tk, D), q.dtype, q)
        _expect(f"v_blocks[{i}]", v_blocks[i], (B, H, Tk, D), q.dtype, q)
        _expect(f"dk_blocks[{i}]", dk_blocks[i], (B, H, Tk, D), _f32(), q)
        _expect(f"dv_blocks[{i}]", dv_blocks[i], (B, H, Tk, D), _f32(), q)
    _expect("dout", dout, (B, H, Tq, D), q.dtype, q)
    _expect("o", o, (B, H, Tq, D), _f32(), q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    _expect("dq_acc", dq_acc, (B, H, Tq, D), _f32(), q)
    ks = (cpattn_tensor * n)(*[_tensor(t) for t in k_blocks])
    vs = (cpattn_tensor * n)(*[_tensor(t) for t in v_blocks])
    dks = (cpattn_tensor * n)(*[_tensor(t) for t in dk_blocks])
    dvs = (cpattn_tensor * n)(*[_tensor(t) for t in dv_blocks])
    ms = (cpattn_posmap * n)(*[_map(m) for m in kmaps])
    _check(load().cpattn_ring_bwd_noalloc(_tensor(q), ks, vs, ms, n, rank, _map(qmap), _dtype(q), B, H, Tq, Tk, D,
                                          int(causal), float(scale), _tensor(dout), _tensor(o), _tensor(lse, 3),
                                          _tensor(dq_acc), dks, dvs, int(accumulate), _stream(stream)))


def cpattn_bwd_preprocess(dout, o, delta, stream=None):
    if dout is None or dout.dim() != 4:
        raise ValueError("dout must be a 4-D tensor [B, H, Tq, D]")
    _dtype(dout)
    B, H, Tq, D = dout.shape
    _expect("o", o, (B, H, Tq, D), _f32(), dout)
    _expect("delta", delta, (B, H, Tq), _f32(), dout)
    _check(load().cpattn_bwd_preprocess(_tensor(dout), _dtype(dout), _tensor(o), _tensor(delta, 3), B, H, Tq, D,
                                        _stream(stream)))


def cpattn_block_bwd(q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc, qmap, kmap, causal: bool = True,
                     scale: float = 0.0, accumulate: bool = True, stream=None):
    B, H, H_kv, Tq, Tk, D = _inputs(q, k, v, q.shape[1] if q is not None and q.dim() == 4 else None)
    _expect("dout", dout, (B, H, Tq, D), q.dtype, q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    _expect("delta", delta, (B, H, Tq), _f32(), q)
    _expect("dq_acc", dq_acc, (B, H, Tq, D), _f32(), q)
    _expect("dk_acc", dk_acc, (B, H_kv, Tk, D), _f32(), q)
    _expect("dv_acc", dv_acc, (B, H_kv, Tk, D), _f32(), q)
    _check(load().cpattn_block_bwd(_tensor(q), _tensor(k), _tensor(v), _tensor(dout), _dtype(q), _tensor(lse, 3),
                                   _tensor(delta, 3), _tensor(dq_acc), _tensor(dk_acc), _tensor(dv_acc), B, H, Tq, Tk,
                                   D, _map(qmap), _map(kmap), int(causal), float(scale), int(accumulate),
                                   _stream(stream)))


def cpattn_block_bwd_dkdv(q, k, v, dout, lse, delta, dk_acc, dv_acc, qmap, kmap, causal: bool = True,
                          scale: float = 0.0, accumulate: bool = True, stream=None):
    B, H, H_kv, Tq, Tk, D = _inputs(q, k, v, q.shape[1] if q is not None and q.dim() == 4 else None)
    _expect("dout", dout, (B, H, Tq, D), q.dtype, q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    _expect("delta", delta, (B, H, Tq), _f32(), q)
    _expect("dk_acc", dk_acc, (B, H_kv, Tk, D), _f32(), q)
    _expect("dv_acc", dv_acc, (B, H_kv, Tk, D), _f32(), q)
    _check(load().cpattn_block_bwd_dkdv(_tensor(q), _tensor(k), _tensor(v), _tensor(dout), _dtype(q),
                                        _tensor(lse, 3), _tensor(delta, 3), _tensor(dk_acc), _tensor(dv_acc), B, H, Tq,
                                        Tk, D, _map(qmap), _map(kmap), int(causal), float(scale), int(accumulate),
                                        _stream(stream)))


def cpattn_block_bwd_dq(q, k, v, dout, lse, delta, dq_acc, qmap, kmap, causal: bool = True, scale: float = 0.0,
                        accumulate: bool = True, stream=None):
    B, H, H_kv, Tq, Tk, D = _inputs(q, k, v, q.shape[1] if q is not None and q.dim() == 4 else None)
    _expect("dout", dout, (B, H, Tq, D), q.dtype, q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    _expect("delta", delta, (B, H, Tq), _f32(), q)
    _expect("dq_acc", dq_acc, (B, H, Tq, D), _f32(), q)
    _check(load().cpattn_block_bwd_dq(_tensor(q), _tensor(k), _tensor(v), _tensor(dout), _dtype(q), _tensor(lse, 3),
                                      _tensor(delta, 3), _tensor(dq_acc), B, H, Tq, Tk, D, _map(qmap), _map(kmap),
                                      int(causal), float(scale), int(accumulate), _stream(stream)))


def cpattn_block_fwd_gqa(q, k, v, qmap, kmap, o, lse, causal: bool = True, scale: float = 0.0, rope_table=None,
                         row_begin: int = 0, row_end: int | None = None, stream=None):
    """Grouped-query block forward: q [B,H,Tq,D], k / v [B,H_kv,Tk,D], query head h uses KV head h // (H // H_kv)."""
    B, H, H_kv, Tq, Tk, D = _inputs(q, k, v)
    _expect("o", o, (B, H, Tq, D), _f32(), q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    _rope_check(rope_table, D, q)
    rp, rr = _rope_args(rope_table)
    row_end = Tq if row_end is None else row_end
    _check(load().cpattn_block_fwd_gqa(_tensor(q), _tensor(k), _tensor(v), _dtype(q), B, H, H_kv, Tq, Tk, D,
                                       _map(qmap), _map(kmap), int(causal), float(scale), rp, rr, row_begin, row_end,
                                       _tensor(o), _tensor(lse, 3), _stream(stream)))


def cpattn_block_fwd_merge(q, k, v, qmap, kmap, o_acc, lse_acc, causal: bool = True, scale: float = 0.0,
                           row_begin: int = 0, row_end: int | None = None, stream=None):
    """Block forward of rows [row_begin, row_end) folded into the running (o_acc, lse_acc) in one launch
    (k / v may have fewer heads than q: grouped-query)."""
    B, H, H_kv, Tq, Tk, D = _inputs(q, k, v)
    _expect("o_acc", o_acc, (B, H, Tq, D), _f32(), q)
    _expect("lse_acc", lse_acc, (B, H, Tq), _f32(), q)
    row_end = Tq if row_end is None else row_end
    _check(load().cpattn_block_fwd_merge(_tensor(q), _tensor(k), _tensor(v), _dtype(q), B, H, H_kv, Tq, Tk, D,
                                         _map(qmap), _map(kmap), int(causal), float(scale), row_begin, row_end,
                                         _tensor(o_acc), _tensor(lse_acc, 3), _stream(stream)))


def cpattn_block_fwd_rotq(q, k, v, qmap, kmap, o, lse, rope_table, causal: bool = True, scale: float = 0.0,
                          row_begin: int = 0, row_end: int | None = None, merge: bool = False, stream=None):
    """Block forward with the Q rows rotated at their global positions as they are loaded (k arrives
    rotated); merge: fold into the running (o, lse) instead of writing them. k / v may have fewer
    heads than q (grouped-query)."""
    B, H, H_kv, Tq, Tk, D = _inputs(q, k, v)
    _expect("o", o, (B, H, Tq, D), _f32(), q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    if rope_table is None:
        raise ValueError("rope_table is required")
    _rope_check(rope_table, D, q)
    rp, rr = _rope_args(rope_table)
    row_end = Tq if row_end is None else row_end
    _check(load().cpattn_block_fwd_rotq(_tensor(q), _tensor(k), _tensor(v), _dtype(q), B, H, H_kv, Tq, Tk, D,
                                        _map(qmap), _map(kmap), int(causal), float(scale), rp, rr, row_begin, row_end,
                                        int(merge), _tensor(o), _tensor(lse, 3), _stream(stream)))


def cpattn_block_bwd_gqa(q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc, qmap, kmap, causal: bool = True,
                         scale: float = 0.0, accumulate: bool = True, stream=None):
    """Grouped-query block backward: dk_acc / dv_acc per KV head, summed over each group."""
    B, H, H_kv, Tq, Tk, D = _inputs(q, k, v, None)
    _expect("dout", dout, (B, H, Tq, D), q.dtype, q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    _expect("delta", delta, (B, H, Tq), _f32(), q)
    _expect("dq_acc", dq_acc, (B, H, Tq, D), _f32(), q)
    _expect("dk_acc", dk_acc, (B, H_kv, Tk, D), _f32(), q)
    _expect("dv_acc", dv_acc, (B, H_kv, Tk, D), _f32(), q)
    _check(load().cpattn_block_bwd_gqa(_tensor(q), _tensor(k), _tensor(v), _tensor(dout), _dtype(q), _tensor(lse, 3),
                                       _tensor(delta, 3), _tensor(dq_acc), _tensor(dk_acc), _tensor(dv_acc), B, H,
                                       H_kv, Tq, Tk, D, _map(qmap), _map(kmap), int(causal), float(scale),
                                       int(accumulate), _stream(stream)))


def cpattn_block_bwd_staged_workspace_bytes(B: int, H: int, Tq: int, Tk: int, D: int) -> int:
    return int(load().cpattn_block_bwd_staged_workspace_bytes(B, H, Tq, Tk, D))


def cpattn_block_bwd_staged(q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc, qmap, kmap, workspace,
                            causal: bool = True, scale: float = 0.0, accumulate: bool = True, stream=None):
    """Block backward with dS staged in ``workspace`` (a device tensor of at least
    cpattn_block_bwd_staged_workspace_bytes bytes; None where that is 0): dQ reuses the dK/dV
    kernel's dS. k / v may have fewer heads than q (grouped-query)."""
    B, H, H_kv, Tq, Tk, D = _inputs(q, k, v, None)
    _expect("dout", dout, (B, H, Tq, D), q.dtype, q)
    _expect("lse", lse, (B, H, Tq), _f32(), q)
    _expect("delta", delta, (B, H, Tq), _f32(), q)
    _expect("dq_acc", dq_acc, (B, H, Tq, D), _f32(), q)
    _expect("dk_acc", dk_acc, (B, H_kv, Tk, D), _f32(), q)
    _expect("dv_acc", dv_acc, (B, H_kv, Tk, D), _f32(), q)
    if workspace is not None and workspace.device != q.device:
        raise ValueError(f"workspace: on {workspace.device}, expected {q.device}")
    ws = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().cpattn_block_bwd_staged(_tensor(q), _tensor(k), _tensor(v), _tensor(dout), _dtype(q),
                                          _tensor(lse, 3), _tensor(delta, 3), _tensor(dq_acc), _tensor(dk_acc),
                                          _tensor(dv_acc), B, H, H_kv, Tq, Tk, D, _map(qmap), _map(kmap), int(causal),
                                          float(scale), int(accumulate), ws, wsb, _stream(stream)))
