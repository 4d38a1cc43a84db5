"""Thin ctypes binding of libulysses.so (C ABI in include/ulysses.h).

Argument marshalling only: tensor shapes become the sizes of the C calls,
``tensor.data_ptr()`` the device pointers and the current torch stream the
HIP stream.  Every step of the path runs in the library's HIP kernels; there
is no fallback.  If the library is missing the import raises.

Layouts (P virtual ranks stacked rank-major, head_dim innermost):
  SEQ  [P, B, S/P, n_heads, head_dim]     HEAD [P, B, S, n_heads/P, head_dim]
  attention (one rank): q, o [B, S, n_q_heads, D];  k, v [B, S, n_kv_heads, D]
  log-sum-exp and its gradient scratch: [B, n_q_heads, S] float32
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libulysses.so")

ULY_OK, ULY_ERR_INVALID_ARGUMENT, ULY_ERR_NOT_DIVISIBLE, ULY_ERR_UNSUPPORTED, ULY_ERR_HIP = range(5)
ULY_DTYPE_BF16, ULY_DTYPE_FP32 = 0, 1
EXPORTS = ("ulysses_seq_to_head", "ulysses_seq_to_head_qkv", "ulysses_head_to_seq",
           "ulysses_attention_local",
           "ulysses_attention_local_lse", "ulysses_attention_local_backward",
           "ulysses_attention_local_split_workspace", "ulysses_attention_local_split",
           "ulysses_attention_local_backward_noalloc",
           "ulysses_attention_local_backward_split_workspace", "ulysses_attention_local_backward_split",
           "ulysses_seq_to_pieces", "ulysses_seq_to_pieces_qkv", "ulysses_pieces_to_seq",
           "ulysses_attention_local_pieces", "ulysses_attention_local_backward_pieces",
           "ulysses_attention_chunk", "ulysses_attention_chunk_accumulate", "ulysses_attention_merge",
           "ulysses_attention_chunk_backward",
           "ulysses_status_string", "ulysses_last_error")


class UlyssesError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libulysses.so not built at {path}; run python sequence_long_context_amd/build.py")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    for name in ("ulysses_seq_to_head", "ulysses_head_to_seq"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, i64, i64, i64, i64, i32, ctypes.c_int, vp]
        f.restype = ctypes.c_int
    lib.ulysses_seq_to_head_qkv.argtypes = [vp] * 6 + [i64] * 5 + [i32, ctypes.c_int, vp]
    lib.ulysses_seq_to_head_qkv.restype = ctypes.c_int
    lib.ulysses_attention_local.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i32,
                                            ctypes.c_int, vp]
    lib.ulysses_attention_local.restype = ctypes.c_int
    lib.ulysses_attention_local_lse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32,
                                                ctypes.c_int, vp]
    lib.ulysses_attention_local_lse.restype = ctypes.c_int
    lib.ulysses_attention_local_split_workspace.argtypes = [i64] * 4 + [i32, ctypes.c_int,
                                                                 ctypes.POINTER(ctypes.c_uint64)]
    lib.ulysses_attention_local_split_workspace.restype = ctypes.c_int
    lib.ulysses_attention_local_split.argtypes = ([vp] * 5 + [i64] * 5 + [i32, ctypes.c_int, vp,
                                                  ctypes.c_uint64, vp])
    lib.ulysses_attention_local_split.restype = ctypes.c_int
    lib.ulysses_attention_local_backward.argtypes = [vp] * 10 + [i64] * 5 + [i32, ctypes.c_int, vp]
    lib.ulysses_attention_local_backward.restype = ctypes.c_int
    lib.ulysses_attention_local_backward_split_workspace.argtypes = [i64] * 5 + [i32, ctypes.c_int,
                                                                        ctypes.POINTER(ctypes.c_uint64)]
    lib.ulysses_attention_local_backward_split.argtypes = ([vp] * 10 + [i64] * 5 +
                                                           [i32, ctypes.c_int, vp, ctypes.c_uint64, vp])
    lib.ulysses_attention_local_backward_noalloc.argtypes = [vp] * 9 + [i64] * 5 + [i32, ctypes.c_int, vp]
    lib.ulysses_attention_local_backward_noalloc.restype = ctypes.c_int
    for name in ("ulysses_seq_to_pieces", "ulysses_pieces_to_seq"):
        getattr(lib, name).argtypes = [vp, vp, i64, i64, i64, i64, i32, ctypes.c_int, vp]
        getattr(lib, name).restype = ctypes.c_int
    lib.ulysses_seq_to_pieces_qkv.argtypes = [vp] * 6 + [i64] * 5 + [i32, ctypes.c_int, vp]
    lib.ulysses_seq_to_pieces_qkv.restype = ctypes.c_int
    lib.ulysses_attention_local_pieces.argtypes = [vp] * 5 + [i64] * 5 + [i32, i32, ctypes.c_int, vp]
    lib.ulysses_attention_local_pieces.restype = ctypes.c_int
    lib.ulysses_attention_local_backward_pieces.argtypes = [vp] * 10 + [i64] * 5 + [i32, i32,
                                                                                ctypes.c_int, vp]
    lib.ulysses_attention_local_backward_pieces.restype = ctypes.c_int
    lib.ulysses_attention_chunk.argtypes = [vp] * 5 + [i64] * 8 + [i32, ctypes.c_int, vp]
    lib.ulysses_attention_chunk.restype = ctypes.c_int
    lib.ulysses_attention_chunk_accumulate.argtypes = [vp] * 5 + [i64] * 8 + [i32, ctypes.c_int, vp]
    lib.ulysses_attention_chunk_accumulate.restype = ctypes.c_int
    lib.ulysses_attention_chunk_backward.argtypes = [vp] * 10 + [i64] * 8 + [i32, i32, i32, ctypes.c_int, vp]
    lib.ulysses_attention_chunk_backward.restype = ctypes.c_int
    lib.ulysses_attention_merge.argtypes = [vp] * 6 + [i64] * 4 + [ctypes.c_int, vp]
    lib.ulysses_attention_merge.restype = ctypes.c_int
    lib.ulysses_status_string.argtypes = [ctypes.c_int]
    lib.ulysses_status_string.restype = ctypes.c_char_p
    lib.ulysses_last_error.argtypes = []
    lib.ulysses_last_error.restype = ctypes.c_char_p
    return lib


_lib = load_library()


def _check(status: int) -> None:
    if status != ULY_OK:
        raise UlyssesError(status, _lib.ulysses_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _elem_code(t: torch.Tensor) -> int:
    size = t.element_size()
    if size == 2:
        return ULY_DTYPE_BF16
    if size == 4:
        return ULY_DTYPE_FP32
    raise TypeError(f"layout change moves 2- or 4-byte elements, got {t.dtype}")


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def ulysses_seq_to_head(seq: torch.Tensor, head: torch.Tensor, P: int) -> torch.Tensor:
    """SEQ [P,B,S/P,H,D] -> HEAD [P,B,S,H/P,D] (bitwise copy), enqueued on the current stream."""
    _dev(seq, "seq")
    _dev(head, "head")
    Pp, B, Sp, H, D = seq.shape
    if Pp != P or head.dtype != seq.dtype or head.shape != (P, B, Sp * P, H // P, D):
        raise ValueError(f"shape mismatch: seq {tuple(seq.shape)} head {tuple(head.shape)} P={P}")
    _check(_lib.ulysses_seq_to_head(seq.data_ptr(), head.data_ptr(), B, Sp * P, H, D, P,
                                    _elem_code(seq), _stream(seq)))
    return head


def ulysses_seq_to_head_qkv(q_seq, k_seq, v_seq, q_head, k_head, v_head, P: int):
    """seq->head of Q, K and V in one launch (shapes as for ulysses_seq_to_head; K and V may
    have fewer heads than Q)."""
    for t, n in ((q_seq, "q_seq"), (k_seq, "k_seq"), (v_seq, "v_seq"), (q_head, "q_head"),
                 (k_head, "k_head"), (v_head, "v_head")):
        _dev(t, n)
    Pp, B, Sp, Hq, D = q_seq.shape
    Hkv = k_seq.shape[3]
    for seq, head, H in ((q_seq, q_head, Hq), (k_seq, k_head, Hkv), (v_seq, v_head, Hkv)):
        if (seq.shape != (P, B, Sp, H, D) or head.shape != (P, B, Sp * P, H // P, D)
                or seq.dtype != q_seq.dtype or head.dtype != q_seq.dtype):
            raise ValueError(f"shape mismatch: seq {tuple(seq.shape)} head {tuple(head.shape)} P={P}")
    _check(_lib.ulysses_seq_to_head_qkv(q_seq.data_ptr(), k_seq.data_ptr(), v_seq.data_ptr(),
                                        q_head.data_ptr(), k_head.data_ptr(), v_head.data_ptr(),
                                        B, Sp * P, Hq, Hkv, D, P, _elem_code(q_seq), _stream(q_seq)))
    return q_head, k_head, v_head


def ulysses_head_to_seq(head: torch.Tensor, seq: torch.Tensor, P: int) -> torch.Tensor:
    """HEAD [P,B,S,H/P,D] -> SEQ [P,B,S/P,H,D] (bitwise copy), enqueued on the current stream."""
    _dev(head, "head")
    _dev(seq, "seq")
    Pp, B, S, hp, D = head.shape
    if Pp != P or head.dtype != seq.dtype or seq.shape != (P, B, S // P, hp * P, D):
        raise ValueError(f"shape mismatch: head {tuple(head.shape)} seq {tuple(seq.shape)} P={P}")
    _check(_lib.ulysses_head_to_seq(head.data_ptr(), seq.data_ptr(), B, S, hp * P, D, P,
                                    _elem_code(head), _stream(head)))
    return seq


def ulysses_seq_to_pieces(seq: torch.Tensor, pieces: torch.Tensor, P: int) -> torch.Tensor:
    """SEQ [P,B,S/P,H,D] -> PIECES [P,P,B,S/P,H/P,D]: the first exchange with each rank's
    pieces left in source-rank order (no unpack), bitwise."""
    _dev(seq, "seq")
    _dev(pieces, "pieces")
    Pp, B, Sp, H, D = seq.shape
    if Pp != P or pieces.dtype != seq.dtype or pieces.shape != (P, P, B, Sp, H // P, D):
        raise ValueError(f"shape mismatch: seq {tuple(seq.shape)} pieces {tuple(pieces.shape)} P={P}")
    _check(_lib.ulysses_seq_to_pieces(seq.data_ptr(), pieces.data_ptr(), B, Sp * P, H, D, P,
                                      _elem_code(seq), _stream(seq)))
    return pieces


def ulysses_seq_to_pieces_qkv(q_seq, k_seq, v_seq, q_pieces, k_pieces, v_pieces, P: int):
    """ulysses_seq_to_pieces of Q, K and V in one launch (K and V may have fewer heads)."""
    for t, n in ((q_seq, "q_seq"), (k_seq, "k_seq"), (v_seq, "v_seq"), (q_pieces, "q_pieces"),
                 (k_pieces, "k_pieces"), (v_pieces, "v_pieces")):
        _dev(t, n)
    Pp, B, Sp, Hq, D = q_seq.shape
    Hkv = k_seq.shape[3]
    for seq, pc, H in ((q_seq, q_pieces, Hq), (k_seq, k_pieces, Hkv), (v_seq, v_pieces, Hkv)):
        if (seq.shape != (P, B, Sp, H, D) or pc.shape != (P, P, B, Sp, H // P, D)
                or seq.dtype != q_seq.dtype or pc.dtype != q_seq.dtype):
            raise ValueError(f"shape mismatch: seq {tuple(seq.shape)} pieces {tuple(pc.shape)} P={P}")
    _check(_lib.ulysses_seq_to_pieces_qkv(q_seq.data_ptr(), k_seq.data_ptr(), v_seq.data_ptr(),
                                          q_pieces.data_ptr(), k_pieces.data_ptr(),
                                          v_pieces.data_ptr(), B, Sp * P, Hq, Hkv, D, P,
                                          _elem_code(q_seq), _stream(q_seq)))
    return q_pieces, k_pieces, v_pieces


def ulysses_pieces_to_seq(pieces: torch.Tensor, seq: torch.Tensor, P: int) -> torch.Tensor:
    """PIECES [P,P,B,S/P,H/P,D] (each rank's output in send order) -> SEQ [P,B,S/P,H,D]."""
    _dev(pieces, "pieces")
    _dev(seq, "seq")
    Pp, Pq, B, Sp, hp, D = pieces.shape
    if Pp != P or Pq != P or seq.dtype != pieces.dtype or seq.shape != (P, B, Sp, hp * P, D):
        raise ValueError(f"shape mismatch: pieces {tuple(pieces.shape)} seq {tuple(seq.shape)} P={P}")
    _check(_lib.ulysses_pieces_to_seq(pieces.data_ptr(), seq.data_ptr(), B, Sp * P, hp * P, D, P,
                                      _elem_code(pieces), _stream(pieces)))
    return seq


def ulysses_attention_local_pieces(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                   o: torch.Tensor, causal: bool, lse=None) -> torch.Tensor:
    """ulysses_attention_local on one rank's pieces: q, o [P,B,S/P,Hq,D], k, v [P,B,S/P,Hkv,D]
    (piece i = the tokens of rank i); o is written in the same order; lse [B,Hq,S] if given."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _dev(t, n)
    P, B, Sp, Hq, D = q.shape
    Hkv = k.shape[3]
    if k.shape != (P, B, Sp, Hkv, D) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, o")
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise ValueError("q, k, v, o must share a dtype")
    code = _dtype_code(q)
    if lse is not None:
        _f32_rows(lse, "lse", B, Hq, P * Sp)
    _check(_lib.ulysses_attention_local_pieces(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
        None if lse is None else lse.data_ptr(), B, P * Sp, Hq, Hkv, D, P, int(bool(causal)), code,
        _stream(q)))
    return o


def ulysses_attention_local_backward_pieces(q, k, v, o, dout, lse, delta, dq, dk, dv, causal: bool):
    """ulysses_attention_local_backward on one rank's pieces: q, o, dout, dq [P,B,S/P,Hq,D],
    k, v, dk, dv [P,B,S/P,Hkv,D]; lse, delta [B,Hq,S] float32."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                 (dv, "dv")):
        _dev(t, n)
    P, B, Sp, Hq, D = q.shape
    Hkv = k.shape[3]
    for t, n, like in ((o, "o", q), (dout, "dout", q), (dq, "dq", q), (v, "v", k), (dk, "dk", k),
                       (dv, "dv", k)):
        if t.shape != like.shape or t.dtype != like.dtype:
            raise ValueError(f"{n} must match {tuple(like.shape)} {like.dtype}")
    if k.shape != (P, B, Sp, Hkv, D) or k.dtype != q.dtype:
        raise ValueError("shape mismatch between q and k")
    _f32_rows(lse, "lse", B, Hq, P * Sp)
    _f32_rows(delta, "delta", B, Hq, P * Sp)
    _check(_lib.ulysses_attention_local_backward_pieces(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, P * Sp, Hq, Hkv, D, P,
        int(bool(causal)), _dtype_code(q), _stream(q)))
    return dq, dk, dv


def _attn_args(q, k, v, o):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _dev(t, n)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, o")
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise ValueError("q, k, v, o must share a dtype")
    if q.dtype == torch.bfloat16:
        code = ULY_DTYPE_BF16
    elif q.dtype == torch.float32:
        code = ULY_DTYPE_FP32
    else:
        raise TypeError(f"attention supports bfloat16 and float32, got {q.dtype}")
    return B, S, Hq, Hkv, D, code


def _f32_rows(t: torch.Tensor, name: str, B: int, Hq: int, S: int) -> None:
    _dev(t, name)
    if t.dtype != torch.float32 or t.shape != (B, Hq, S):
        raise ValueError(f"{name} must be float32 [B, n_q_heads, S] = {(B, Hq, S)}, got "
                         f"{t.dtype} {tuple(t.shape)}")


def ulysses_attention_local(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                            causal: bool) -> torch.Tensor:
    """o = softmax(q k^T / sqrt(D)) v per head for one rank; q,o [B,S,Hq,D], k,v [B,S,Hkv,D]."""
    B, S, Hq, Hkv, D, code = _attn_args(q, k, v, o)
    _check(_lib.ulysses_attention_local(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        B, S, Hq, Hkv, D, int(bool(causal)), code, _stream(q)))
    return o


def ulysses_attention_local_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                o: torch.Tensor, lse: torch.Tensor, causal: bool) -> torch.Tensor:
    """As ulysses_attention_local, also writing lse [B,Hq,S] (natural log of each row's sum of exp)."""
    B, S, Hq, Hkv, D, code = _attn_args(q, k, v, o)
    _f32_rows(lse, "lse", B, Hq, S)
    _check(_lib.ulysses_attention_local_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                            lse.data_ptr(), B, S, Hq, Hkv, D, int(bool(causal)),
                                            code, _stream(q)))
    return o


def ulysses_attention_local_split_workspace(B: int, S: int, n_q_heads: int, causal: bool,
                                            head_dim: int = 128) -> int:
    """Bytes of workspace ulysses_attention_local_split needs on the current device (0: none)."""
    out = ctypes.c_uint64(0)
    _check(_lib.ulysses_attention_local_split_workspace(B, S, n_q_heads, head_dim,
                                                        int(bool(causal)), ULY_DTYPE_BF16,
                                                        ctypes.byref(out)))
    return int(out.value)


def ulysses_attention_local_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  o: torch.Tensor, causal: bool, workspace=None,
                                  lse=None) -> torch.Tensor:
    """ulysses_attention_local with each query block's keys split across workgroups and
    merged (few heads, medium lengths); workspace: a device tensor of at least
    ulysses_attention_local_split_workspace(...) bytes (None when that is 0); lse
    [B,Hq,S] float32 or None."""
    B, S, Hq, Hkv, D, code = _attn_args(q, k, v, o)
    if lse is not None:
        _f32_rows(lse, "lse", B, Hq, S)
    if workspace is not None:
        _dev(workspace, "workspace")
    _check(_lib.ulysses_attention_local_split(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
        None if lse is None else lse.data_ptr(), B, S, Hq, Hkv, D, int(bool(causal)), code,
        None if workspace is None else workspace.data_ptr(),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(q)))
    return o


def ulysses_attention_local_backward(q, k, v, o, dout, lse, delta, dq, dk, dv, causal: bool):
    """dq, dk, dv of the local attention for output gradient dout (bf16, D = 128).

    lse from ulysses_attention_local_lse; delta [B,Hq,S] float32 is scratch."""
    B, S, Hq, Hkv, D, code = _attn_args(q, k, v, o)
    for t, n, like in ((dout, "dout", q), (dq, "dq", q), (dk, "dk", k), (dv, "dv", k)):
        _dev(t, n)
        if t.shape != like.shape or t.dtype != like.dtype:
            raise ValueError(f"{n} must match {tuple(like.shape)} {like.dtype}")
    _f32_rows(lse, "lse", B, Hq, S)
    _f32_rows(delta, "delta", B, Hq, S)
    _check(_lib.ulysses_attention_local_backward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, S, Hq, Hkv, D,
        int(bool(causal)), code, _stream(q)))
    return dq, dk, dv


def ulysses_attention_local_backward_split_workspace(B: int, S: int, n_q_heads: int, n_kv_heads: int,
                                                     causal: bool, head_dim: int = 128) -> int:
    """Bytes of workspace ulysses_attention_local_backward_split needs on the current device (0: none)."""
    out = ctypes.c_uint64(0)
    _check(_lib.ulysses_attention_local_backward_split_workspace(
        B, S, n_q_heads, n_kv_heads, head_dim, int(bool(causal)), ULY_DTYPE_BF16, ctypes.byref(out)))
    return int(out.value)


def ulysses_attention_local_backward_split(q, k, v, o, dout, lse, delta, dq, dk, dv, causal: bool,
                                           workspace=None):
    """As ulysses_attention_local_backward, with the longest dK/dV blocks on several workgroups:
    workspace a device tensor of at least ulysses_attention_local_backward_split_workspace bytes
    (None when that is 0)."""
    B, S, Hq, Hkv, D, code = _attn_args(q, k, v, o)
    for t, n, like in ((dout, "dout", q), (dq, "dq", q), (dk, "dk", k), (dv, "dv", k)):
        _dev(t, n)
        if t.shape != like.shape or t.dtype != like.dtype:
            raise ValueError(f"{n} must match {tuple(like.shape)} {like.dtype}")
    _f32_rows(lse, "lse", B, Hq, S)
    _f32_rows(delta, "delta", B, Hq, S)
    if workspace is not None:
        _dev(workspace, "workspace")
    wp = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.ulysses_attention_local_backward_split(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, S, Hq, Hkv, D,
        int(bool(causal)), code, wp, wb, _stream(q)))
    return dq, dk, dv


def ulysses_attention_local_backward_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal: bool):
    """As ulysses_attention_local_backward, with delta kept in the library's per-GPU
    scratch (for callers that cannot allocate): B * n_q_heads * S <= 2^20."""
    B, S, Hq, Hkv, D, code = _attn_args(q, k, v, o)
    for t, n, like in ((dout, "dout", q), (dq, "dq", q), (dk, "dk", k), (dv, "dv", k)):
        _dev(t, n)
        if t.shape != like.shape or t.dtype != like.dtype:
            raise ValueError(f"{n} must match {tuple(like.shape)} {like.dtype}")
    _f32_rows(lse, "lse", B, Hq, S)
    _check(_lib.ulysses_attention_local_backward_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, S, Hq, Hkv, D, int(bool(causal)), code,
        _stream(q)))
    return dq, dk, dv


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ULY_DTYPE_BF16
    if t.dtype == torch.float32:
        return ULY_DTYPE_FP32
    raise TypeError(f"attention supports bfloat16 and float32, got {t.dtype}")


def ulysses_attention_chunk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                            lse: torch.Tensor, causal: bool, q_pos0: int = 0,
                            k_pos0: int = 0) -> torch.Tensor:
    """Attention of q [B,Sq,Hq,D] over one key/value chunk k, v [B,Skv,Hkv,D] at global
    positions q_pos0 + i and k_pos0 + j; writes o [B,Sq,Hq,D] and lse [B,Hq,Sq]."""
    return _chunk(_lib.ulysses_attention_chunk, q, k, v, o, lse, causal, q_pos0, k_pos0)


def _chunk(fn, q, k, v, o, lse, causal, q_pos0, k_pos0):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _dev(t, n)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Skv, Hkv, D) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, o")
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise ValueError("q, k, v, o must share a dtype")
    _f32_rows(lse, "lse", B, Hq, Sq)
    _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Sq, Skv,
              Hq, Hkv, D, int(q_pos0), int(k_pos0), int(bool(causal)), _dtype_code(q), _stream(q)))
    return o


def ulysses_attention_chunk_accumulate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                       o: torch.Tensor, lse: torch.Tensor, causal: bool,
                                       q_pos0: int = 0, k_pos0: int = 0) -> torch.Tensor:
    """One key/value chunk merged into the running result (o [B,Sq,Hq,D], lse [B,Hq,Sq], read
    and written) in the same launch; arguments as for ulysses_attention_chunk."""
    return _chunk(_lib.ulysses_attention_chunk_accumulate, q, k, v, o, lse, causal, q_pos0, k_pos0)


def ulysses_attention_merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor,
                            lse_b: torch.Tensor, o: torch.Tensor, lse: torch.Tensor) -> torch.Tensor:
    """Combine two partial results over disjoint key sets; o [B,S,H,D], lse [B,H,S].
    o may be o_a or o_b and lse may be lse_a or lse_b (in place)."""
    for t, n in ((o_a, "o_a"), (o_b, "o_b"), (o, "o")):
        _dev(t, n)
        if t.shape != o_a.shape or t.dtype != o_a.dtype:
            raise ValueError(f"{n} must match o_a {tuple(o_a.shape)} {o_a.dtype}")
    B, S, H, D = o_a.shape
    for t, n in ((lse_a, "lse_a"), (lse_b, "lse_b"), (lse, "lse")):
        _f32_rows(t, n, B, H, S)
    _check(_lib.ulysses_attention_merge(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(),
                                        lse_b.data_ptr(), o.data_ptr(), lse.data_ptr(), B, S, H, D,
                                        _dtype_code(o_a), _stream(o_a)))
    return o


def ulysses_attention_chunk_backward(q, k, v, o, dout, lse, delta, dq, dk, dv, causal: bool,
                                     q_pos0: int = 0, k_pos0: int = 0, accumulate_dq: bool = False,
                                     accumulate_dkv: bool = False):
    """Gradient contributions of one key/value chunk visit (bf16, D = 128): q, o, dout, dq
    [B,Sq,Hq,D]; k, v, dk, dv [B,Skv,Hkv,D]; o and lse [B,Hq,Sq] the query block's merged
    forward result; delta [B,Hq,Sq] float32 scratch.  accumulate_dq adds to dq,
    accumulate_dkv to dk and dv (otherwise they are written)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                 (dv, "dv")):
        _dev(t, n)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    for t, n, like in ((o, "o", q), (dout, "dout", q), (dq, "dq", q), (v, "v", k), (dk, "dk", k),
                       (dv, "dv", k)):
        if t.shape != like.shape or t.dtype != like.dtype:
            raise ValueError(f"{n} must match {tuple(like.shape)} {like.dtype}")
    if k.shape != (B, Skv, Hkv, D):
        raise ValueError("shape mismatch between q and k")
    _f32_rows(lse, "lse", B, Hq, Sq)
    _f32_rows(delta, "delta", B, Hq, Sq)
    _check(_lib.ulysses_attention_chunk_backward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Sq, Skv, Hq, Hkv, D,
        int(q_pos0), int(k_pos0), int(bool(causal)), int(bool(accumulate_dq)),
        int(bool(accumulate_dkv)), _dtype_code(q), _stream(q)))
    return dq, dk, dv


def status_string(status: int) -> str:
    return _lib.ulysses_status_string(status).decode()


def library() -> ctypes.CDLL:
    return _lib
