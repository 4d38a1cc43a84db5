"""CPU oracle for the Ulysses attention path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 host implementation (oracle.c) of the
three steps of the path, loaded through ctypes:

* ``seq_to_head`` / ``head_to_seq``: the sequence-shard <-> head-shard layout
  change of "Sequence Parallelism II: DeepSpeed Ulysses and All-to-All
  Attention" (sections 1-3) and "Comparing Ulysses and Megatron Sequence
  Parallelism" (section "DeepSpeed Attention"), as raw byte copies.
* ``attention``: softmax(Q K^T / sqrt(D)) V per head in fp64, two passes per
  row (the attention skeleton in the second page's Introduction).
* ``seq_to_pieces`` / ``pieces_to_seq``: the same two exchanges written as
  the collective (each rank cuts its tensor into P pieces, piece j goes to
  rank j, which keeps one piece from every rank in rank order; first page,
  section 3), with the pieces left as the exchange delivers them: the
  receive buffer of the first exchange before any unpack, the send buffer of
  the second.
* ``send_bytes``: per-rank bytes one exchange sends to other ranks (first
  page section 4; second page section "DeepSpeed Attention costs").
* ``attention_backward``: the row log-sum-exp and dQ, dK, dV of ``attention``
  in fp64, the derivative of its definition (the backward pass of the first
  page's section 6 runs between the reversed layout changes).
* ``attention_chunk`` / ``softmax_merge`` / ``attention_chunk_backward``
  (numpy, ``chunk.py``): attention of a query block over one key/value chunk
  at given global positions, the merge of two partial results over disjoint
  key sets (the circulating key/value blocks of Ring Attention, first page
  section 8), and the gradient contributions of one such visit.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library never does, and shares no code with it.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build
from .chunk import attention_chunk, attention_chunk_backward, softmax_merge  # noqa: F401

BF16, F32, F64 = 0, 1, 2
_ERRORS = {1: "invalid argument", 2: "not divisible", 3: "out of memory"}
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        for name in ("oracle_seq_to_head", "oracle_head_to_seq", "oracle_seq_to_pieces",
                     "oracle_pieces_to_seq"):
            f = getattr(lib, name)
            f.argtypes = [vp, vp, i64, i64, i64, i64, i32, i32]
            f.restype = ctypes.c_int
        lib.oracle_send_bytes.argtypes = [i64, i64, i64, i64, i32, i32, i32]
        lib.oracle_send_bytes.restype = i64
        lib.oracle_attention.argtypes = [vp, vp, vp, i32, vp, i64, i64, i64, i64,
                                         i64, i32, vp, i64, i32]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention_backward.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, i64, i64,
                                                  i64, i64, i64, i32, i32, i32]
        lib.oracle_attention_backward.restype = ctypes.c_int
        lib.oracle_attention_backward_sampled.argtypes = [vp, vp, vp, vp, i32, vp, i64, vp, i64, vp,
                                                          vp, vp, i64, i64, i64, i64, i64, i32, i32,
                                                          i32]
        lib.oracle_attention_backward_sampled.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [vp, vp, i64]
        lib.oracle_round_bf16.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def seq_to_head(seq: np.ndarray, P: int) -> np.ndarray:
    """SEQ[P][B][S/P][H][D] -> HEAD[P][B][S][H/P][D] (any dtype, copied bitwise)."""
    Pp, B, Sp, H, D = seq.shape
    assert Pp == P
    seq = np.ascontiguousarray(seq)
    if H % P:
        raise ValueError("oracle: not divisible")
    out = np.empty((P, B, Sp * P, H // P, D), dtype=seq.dtype)
    _check(_load().oracle_seq_to_head(_ptr(seq), _ptr(out), B, Sp * P, H, D, P,
                                      seq.dtype.itemsize))
    return out


def head_to_seq(head: np.ndarray, P: int) -> np.ndarray:
    """HEAD[P][B][S][H/P][D] -> SEQ[P][B][S/P][H][D] (any dtype, copied bitwise)."""
    Pp, B, S, hp, D = head.shape
    assert Pp == P
    head = np.ascontiguousarray(head)
    if S % P:
        raise ValueError("oracle: not divisible")
    out = np.empty((P, B, S // P, hp * P, D), dtype=head.dtype)
    _check(_load().oracle_head_to_seq(_ptr(head), _ptr(out), B, S, hp * P, D, P,
                                      head.dtype.itemsize))
    return out


def seq_to_pieces(seq: np.ndarray, P: int) -> np.ndarray:
    """SEQ[P][B][S/P][H][D] -> PIECES[P][P][B][S/P][H/P][D]: the first exchange
    without the unpack (rank j's pieces from ranks 0..P-1 in order), bitwise."""
    Pp, B, Sp, H, D = seq.shape
    assert Pp == P
    seq = np.ascontiguousarray(seq)
    if H % P:
        raise ValueError("oracle: not divisible")
    out = np.empty((P, P, B, Sp, H // P, D), dtype=seq.dtype)
    _check(_load().oracle_seq_to_pieces(_ptr(seq), _ptr(out), B, Sp * P, H, D, P,
                                        seq.dtype.itemsize))
    return out


def pieces_to_seq(pieces: np.ndarray, P: int) -> np.ndarray:
    """PIECES[P][P][B][S/P][H/P][D] (each rank's output cut into pieces by
    destination rank) -> SEQ[P][B][S/P][H][D]: the second exchange, bitwise."""
    Pp, Pq, B, Sp, hp, D = pieces.shape
    assert Pp == P and Pq == P
    pieces = np.ascontiguousarray(pieces)
    out = np.empty((P, B, Sp, hp * P, D), dtype=pieces.dtype)
    _check(_load().oracle_pieces_to_seq(_ptr(pieces), _ptr(out), B, Sp * P, hp * P, D, P,
                                        pieces.dtype.itemsize))
    return out


def send_bytes(B, S, H, D, P, elem_bytes, rank=0) -> int:
    n = _load().oracle_send_bytes(B, S, H, D, P, elem_bytes, rank)
    if n < 0:
        raise ValueError("oracle: bad layout")
    return int(n)


def _dtype_code(a: np.ndarray, bf16: bool) -> int:
    if bf16:
        assert a.dtype == np.uint16, "bf16 inputs are passed as their uint16 bit patterns"
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported oracle dtype {a.dtype}")


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
              bf16: bool = False, rows=None, threads: int = 0) -> np.ndarray:
    """softmax(Q K^T / sqrt(D)) V for one rank, in fp64.

    q: [B][S][Hq][D]; k, v: [B][S][Hkv][D]; bf16 inputs as uint16 bit arrays.
    rows: optional token indices; then the result is [B][len(rows)][Hq][D].
    """
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, S, Hkv, D) and v.shape == k.shape
    assert q.dtype == k.dtype == v.dtype
    code = _dtype_code(q, bf16)
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    if rows is None:
        out = np.empty((B, S, Hq, D), dtype=np.float64)
        rp, nr = None, 0
    else:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((B, rows_a.size, Hq, D), dtype=np.float64)
        rp, nr = _ptr(rows_a), rows_a.size
    _check(_load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), code, _ptr(out), B, S,
                                    Hq, Hkv, D, int(bool(causal)), rp, nr, threads))
    return out


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                       causal: bool, bf16: bool = False, round_o: bool = False, threads: int = 0):
    """Gradients of attention(q, k, v) for output gradient dout, in fp64.

    Returns (dq [B][S][Hq][D], dk [B][S][Hkv][D], dv [B][S][Hkv][D],
    lse [B][Hq][S]) with lse the natural log of each row's sum of exp(scores).
    round_o: take delta = sum(dout * o) from o rounded to bfloat16, as a bf16
    forward output handed to the gradient step is.
    """
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, S, Hkv, D) and v.shape == k.shape and dout.shape == q.shape
    assert q.dtype == k.dtype == v.dtype == dout.dtype
    code = _dtype_code(q, bf16)
    q, k, v, dout = (np.ascontiguousarray(x) for x in (q, k, v, dout))
    dq = np.empty((B, S, Hq, D), dtype=np.float64)
    dk = np.empty((B, S, Hkv, D), dtype=np.float64)
    dv = np.empty((B, S, Hkv, D), dtype=np.float64)
    lse = np.empty((B, Hq, S), dtype=np.float64)
    _check(_load().oracle_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), code,
                                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(lse), B, S, Hq,
                                             Hkv, D, int(bool(causal)), int(bool(round_o)),
                                             threads))
    return dq, dk, dv, lse


def round_bf16(x) -> np.ndarray:
    """Each value of x (fp64) rounded to the nearest bfloat16 value, ties to even,
    returned as fp64 (the rounding ``attention_backward`` applies with round_o)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty_like(x)
    _check(_load().oracle_round_bf16(_ptr(x), _ptr(out), x.size))
    return out


def attention_backward_sampled(q, k, v, dout, causal: bool, rows, keys, bf16: bool = False,
                               round_o: bool = False, threads: int = 0):
    """dq at the given rows ([B][len(rows)][Hq][D]) and dk, dv at the given keys
    ([B][len(keys)][Hkv][D]), in fp64, as attention_backward computes them."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, S, Hkv, D) and v.shape == k.shape and dout.shape == q.shape
    code = _dtype_code(q, bf16)
    q, k, v, dout = (np.ascontiguousarray(x) for x in (q, k, v, dout))
    rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    keys_a = np.ascontiguousarray(np.asarray(keys, dtype=np.int64))
    dq = np.empty((B, rows_a.size, Hq, D), dtype=np.float64)
    dk = np.empty((B, keys_a.size, Hkv, D), dtype=np.float64)
    dv = np.empty((B, keys_a.size, Hkv, D), dtype=np.float64)
    _check(_load().oracle_attention_backward_sampled(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), code, _ptr(rows_a), rows_a.size, _ptr(keys_a),
        keys_a.size, _ptr(dq), _ptr(dk), _ptr(dv), B, S, Hq, Hkv, D, int(bool(causal)),
        int(bool(round_o)), threads))
    return dq, dk, dv
