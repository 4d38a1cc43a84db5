"""Attention over one key/value chunk, its gradients, and the merge of two
partial results -- TEST INFRASTRUCTURE ONLY (plain fp64 numpy).

"Sequence Parallelism II: DeepSpeed Ulysses and All-to-All Attention",
section 8, names the step past the head-count bound: keep the local query
block and let key/value blocks circulate (Ring Attention).  Each visit of a
key/value block yields the softmax restricted to that block's keys; the
pages do not spell out how the visits combine.  The plain reading: the
softmax over a union of disjoint key sets equals the combination of the
per-set results weighted by each set's share of the total exp-sum,

    lse = log(exp(lse_a) + exp(lse_b)),
    o   = exp(lse_a - lse) * o_a + exp(lse_b - lse) * o_b,

with o_x the normalised output over key set x and lse_x the natural log of
its exp-sum.  A row with no visible key in a chunk has o = 0 and
lse = -inf, the identity of the merge.

Gradients of a visit: the softmax weight of a visible (row, key) pair over
every visit is exp(s - lse) with lse the log of the total exp-sum, so the
derivative of the whole attention is a sum of per-visit terms, each written
with the merged output o and lse (the derivative of softmax(S) V, section 6
of the same page: the backward pass between the reversed exchanges).

Positions: query row i of the chunk call sits at global position
q_pos0 + i, key j at k_pos0 + j; with causal, key j is visible to row i iff
k_pos0 + j <= q_pos0 + i (the triangular mask of section 8 in global token
order).
"""
import numpy as np


def _decode(a: np.ndarray, bf16: bool) -> np.ndarray:
    if bf16:
        assert a.dtype == np.uint16, "bf16 inputs are passed as their uint16 bit patterns"
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def attention_chunk(q, k, v, causal: bool, q_pos0: int = 0, k_pos0: int = 0, bf16: bool = False):
    """Softmax attention of q over the keys of one chunk, in fp64.

    q: [B][Sq][Hq][D]; k, v: [B][Skv][Hkv][D] (Hq a multiple of Hkv; query head
    c reads kv head c // (Hq // Hkv)).  Returns (o [B][Sq][Hq][D],
    lse [B][Hq][Sq]); rows with no visible key get o = 0 and lse = -inf.
    """
    qd, kd, vd = (_decode(x, bf16) for x in (q, k, v))
    B, Sq, Hq, D = qd.shape
    Skv, Hkv = kd.shape[1], kd.shape[2]
    assert kd.shape == (B, Skv, Hkv, D) and vd.shape == kd.shape and Hq % Hkv == 0
    group = Hq // Hkv
    o = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Hq, Sq), -np.inf)
    if Sq == 0 or Skv == 0:
        return o, lse
    qpos = q_pos0 + np.arange(Sq)
    kpos = k_pos0 + np.arange(Skv)
    visible = (kpos[None, :] <= qpos[:, None]) if causal else np.ones((Sq, Skv), dtype=bool)
    any_visible = visible.any(axis=1)
    for b in range(B):
        for c in range(Hq):
            g = c // group
            s = (qd[b, :, c, :] @ kd[b, :, g, :].T) / np.sqrt(D)
            s = np.where(visible, s, -np.inf)
            m = np.where(any_visible, s.max(axis=1), 0.0)
            p = np.where(visible, np.exp(s - m[:, None]), 0.0)
            l = p.sum(axis=1)
            rows = any_visible
            o[b, rows, c, :] = (p[rows] @ vd[b, :, g, :]) / l[rows, None]
            lse[b, c, rows] = m[rows] + np.log(l[rows])
    return o, lse


def softmax_merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial results over disjoint key sets (fp64).

    o_x: [B][S][H][D]; lse_x: [B][H][S].  Returns (o, lse) of the union.
    """
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    assert o_a.shape == o_b.shape and lse_a.shape == lse_b.shape
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    ea = np.exp(lse_a - m_safe)  # exp(-inf) = 0 for an empty side
    eb = np.exp(lse_b - m_safe)
    tot = ea + eb
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    wa = np.where(empty, 0.0, ea / np.where(empty, 1.0, tot))
    wb = np.where(empty, 0.0, eb / np.where(empty, 1.0, tot))
    # weights are [B][H][S]; outputs [B][S][H][D]
    wa_t = np.transpose(wa, (0, 2, 1))[..., None]
    wb_t = np.transpose(wb, (0, 2, 1))[..., None]
    return wa_t * o_a + wb_t * o_b, lse


def attention_chunk_backward(q, k, v, dout, o, lse, causal: bool, q_pos0: int = 0,
                             k_pos0: int = 0, bf16: bool = False):
    """Gradient contributions of one key/value chunk visit, in fp64.

    q, dout, o: [B][Sq][Hq][D]; k, v: [B][Skv][Hkv][D]; lse: [B][Hq][Sq] (the
    natural log of each row's exp-sum over every key of every visit; o the
    merged output over every key).  bf16 applies to q, k, v, dout and o (uint16
    bit patterns); lse is taken as given.  For a visible pair (i, j):
        p_ij  = exp(s_ij - lse_i),  s_ij = q_i . k_j / sqrt(D)
        delta_i = sum_d dout_id o_id
        ds_ij = p_ij (dout_i . v_j - delta_i)
        dq_i += ds_ij k_j / sqrt(D);  dk_j += ds_ij q_i / sqrt(D);  dv_j += p_ij dout_i
    (dk, dv summed over the query heads that share a key/value head).  Returns
    (dq [B][Sq][Hq][D], dk [B][Skv][Hkv][D], dv [B][Skv][Hkv][D]); rows that see
    no key of the chunk contribute nothing.
    """
    qd, kd, vd, gd, od = (_decode(x, bf16) for x in (q, k, v, dout, o))
    lse = np.asarray(lse, np.float64)
    B, Sq, Hq, D = qd.shape
    Skv, Hkv = kd.shape[1], kd.shape[2]
    assert kd.shape == (B, Skv, Hkv, D) and vd.shape == kd.shape and Hq % Hkv == 0
    assert gd.shape == qd.shape and od.shape == qd.shape and lse.shape == (B, Hq, Sq)
    group = Hq // Hkv
    dq = np.zeros((B, Sq, Hq, D))
    dk = np.zeros((B, Skv, Hkv, D))
    dv = np.zeros((B, Skv, Hkv, D))
    if Sq == 0 or Skv == 0:
        return dq, dk, dv
    qpos = q_pos0 + np.arange(Sq)
    kpos = k_pos0 + np.arange(Skv)
    visible = (kpos[None, :] <= qpos[:, None]) if causal else np.ones((Sq, Skv), dtype=bool)
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        for c in range(Hq):
            g = c // group
            s = (qd[b, :, c, :] @ kd[b, :, g, :].T) * scale
            p = np.exp(np.where(visible, s - lse[b, c][:, None], -np.inf))
            delta = (gd[b, :, c, :] * od[b, :, c, :]).sum(axis=1)
            dp = gd[b, :, c, :] @ vd[b, :, g, :].T
            ds = p * (dp - delta[:, None])
            dq[b, :, c, :] = (ds @ kd[b, :, g, :]) * scale
            dk[b, :, g, :] += (ds.T @ qd[b, :, c, :]) * scale
            dv[b, :, g, :] += p.T @ gd[b, :, c, :]
    return dq, dk, dv
