/*
 * ulysses.h -- C ABI of libulysses.so: the DeepSpeed-Ulysses attention hot
 * path on one MI355X (gfx950), with the P ranks of a sequence-parallel group
 * simulated as P contiguous sub-buffers of one device allocation.
 *
 * The path ("Sequence Parallelism II: DeepSpeed Ulysses and All-to-All
 * Attention", section 2 "Forward Pass in Slow Motion", steps three to five,
 * and section 7, which describes the attention module as layout transpose,
 * local attention, inverse transpose):
 *
 *   ulysses_seq_to_head      Q, K, V: sequence shards -> head shards
 *                            (ulysses_seq_to_head_qkv: all three in one launch)
 *   ulysses_attention_local  one rank: softmax(Q K^T / sqrt(D)) V per head
 *   ulysses_head_to_seq      attention output: head shards -> sequence shards
 *
 * Gradients of the local attention: ulysses_attention_local_lse (forward with
 * each row's log-sum-exp) and ulysses_attention_local_backward.  Past the
 * head-count bound (section 8), the per-visit calls of a ring over key/value
 * blocks: ulysses_attention_chunk, ulysses_attention_merge (or both at once,
 * ulysses_attention_chunk_accumulate) and ulysses_attention_chunk_backward.
 *
 * Buffer layouts (row-major, head_dim innermost, rank outermost):
 *   SEQ [P][B][S/P][n_heads][head_dim]   rank i holds tokens [i*S/P, (i+1)*S/P)
 *   HEAD[P][B][S][n_heads/P][head_dim]   rank j holds heads  [j*n_heads/P, (j+1)*n_heads/P)
 *   PIECES[P][P][B][S/P][n_heads/P][head_dim]
 *                                        rank j's heads as P pieces, one per peer
 *                                        rank i (tokens [i*S/P, (i+1)*S/P)), in rank
 *                                        order: what the exchange delivers before
 *                                        any unpack (ulysses_seq_to_pieces*,
 *                                        ulysses_attention_local_pieces,
 *                                        ulysses_pieces_to_seq)
 * These are the rank-local shapes [B, S/P, num_heads, head_dim] and
 * [B, S, num_heads/P, head_dim] of "Comparing Ulysses and Megatron Sequence
 * Parallelism", section "DeepSpeed Attention", stacked over the P ranks.
 * For B = 1, SEQ is byte-identical to the global [S][n_heads][head_dim] tensor.
 *
 * Conventions shared by every call:
 *  - All data pointers are device pointers.  The caller allocates and owns
 *    every buffer; the library never allocates, frees or keeps a pointer.
 *  - Calls are asynchronous: they enqueue on `stream` (a hipStream_t;
 *    NULL means the default stream) and return.  Device-side faults surface at
 *    the caller's next synchronisation of that stream.
 *  - Every precondition is checked before anything is enqueued, so a call that
 *    returns an error has written nothing.  Nothing is thrown across the ABI.
 *  - Sizes of zero are valid: with B = 0 or S = 0 (Sq = 0 for the chunk
 *    forward calls) nothing is enqueued and a pointer may then be NULL; the
 *    chunk calls state what an empty key chunk or query block writes.
 *  - Outputs must not overlap inputs (except the in/out buffers a call names:
 *    the running result of the chunk calls and the in-place merge).
 *  - ulysses_last_error() returns a per-thread description of the last error.
 */
#ifndef ULYSSES_H
#define ULYSSES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ULY_OK = 0,
    ULY_ERR_INVALID_ARGUMENT = 1, /* NULL/misaligned pointer, negative size, overlap */
    ULY_ERR_NOT_DIVISIBLE = 2,    /* S % P, n_heads % P, n_q_heads % n_kv_heads, P > n_heads */
    ULY_ERR_UNSUPPORTED = 3,      /* dtype / head_dim / size without a kernel */
    ULY_ERR_HIP = 4               /* the HIP runtime refused a launch */
} uly_status_t;

typedef enum {
    ULY_DTYPE_BF16 = 0, /* 2-byte elements (bfloat16 for attention) */
    ULY_DTYPE_FP32 = 1  /* 4-byte elements (float32 for attention) */
} uly_dtype_t;

/*
 * Sequence shards -> head shards: the first All-to-All, applied to each of
 * Q, K and V ("Sequence Parallelism II...", section 1 "The Layout Problem"
 * and section 3 "Why All-to-All Is the Right Collective"; "Comparing Ulysses
 * and Megatron...", section "DeepSpeed Attention").  Each rank cuts its
 * tokens' heads into P groups; group j goes to rank j, which stores the
 * groups it receives in source-rank order, so it holds every token for its
 * heads:
 *
 *   HEAD[j][b][i*S/P + t][c][d] = SEQ[i][b][t][j*(n_heads/P) + c][d]
 *
 * seq_shards   device, read:  P*B*(S/P)*n_heads*head_dim elements (SEQ layout)
 * head_shards  device, write: the same number of elements (HEAD layout)
 * B >= 0, S >= 0, n_heads >= 1, head_dim >= 1, P >= 1; S % P == 0,
 * n_heads % P == 0 (so P <= n_heads, the head-count bound of section 4 of
 * the first page), P*B <= 65535.
 * dtype only sets the element size: elements are moved as raw bits (NaN
 * payloads included), so any 2- or 4-byte type may be passed.
 * Both pointers must be aligned to the element size and must not overlap.
 */
uly_status_t ulysses_seq_to_head(const void *seq_shards, void *head_shards, int64_t B,
                                 int64_t S, int64_t n_heads, int64_t head_dim, int32_t P,
                                 uly_dtype_t dtype, void *stream);

/*
 * The first All-to-All of Q, K and V in one launch (the three exchanges
 * "Comparing Ulysses and Megatron...", section "DeepSpeed Attention costs",
 * counts for one attention layer): exactly ulysses_seq_to_head applied to
 * (q_seq -> q_head, n_q_heads) and to (k_seq -> k_head) and (v_seq -> v_head)
 * with n_kv_heads, with one kernel launch instead of three (three again when
 * the three tensors' (rank, batch) slices together reach 2^32 16-byte
 * vectors, where each launch is long anyway).
 *
 * Arguments and errors as for ulysses_seq_to_head, applied to each pair; in
 * addition no destination may overlap any source or another destination.
 * With B = 0 or S = 0 nothing is enqueued.
 */
uly_status_t ulysses_seq_to_head_qkv(const void *q_seq, const void *k_seq, const void *v_seq,
                                     void *q_head, void *k_head, void *v_head, int64_t B,
                                     int64_t S, int64_t n_q_heads, int64_t n_kv_heads,
                                     int64_t head_dim, int32_t P, uly_dtype_t dtype,
                                     void *stream);

/*
 * Head shards -> sequence shards: the second All-to-All that returns the
 * attention output to sequence ownership ("Sequence Parallelism II...",
 * section 2, fifth step; for the output the pieces are sequence slices,
 * section 3).  Exact inverse of ulysses_seq_to_head:
 *
 *   SEQ[i][b][t][j*(n_heads/P) + c][d] = HEAD[j][b][i*S/P + t][c][d]
 *
 * Arguments and errors as for ulysses_seq_to_head, with the roles of the two
 * buffers swapped (head_shards is read, seq_shards is written).
 */
uly_status_t ulysses_head_to_seq(const void *head_shards, void *seq_shards, int64_t B,
                                 int64_t S, int64_t n_heads, int64_t head_dim, int32_t P,
                                 uly_dtype_t dtype, void *stream);

/*
 * One rank's local attention over the full sequence for its heads
 * ("Sequence Parallelism II...", section 2, fourth step; the attention
 * skeleton in the Introduction of "Comparing Ulysses and Megatron...", which
 * calls scaled-dot-product attention with its default scale):
 *
 *   o[b][i][c][:] = sum_{k in K(i)} softmax_k(<q[b][i][c], k[b][k][g]> / sqrt(head_dim)) v[b][k][g][:]
 *
 * with g = c / (n_q_heads / n_kv_heads) (grouped key/value heads, n_kv_head
 * of the skeleton), K(i) = {0..S-1}, or {0..i} when causal (the triangular
 * pattern of section 8 of the first page, in global token order).
 *
 * q, o  device, [B][S][n_q_heads][head_dim];  k, v  device, [B][S][n_kv_heads][head_dim].
 * q is read, o is written; o must not overlap q, k or v (q, k, v may alias).
 * B >= 0, S >= 0, n_q_heads >= 1, n_kv_heads >= 1, n_q_heads % n_kv_heads == 0.
 * Supported: ULY_DTYPE_BF16 with head_dim 128 (bf16 MFMA, fp32 accumulation
 * and softmax, output rounded to nearest even), pointers 16-byte aligned;
 * ULY_DTYPE_FP32 with head_dim 32, 64 or 128 (fp32 throughout), pointers
 * 4-byte aligned.  Anything else returns ULY_ERR_UNSUPPORTED.
 * S < 2^31 and B*n_q_heads < 2^31; for ULY_DTYPE_BF16 also n_kv_heads <= 65536.
 */
uly_status_t ulysses_attention_local(const void *q, const void *k, const void *v, void *o,
                                     int64_t B, int64_t S, int64_t n_q_heads,
                                     int64_t n_kv_heads, int64_t head_dim, int32_t causal,
                                     uly_dtype_t dtype, void *stream);

/*
 * ulysses_attention_local, also writing each row's log-sum-exp, which the
 * gradient call needs:
 *
 *   lse[b][c][i] = log( sum_{k in K(i)} exp(<q[b][i][c], k[b][k][g]> / sqrt(head_dim)) )
 *
 * (natural log).  lse  device, write, [B][n_q_heads][S] float32, 4-byte
 * aligned, must not overlap q, k, v or o.  Everything else as for
 * ulysses_attention_local.
 */
uly_status_t ulysses_attention_local_lse(const void *q, const void *k, const void *v, void *o,
                                         float *lse, int64_t B, int64_t S, int64_t n_q_heads,
                                         int64_t n_kv_heads, int64_t head_dim, int32_t causal,
                                         uly_dtype_t dtype, void *stream);

/*
 * ulysses_attention_local(_lse) for sequences too short to fill the GPU with
 * query blocks.  Causal attention keeps its triangular work inside each head
 * ("Sequence Parallelism II...", section 8 "Where Ulysses Does Not Solve
 * Everything"): the last query block sees every key, and at a few thousand
 * tokens that one block's walk over the keys bounds the call.  Here the key
 * tiles of each 64-row query block may be cut into ranges handled by
 * different workgroups; the partial results, attention over disjoint key
 * sets, combine by their share of the exp-sum
 *
 *   lse = log sum_u exp(lse_u),   o = sum_u exp(lse_u - lse) o_u
 *
 * with o_u, lse_u the normalised output and log-sum-exp over key range u,
 * kept in fp32 in the workspace and rounded to bf16 once by a second
 * launch.  Results agree with ulysses_attention_local(_lse) to rounding (the
 * sums are taken in another order), not bit for bit; repeated calls give the
 * same bits.
 *
 * ulysses_attention_local_split_workspace: *bytes = the workspace the call
 * needs for these sizes on the current device (0 when nothing is split: the
 * call is then ulysses_attention_local(_lse) itself).  bytes  host, write.
 * ulysses_attention_local_split: arguments as ulysses_attention_local_lse,
 * with lse optional (NULL: not written), plus workspace (device, at least
 * the queried bytes, 16-byte aligned, must not overlap any tensor; may be
 * NULL when 0 bytes are needed; overwritten, nothing carried between calls)
 * and workspace_bytes (its size).  Calls that share a workspace must not
 * overlap in time.  Supported: ULY_DTYPE_BF16 with head_dim 128 and
 * B * n_q_heads <= 65535 (else ULY_ERR_UNSUPPORTED); a missing or too small
 * workspace is ULY_ERR_INVALID_ARGUMENT.  The split pays where a few heads
 * leave the compute units with one long block each (measured on MI355X:
 * S = 16384 with 1 head 150 -> 115 us, S = 8192 with 2 heads 83 -> 73 us); a
 * schedule model of the two launches decides, so that nothing is split where
 * the query blocks alone already balance the compute units (S = 4096 with 4
 * heads), or beyond 512 blocks of 64 rows.
 */
uly_status_t ulysses_attention_local_split_workspace(int64_t B, int64_t S, int64_t n_q_heads,
                                                    int64_t head_dim, int32_t causal,
                                                    uly_dtype_t dtype, uint64_t *bytes);
uly_status_t ulysses_attention_local_split(const void *q, const void *k, const void *v, void *o,
                                           float *lse, int64_t B, int64_t S, int64_t n_q_heads,
                                           int64_t n_kv_heads, int64_t head_dim, int32_t causal,
                                           uly_dtype_t dtype, void *workspace,
                                           uint64_t workspace_bytes, void *stream);

/*
 * The two exchanges with their pieces left where the collective delivers
 * them, and the attention that reads and writes that order, so that the
 * unpack after the first exchange and the pack before the second are not
 * separate passes over HBM ("Sequence Parallelism II...", section 3: every
 * rank cuts its tensor into P pieces and after the exchange holds one piece
 * from every rank; section 2 puts the attention between the two exchanges).
 *
 *   PIECES[j][i][b][t][c][d] = SEQ[i][b][t][j*(n_heads/P) + c][d]
 *
 * Rank j's buffer PIECES[j] is [P][B][S/P][n_heads/P][head_dim]: piece i
 * holds rank i's tokens, for every batch entry.  It is HEAD[j] with the token
 * axis cut at the piece boundaries and the batch axis moved inside the
 * pieces; for B = 1 the two layouts are the same bytes.  For the output the
 * same buffer is the send order of the second exchange: piece i of rank j
 * is what rank j sends to rank i.
 *
 * ulysses_seq_to_pieces: SEQ -> PIECES (the first exchange without the
 * unpack); ulysses_seq_to_pieces_qkv: the same for Q (n_q_heads), K and V
 * (n_kv_heads) in one launch; ulysses_pieces_to_seq: PIECES -> SEQ (the
 * second exchange), the exact inverse of ulysses_seq_to_pieces.  Arguments,
 * limits and errors as for ulysses_seq_to_head, ulysses_seq_to_head_qkv and
 * ulysses_head_to_seq.
 */
uly_status_t ulysses_seq_to_pieces(const void *seq_shards, void *pieces, int64_t B, int64_t S,
                                   int64_t n_heads, int64_t head_dim, int32_t P, uly_dtype_t dtype,
                                   void *stream);
uly_status_t ulysses_seq_to_pieces_qkv(const void *q_seq, const void *k_seq, const void *v_seq,
                                       void *q_pieces, void *k_pieces, void *v_pieces, int64_t B,
                                       int64_t S, int64_t n_q_heads, int64_t n_kv_heads,
                                       int64_t head_dim, int32_t P, uly_dtype_t dtype,
                                       void *stream);
uly_status_t ulysses_pieces_to_seq(const void *pieces, void *seq_shards, int64_t B, int64_t S,
                                   int64_t n_heads, int64_t head_dim, int32_t P, uly_dtype_t dtype,
                                   void *stream);

/*
 * ulysses_attention_local (with lse if lse is not NULL) on one rank's
 * buffers in pieces order: q, k, v are read as PIECES[j] and o is written in
 * the same order, [P][B][S/P][heads][head_dim]; token s of batch entry b is
 * row (s / (S/P)) * B * (S/P) + b * (S/P) + s % (S/P).  lse stays
 * [B][n_q_heads][S] in token order.  The result equals unpacking q, k, v to
 * [B][S][heads][head_dim], ulysses_attention_local(_lse), and cutting o back
 * into the pieces, bit for bit.  P >= 1 and S % P == 0 (else
 * ULY_ERR_INVALID_ARGUMENT / ULY_ERR_NOT_DIVISIBLE); for ULY_DTYPE_BF16 with
 * B > 1, S/P must be a multiple of 64 (a key tile never spans two pieces),
 * else ULY_ERR_UNSUPPORTED.  Everything else as for ulysses_attention_local.
 */
uly_status_t ulysses_attention_local_pieces(const void *q, const void *k, const void *v, void *o,
                                            float *lse, int64_t B, int64_t S, int64_t n_q_heads,
                                            int64_t n_kv_heads, int64_t head_dim, int32_t P,
                                            int32_t causal, uly_dtype_t dtype, void *stream);

/*
 * ulysses_attention_local_backward on one rank's buffers in piece order: the
 * backward pass runs the two exchanges in reverse ("Sequence Parallelism
 * II...", section 6), so dout arrives in the first exchange's receive order
 * and dq, dk, dv leave in the second's send order, like q, k, v and o of the
 * forward.  q, k, v, o, dout are read and dq, dk, dv written as
 * [P][B][S/P][heads][head_dim] (token s of batch entry b as for
 * ulysses_attention_local_pieces); lse and delta stay [B][n_q_heads][S].  The
 * result equals the gradient call on unpacked buffers, cut back into pieces,
 * bit for bit.  P >= 1 and S % P == 0 (else ULY_ERR_INVALID_ARGUMENT /
 * ULY_ERR_NOT_DIVISIBLE); with B > 1, S/P must be a multiple of 64 (else
 * ULY_ERR_UNSUPPORTED).  Everything else as for
 * ulysses_attention_local_backward.
 */
uly_status_t ulysses_attention_local_backward_pieces(
    const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
    float *delta, void *dq, void *dk, void *dv, int64_t B, int64_t S, int64_t n_q_heads,
    int64_t n_kv_heads, int64_t head_dim, int32_t P, int32_t causal, uly_dtype_t dtype,
    void *stream);

/*
 * Gradients of one rank's local attention.  The backward pass of the path
 * runs the two layout changes in reverse ("Sequence Parallelism II...",
 * section 6: the output gradient goes seq->head with ulysses_seq_to_head, the
 * Q, K and V gradients head->seq with ulysses_head_to_seq); this call is the
 * step between them, the derivative of ulysses_attention_local.  With
 * p = exp(s - lse[i]) the softmax weight of score s = <q_i, k_k>/sqrt(head_dim)
 * and delta_i = sum_d dout[i][d] o[i][d]:
 *
 *   dS    = p (<dout_i, v_k> - delta_i)
 *   dq[i] = sum_k dS k_k / sqrt(head_dim)
 *   dk[k] = sum over the query heads of kv head g and rows i of dS q_i / sqrt(head_dim)
 *   dv[k] = sum over the same of p dout_i
 *
 * q, o, dout, dq  device, [B][S][n_q_heads][head_dim];  k, v, dk, dv  device,
 * [B][S][n_kv_heads][head_dim]; lse  device, read, [B][n_q_heads][S] float32 as
 * written by ulysses_attention_local_lse for the same q, k, v (o is its
 * output); delta  device, scratch, [B][n_q_heads][S] float32, overwritten.
 * dq, dk, dv and delta are written; they must not overlap each other or any
 * input.  Supported: ULY_DTYPE_BF16 with head_dim 128 (bf16 MFMA, fp32
 * accumulation, weights and dS rounded to bf16 for the products, outputs
 * rounded to nearest even); tensors 16-byte aligned, lse and delta 4-byte
 * aligned; n_q_heads <= 65536 and n_kv_heads <= 65536.  Anything else returns
 * ULY_ERR_UNSUPPORTED.  Shape rules as for ulysses_attention_local.
 */
uly_status_t ulysses_attention_local_backward(const void *q, const void *k, const void *v,
                                              const void *o, const void *dout, const float *lse,
                                              float *delta, void *dq, void *dk, void *dv,
                                              int64_t B, int64_t S, int64_t n_q_heads,
                                              int64_t n_kv_heads, int64_t head_dim,
                                              int32_t causal, uly_dtype_t dtype, void *stream);

/*
 * Split gradients: ulysses_attention_local_backward for sizes where the
 * longest dK/dV key blocks (the first ones under the causal mask, or every
 * one of a few grouped heads) would leave most compute units idle while they
 * run.  The query stream of such a block (every query head of its group,
 * every query tile) is cut into up to 8 units of consecutive tiles on
 * different workgroups; each unit keeps its fp32 sums in a slot of the
 * workspace, and a second launch adds the slots in unit order and writes dk
 * and dv.  dq is the plain
 * call's, bit for bit; dk and dv agree with it to rounding (the sums are
 * added in another order), and repeated calls give the same bits.  The
 * gradients are those of ulysses_attention_local_backward, the step between
 * the reversed layout changes ("Sequence Parallelism II...", section 6).
 *
 * ulysses_attention_local_backward_split_workspace: *bytes = the workspace
 * the call needs for these sizes on the current device (0 when nothing is
 * split: the call is then ulysses_attention_local_backward itself).  bytes
 * host, write.
 * ulysses_attention_local_backward_split: arguments and errors as
 * ulysses_attention_local_backward, plus workspace (device, at least the
 * queried bytes, 256-byte aligned, must not overlap any tensor; may be NULL
 * when 0 bytes are needed; overwritten, nothing carried between calls) and
 * workspace_bytes (its size); a missing or too small workspace is
 * ULY_ERR_INVALID_ARGUMENT.  Calls that share a workspace must not overlap
 * in time.  A schedule model of the launch decides what to cut.
 */
uly_status_t ulysses_attention_local_backward_split_workspace(int64_t B, int64_t S,
                                                             int64_t n_q_heads, int64_t n_kv_heads,
                                                             int64_t head_dim, int32_t causal,
                                                             uly_dtype_t dtype, uint64_t *bytes);
uly_status_t ulysses_attention_local_backward_split(
    const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
    float *delta, void *dq, void *dk, void *dv, int64_t B, int64_t S, int64_t n_q_heads,
    int64_t n_kv_heads, int64_t head_dim, int32_t causal, uly_dtype_t dtype, void *workspace,
    uint64_t workspace_bytes, void *stream);

/*
 * ulysses_attention_local_backward without the delta workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, results
 * and errors as ulysses_attention_local_backward, minus delta: the library
 * keeps delta in a file-scope array of 2^20 floats (4 MiB) in each GPU's
 * memory, held until the process ends, whose address it looks up on the first
 * call on each device.  Limit: B * n_q_heads * S <= 1048576 (e.g. 4 heads x
 * 262144 rows); larger sizes return ULY_ERR_UNSUPPORTED before anything is
 * enqueued.  The call allocates nothing (no hipMalloc, no allocating library
 * routine).  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (different streams, or threads) race on it and must be
 * ordered by the caller; each call writes its delta before reading it, so
 * nothing from an earlier call is read.  A failure of the one-time address
 * lookup returns ULY_ERR_HIP.
 */
uly_status_t ulysses_attention_local_backward_noalloc(const void *q, const void *k, const void *v,
                                                      const void *o, const void *dout,
                                                      const float *lse, void *dq, void *dk,
                                                      void *dv, int64_t B, int64_t S,
                                                      int64_t n_q_heads, int64_t n_kv_heads,
                                                      int64_t head_dim, int32_t causal,
                                                      uly_dtype_t dtype, void *stream);

/*
 * One visit of a key/value chunk.  Past the head-count bound the sequence
 * degree can grow only if a query block stays put while key/value blocks
 * circulate among the ranks of a head group ("Sequence Parallelism II...",
 * section 8, which names Ring Attention and blockwise key/value partitioning
 * for that case).  Each visit is attention restricted to the keys of one
 * chunk, in global token positions:
 *
 *   query row i sits at position q_pos0 + i, key j at k_pos0 + j;
 *   K(i) = every j, or with causal the j with k_pos0 + j <= q_pos0 + i;
 *   o[b][i][c][:] = sum_{j in K(i)} softmax_j(<q[b][i][c], k[b][j][g]> / sqrt(head_dim)) v[b][j][g][:]
 *   lse[b][c][i]  = log( sum_{j in K(i)} exp(<q[b][i][c], k[b][j][g]> / sqrt(head_dim)) )
 *
 * with g as in ulysses_attention_local.  A row with K(i) empty gets o = 0 and
 * lse = -inf (the identity of ulysses_attention_merge).  With Sq = Skv = S and
 * q_pos0 = k_pos0 this is ulysses_attention_local_lse.
 *
 * q, o  device, [B][Sq][n_q_heads][head_dim];  k, v  device,
 * [B][Skv][n_kv_heads][head_dim];  lse  device, write, [B][n_q_heads][Sq]
 * float32 (required).  o and lse must not overlap each other or any input.
 * Sq, Skv in [0, 2^30); Skv = 0 is valid (every row empty; k and v may then
 * be NULL); positions within +-2^62.  Supported dtypes, head_dim, alignment
 * and other limits as for ulysses_attention_local.
 */
uly_status_t ulysses_attention_chunk(const void *q, const void *k, const void *v, void *o,
                                     float *lse, int64_t B, int64_t Sq, int64_t Skv,
                                     int64_t n_q_heads, int64_t n_kv_heads, int64_t head_dim,
                                     int64_t q_pos0, int64_t k_pos0, int32_t causal,
                                     uly_dtype_t dtype, void *stream);

/*
 * One visit of a key/value chunk merged into a running result in the same
 * launch: on entry o and lse hold the result over the keys of earlier visits
 * (as written by ulysses_attention_chunk or by this call), on exit the result
 * over those keys and this chunk's.  The same as ulysses_attention_chunk into
 * temporaries followed by ulysses_attention_merge into (o, lse), without the
 * temporaries and the merge's pass over them:
 *
 *   lse' = log(exp(lse) + exp(lse_c)),  o' = exp(lse - lse') o + exp(lse_c - lse') o_c
 *
 * with (o_c, lse_c) this chunk's attention as defined for
 * ulysses_attention_chunk.  Rows with no visible key in this chunk keep o and
 * lse bit for bit.  o and lse are read and written (bf16 o rounded to nearest
 * even); everything else as for ulysses_attention_chunk (ULY_DTYPE_BF16 with
 * head_dim 128 only; anything else returns ULY_ERR_UNSUPPORTED).
 */
uly_status_t ulysses_attention_chunk_accumulate(const void *q, const void *k, const void *v, void *o,
                                                float *lse, int64_t B, int64_t Sq, int64_t Skv,
                                                int64_t n_q_heads, int64_t n_kv_heads,
                                                int64_t head_dim, int64_t q_pos0, int64_t k_pos0,
                                                int32_t causal, uly_dtype_t dtype, void *stream);

/*
 * Combination of two partial results over disjoint key sets (the visits of
 * ulysses_attention_chunk): the softmax over the union weights each part by
 * its share of the total exp-sum,
 *
 *   lse = log(exp(lse_a) + exp(lse_b))
 *   o   = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b
 *
 * computed in fp32 against max(lse_a, lse_b); a row with lse_a = lse_b = -inf
 * gives o = 0 and lse = -inf.
 *
 * o_a, o_b, o  device, [B][S][n_heads][head_dim] of dtype (bf16 outputs
 * rounded to nearest even), 16-byte aligned; lse_a, lse_b, lse  device,
 * [B][n_heads][S] float32, 4-byte aligned.  In place is allowed: o may be
 * o_a or o_b (the same pointer) and lse may be lse_a or lse_b; any other
 * overlap is an error.  head_dim * element size must be a power of two in
 * [16, 1024] bytes; B*S*n_heads < 2^32.
 */
uly_status_t ulysses_attention_merge(const void *o_a, const float *lse_a, const void *o_b,
                                     const float *lse_b, void *o, float *lse, int64_t B, int64_t S,
                                     int64_t n_heads, int64_t head_dim, uly_dtype_t dtype,
                                     void *stream);

/*
 * Gradient contributions of one key/value chunk visit, for training past the
 * head-count bound (the visits of ulysses_attention_chunk; the derivative of
 * ulysses_attention_local restricted to the chunk's keys).  With o and lse the
 * query block's merged forward result over every key of the ring (the last
 * ulysses_attention_chunk_accumulate or ulysses_attention_merge), the softmax
 * weight of a visible pair is p = exp(s - lse[i]) for s = <q_i, k_j>/sqrt(D),
 * delta_i = sum_d dout[i][d] o[i][d], dS = p (<dout_i, v_j> - delta_i), and
 *
 *   dq[i] (+)= sum over this chunk's visible keys j of dS k_j / sqrt(D)
 *   dk[j] (+)= sum over the rows i and query heads of kv head g of dS q_i / sqrt(D)
 *   dv[j] (+)= sum over the same of p dout_i
 *
 * Visibility, positions and head grouping as for ulysses_attention_chunk.
 * With accumulate_dq = 0 the contribution to dq is written (a row that this
 * visit does not reach gets zeros), otherwise added to dq (fp32 sum of the
 * stored bf16 value and the contribution, rounded once); accumulate_dkv does
 * the same for dk and dv.  Summed over a ring's visits (the first visit of a
 * query block writes its dq, the first visit of a chunk its dk and dv) the
 * contributions are the gradients of the whole attention.
 *
 * q, o, dout, dq  device, [B][Sq][n_q_heads][head_dim];  k, v, dk, dv  device,
 * [B][Skv][n_kv_heads][head_dim];  lse  device, read, [B][n_q_heads][Sq]
 * float32;  delta  device, scratch, [B][n_q_heads][Sq] float32, overwritten.
 * Outputs must not overlap each other or any input.  ULY_DTYPE_BF16 with
 * head_dim 128 only; Sq, Skv in [0, 2^30); other limits as for
 * ulysses_attention_local_backward.  Sq = 0 (Skv = 0) leaves only the key
 * (query) side, whose contributions are then zero; the pointers of the empty
 * side may be NULL.
 */
uly_status_t ulysses_attention_chunk_backward(const void *q, const void *k, const void *v,
                                              const void *o, const void *dout, const float *lse,
                                              float *delta, void *dq, void *dk, void *dv, int64_t B,
                                              int64_t Sq, int64_t Skv, int64_t n_q_heads,
                                              int64_t n_kv_heads, int64_t head_dim, int64_t q_pos0,
                                              int64_t k_pos0, int32_t causal, int32_t accumulate_dq,
                                              int32_t accumulate_dkv, uly_dtype_t dtype,
                                              void *stream);

/* Static English name of a status code. */
const char *ulysses_status_string(uly_status_t s);

/* Detail of the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next library call on this thread. */
const char *ulysses_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H */
