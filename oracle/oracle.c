/*
 * CPU oracle for the Ulysses attention path -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct host implementation of what the path
 * computes, used to check the HIP library.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the product
 * path never calls it and shares no code, header or table with it.
 *
 * Sources (the pages this follows):
 *  [P1] "Sequence Parallelism II: DeepSpeed Ulysses and All-to-All Attention"
 *  [P2] "Comparing Ulysses and Megatron Sequence Parallelism"
 *
 * Layout of P virtual ranks held in one buffer (rank-major, head_dim innermost):
 *   SEQ [P][B][S/P][H][D]   rank i owns tokens [i*S/P, (i+1)*S/P), all heads
 *   HEAD[P][B][S][H/P][D]   rank j owns heads  [j*H/P, (j+1)*H/P), all tokens
 *   PIECES[P][P][B][S/P][H/P][D]  rank j's P pieces, one per peer rank, in
 *                           rank order (what the exchange delivers, before
 *                           any unpack)
 *
 * Everything is written as explicit loops over the definitions.  Floating
 * point work is fp64 from the exact values of the stored inputs; there is no
 * blocking, fusion or reordering.  OpenMP only splits independent output rows
 * among threads, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_OK = 0, ORC_BAD_ARG = 1, ORC_NOT_DIVISIBLE = 2, ORC_NO_MEMORY = 3 };
enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_F64 = 2 };

static int check_layout(int64_t B, int64_t S, int64_t H, int64_t D, int32_t P,
                        int32_t elem_bytes)
{
    if (B < 0 || S < 0 || H < 1 || D < 1 || P < 1 || elem_bytes < 1)
        return ORC_BAD_ARG;
    if (S % P != 0 || H % P != 0)
        return ORC_NOT_DIVISIBLE;
    return ORC_OK;
}

/*
 * Sequence shards -> head shards ([P1] section 1 "The Layout Problem" and
 * section 3 "Why All-to-All Is the Right Collective"; [P2] section
 * "DeepSpeed Attention").  Every rank splits its local tensor into P pieces
 * along the head axis and piece j goes to rank j, which stacks the pieces it
 * receives in source-rank order, so that it ends up with every token of the
 * sequence for its own group of heads.
 *
 * Element (source rank i, batch b, local token t, head h, dim d) moves to
 * destination rank j = h / (H/P), local head c = h mod (H/P), global token
 * i*(S/P) + t.  Elements are copied as raw bytes (no arithmetic on values).
 */
int oracle_seq_to_head(const void *seq, void *head, int64_t B, int64_t S,
                       int64_t H, int64_t D, int32_t P, int32_t elem_bytes)
{
    int rc = check_layout(B, S, H, D, P, elem_bytes);
    if (rc != ORC_OK)
        return rc;
    const int64_t Sp = S / P, hp = H / P;
    const unsigned char *src = (const unsigned char *)seq;
    unsigned char *dst = (unsigned char *)head;
    for (int64_t i = 0; i < P; ++i)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t t = 0; t < Sp; ++t)
                for (int64_t h = 0; h < H; ++h) {
                    const int64_t j = h / hp, c = h % hp, s = i * Sp + t;
                    for (int64_t d = 0; d < D; ++d) {
                        const int64_t from = (((i * B + b) * Sp + t) * H + h) * D + d;
                        const int64_t to = (((j * B + b) * S + s) * hp + c) * D + d;
                        memcpy(dst + to * elem_bytes, src + from * elem_bytes,
                               (size_t)elem_bytes);
                    }
                }
    return ORC_OK;
}

/*
 * Head shards -> sequence shards, the second All-to-All that returns the
 * attention output to sequence ownership ([P1] section 2 "Forward Pass in
 * Slow Motion", fifth step; [P2] section "DeepSpeed Attention").  For the
 * output the pieces are sequence slices: rank j sends tokens
 * [i*S/P, (i+1)*S/P) of its heads to rank i.
 *
 * Element (rank j, batch b, global token s, local head c, dim d) moves to
 * rank i = s / (S/P), local token s mod (S/P), head j*(H/P) + c.
 */
int oracle_head_to_seq(const void *head, void *seq, int64_t B, int64_t S,
                       int64_t H, int64_t D, int32_t P, int32_t elem_bytes)
{
    int rc = check_layout(B, S, H, D, P, elem_bytes);
    if (rc != ORC_OK)
        return rc;
    const int64_t Sp = S / P, hp = H / P;
    const unsigned char *src = (const unsigned char *)head;
    unsigned char *dst = (unsigned char *)seq;
    for (int64_t j = 0; j < P; ++j)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t s = 0; s < S; ++s)
                for (int64_t c = 0; c < hp; ++c) {
                    const int64_t i = s / Sp, t = s % Sp, h = j * hp + c;
                    for (int64_t d = 0; d < D; ++d) {
                        const int64_t from = (((j * B + b) * S + s) * hp + c) * D + d;
                        const int64_t to = (((i * B + b) * Sp + t) * H + h) * D + d;
                        memcpy(dst + to * elem_bytes, src + from * elem_bytes,
                               (size_t)elem_bytes);
                    }
                }
    return ORC_OK;
}

/*
 * The first All-to-All as the collective itself, without the unpack ([P1]
 * section 3 "Why All-to-All Is the Right Collective": every rank splits its
 * local tensor into P pieces, keeps the piece addressed to itself and sends
 * piece j to rank j; afterwards each rank holds one piece from every rank).
 * For sequence shards the pieces are head groups ([P1] section 1; [P2]
 * section "DeepSpeed Attention"): piece j of rank i is [B][S/P][H/P][D], its
 * tokens' heads [j*H/P, (j+1)*H/P).  Rank j keeps the pieces it receives in
 * source-rank order:
 *   1. every rank i cuts its shard into its P send pieces,
 *   2. the exchange: rank j's piece slot i takes what rank i sent to rank j.
 * Raw byte copies.
 */
int oracle_seq_to_pieces(const void *seq, void *pieces, int64_t B, int64_t S,
                         int64_t H, int64_t D, int32_t P, int32_t elem_bytes)
{
    int rc = check_layout(B, S, H, D, P, elem_bytes);
    if (rc != ORC_OK)
        return rc;
    const int64_t Sp = S / P, hp = H / P;
    const size_t piece = (size_t)(B * Sp * hp * D * elem_bytes);
    unsigned char *send = (unsigned char *)malloc(piece * (size_t)P * (size_t)P + 1);
    if (!send)
        return ORC_NO_MEMORY;
    const unsigned char *src = (const unsigned char *)seq;
    unsigned char *dst = (unsigned char *)pieces;
    /* 1. send[i][j][b][t][c][d] = SEQ[i][b][t][j*hp + c][d] */
    for (int64_t i = 0; i < P; ++i)
        for (int64_t j = 0; j < P; ++j)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t t = 0; t < Sp; ++t)
                    for (int64_t c = 0; c < hp; ++c)
                        for (int64_t d = 0; d < D; ++d) {
                            const int64_t from = (((i * B + b) * Sp + t) * H + j * hp + c) * D + d;
                            const int64_t to = ((((i * P + j) * B + b) * Sp + t) * hp + c) * D + d;
                            memcpy(send + to * elem_bytes, src + from * elem_bytes,
                                   (size_t)elem_bytes);
                        }
    /* 2. rank j, slot i <- the piece rank i addressed to rank j */
    for (int64_t j = 0; j < P; ++j)
        for (int64_t i = 0; i < P; ++i)
            memcpy(dst + (size_t)(j * P + i) * piece, send + (size_t)(i * P + j) * piece, piece);
    free(send);
    return ORC_OK;
}

/*
 * The second All-to-All from pieces in send order ([P1] section 2, fifth
 * step, and section 3: for the output the pieces are sequence slices).  Rank
 * j holds its output cut into P pieces, piece i = its heads [j*H/P,
 * (j+1)*H/P) over the tokens of rank i, [B][S/P][H/P][D]:
 *   1. the exchange: rank i's slot j takes the piece rank j addressed to it,
 *   2. rank i places the piece from rank j at heads [j*H/P, (j+1)*H/P) of
 *      its tokens.
 * Raw byte copies.
 */
int oracle_pieces_to_seq(const void *pieces, void *seq, int64_t B, int64_t S,
                         int64_t H, int64_t D, int32_t P, int32_t elem_bytes)
{
    int rc = check_layout(B, S, H, D, P, elem_bytes);
    if (rc != ORC_OK)
        return rc;
    const int64_t Sp = S / P, hp = H / P;
    const size_t piece = (size_t)(B * Sp * hp * D * elem_bytes);
    unsigned char *recv = (unsigned char *)malloc(piece * (size_t)P * (size_t)P + 1);
    if (!recv)
        return ORC_NO_MEMORY;
    const unsigned char *src = (const unsigned char *)pieces;
    unsigned char *dst = (unsigned char *)seq;
    /* 1. recv[i][j] = the piece rank j addressed to rank i */
    for (int64_t i = 0; i < P; ++i)
        for (int64_t j = 0; j < P; ++j)
            memcpy(recv + (size_t)(i * P + j) * piece, src + (size_t)(j * P + i) * piece, piece);
    /* 2. SEQ[i][b][t][j*hp + c][d] = recv[i][j][b][t][c][d] */
    for (int64_t i = 0; i < P; ++i)
        for (int64_t j = 0; j < P; ++j)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t t = 0; t < Sp; ++t)
                    for (int64_t c = 0; c < hp; ++c)
                        for (int64_t d = 0; d < D; ++d) {
                            const int64_t from = ((((i * P + j) * B + b) * Sp + t) * hp + c) * D + d;
                            const int64_t to = (((i * B + b) * Sp + t) * H + j * hp + c) * D + d;
                            memcpy(dst + to * elem_bytes, recv + from * elem_bytes,
                                   (size_t)elem_bytes);
                        }
    free(recv);
    return ORC_OK;
}

/*
 * Bytes that sequence-shard rank `rank` sends to other ranks in one
 * seq->head exchange ([P1] section 4 "Communication Volume Compared with
 * Megatron SP": each rank keeps the piece addressed to itself and sends the
 * rest; [P2] section "DeepSpeed Attention costs").  Counted one element at a
 * time by asking where each element of the rank's shard goes.
 */
int64_t oracle_send_bytes(int64_t B, int64_t S, int64_t H, int64_t D, int32_t P,
                          int32_t elem_bytes, int32_t rank)
{
    if (check_layout(B, S, H, D, P, elem_bytes) != ORC_OK || rank < 0 || rank >= P)
        return -1;
    const int64_t Sp = S / P, hp = H / P;
    int64_t sent = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < Sp; ++t)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t dest = h / hp;
                    if (dest != rank)
                        sent += elem_bytes;
                }
    return sent;
}

/* Exact value of one stored input element. */
static double load_value(const void *base, int32_t dtype, int64_t idx)
{
    if (dtype == ORC_BF16) {
        /* bfloat16 is the upper half of an IEEE binary32 word. */
        uint16_t h;
        memcpy(&h, (const unsigned char *)base + idx * 2, 2);
        uint32_t w = (uint32_t)h << 16;
        float f;
        memcpy(&f, &w, 4);
        return (double)f;
    }
    if (dtype == ORC_F32) {
        float f;
        memcpy(&f, (const unsigned char *)base + idx * 4, 4);
        return (double)f;
    }
    double x;
    memcpy(&x, (const unsigned char *)base + idx * 8, 8);
    return x;
}

/*
 * One rank's local attention ([P1] section 2, fourth step: each rank now has
 * the whole sequence for its heads and computes their attention alone;
 * [P2] attention skeleton in the Introduction, which calls PyTorch's
 * scaled-dot-product attention with no scale, mask or dropout arguments,
 * i.e. softmax(Q K^T / sqrt(D)) V per head).
 *
 *   q, o: [B][S][Hq][D];  k, v: [B][S][Hkv][D]
 *   Query head c reads key/value head c / (Hq/Hkv) (grouped heads, [P2]
 *   skeleton: n_head query heads, n_kv_head key/value heads).
 *   Causal ([P1] section 8, the triangular pattern inside each head): query
 *   token i sees keys 0..i in global token order; otherwise keys 0..S-1.
 *
 * Each output row is computed in two passes over its visible keys:
 *   s_k = (sum_d q[i,d] k[k,d]) / sqrt(D);  m = max_k s_k
 *   p_k = exp(s_k - m);  l = sum_k p_k;     o[i,d] = (sum_k p_k v[k,d]) / l
 *
 * rows == NULL: all S rows, o is [B][S][Hq][D] (fp64).
 * rows != NULL: only the nrows listed token indices, o is [B][nrows][Hq][D].
 */
int oracle_attention(const void *q, const void *k, const void *v, int32_t dtype,
                     double *o, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                     int64_t D, int32_t causal, const int64_t *rows, int64_t nrows,
                     int32_t nthreads)
{
    if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || D < 1 ||
        (dtype != ORC_BF16 && dtype != ORC_F32 && dtype != ORC_F64))
        return ORC_BAD_ARG;
    if (Hq % Hkv != 0)
        return ORC_NOT_DIVISIBLE;
    const int64_t nr = rows ? nrows : S;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= S)
                return ORC_BAD_ARG;
    const int64_t group = Hq / Hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    const int64_t units = B * nr * Hq;
    int failed = 0;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!s || !acc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t u = 0; u < units; ++u) {
            if (!s || !acc)
                continue;
            const int64_t c = u % Hq;
            const int64_t r = (u / Hq) % nr;
            const int64_t b = u / (Hq * nr);
            const int64_t i = rows ? rows[r] : r;
            const int64_t ck = c / group;
            const int64_t last = causal ? i : S - 1;

            /* pass 1: scaled scores and their maximum */
            double m = -INFINITY;
            for (int64_t kk = 0; kk <= last; ++kk) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += load_value(q, dtype, ((b * S + i) * Hq + c) * D + d) *
                           load_value(k, dtype, ((b * S + kk) * Hkv + ck) * D + d);
                s[kk] = dot * inv_sqrt_d;
                if (s[kk] > m)
                    m = s[kk];
            }
            /* pass 2: exponentials, their sum and the weighted sum of values */
            double l = 0.0;
            for (int64_t d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (int64_t kk = 0; kk <= last; ++kk) {
                const double p = exp(s[kk] - m);
                l += p;
                for (int64_t d = 0; d < D; ++d)
                    acc[d] += p * load_value(v, dtype, ((b * S + kk) * Hkv + ck) * D + d);
            }
            for (int64_t d = 0; d < D; ++d)
                o[((b * nr + r) * Hq + c) * D + d] = acc[d] / l;
        }
        free(s);
        free(acc);
    }
    return failed ? ORC_NO_MEMORY : ORC_OK;
}

/*
 * Row log-sum-exp and gradients of one rank's local attention.  The pages say
 * that the backward pass runs the same layout changes in reverse ([P1]
 * section 6: the output gradient moves into the head-major layout, the Q, K
 * and V gradients back to the sequence-major layout; [P2] section "DeepSpeed
 * Attention costs": one inverse exchange per tensor).  Between them sits the
 * derivative of the local attention above, written out from its definition
 * (chain rule through O = P V and the row softmax P = softmax(S), S = Q K^T /
 * sqrt(D)); for each row i of query head c (key/value head c / (Hq/Hkv)):
 *
 *   lse_i   = m + log(l)                 (natural log of sum_k exp(s_k))
 *   p_k     = exp(s_k - lse_i)            (the softmax weights)
 *   o_i     = sum_k p_k v_k
 *   dP_k    = sum_d dO[i,d] v_k[d]
 *   delta_i = sum_d dO[i,d] o_i[d]        (= sum_k p_k dP_k)
 *   dS_k    = p_k (dP_k - delta_i)
 *   dQ[i]  += sum_k dS_k k_k / sqrt(D)
 *   dK[k]  += dS_k q_i / sqrt(D)          (summed over rows and over the
 *   dV[k]  += p_k dO[i]                    query heads that share the kv head)
 *
 * round_o != 0 takes delta from the output row rounded to bfloat16 (to
 * nearest, ties to even), the precision in which a bf16 forward hands its
 * output to the gradient step; 0 uses the exact row.
 *
 * dq: [B][S][Hq][D], dk, dv: [B][S][Hkv][D], lse: [B][Hq][S] (may be NULL),
 * all fp64.  Work is split over (batch, kv head) units, each of which owns
 * its dK/dV slice and the dQ rows of its query heads, so no two threads
 * write the same element and the order of every sum is fixed.
 */
/*
 * x rounded to the nearest bfloat16 value, ties to the one whose last stored
 * bit is zero (IEEE round to nearest even), returned as a double.  bfloat16
 * keeps 8 significant bits and the exponent range of binary32: normal numbers
 * are multiples of 2^(e-7) in [2^e, 2^(e+1)) for e >= -126, subnormals
 * multiples of 2^-133, and magnitudes from the midpoint between the largest
 * finite value (2 - 2^-7) * 2^127 and 2^128 upwards round to infinity.  The
 * double is rounded once, directly (no detour through binary32, which would
 * round twice).  NaN stays NaN.
 */
static double round_bf16(double x)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    int e;
    (void)frexp(x, &e);      /* |x| in [2^(e-1), 2^e) */
    int q = e - 1 - 7;       /* exponent of the spacing at |x| */
    if (q < -133)
        q = -133;            /* subnormal range: fixed spacing 2^-133 */
    /* nearbyint rounds to nearest, ties to even, in the default mode; the
     * scaling by a power of two is exact */
    const double r = ldexp(nearbyint(ldexp(x, -q)), q);
    if (fabs(r) >= 0x1p128)
        return x > 0 ? INFINITY : -INFINITY;
    return r;
}

/* Element-wise round_bf16 (exported so that it can be checked on its own). */
int oracle_round_bf16(const double *x, double *y, int64_t n)
{
    if (n < 0)
        return ORC_BAD_ARG;
    for (int64_t i = 0; i < n; ++i)
        y[i] = round_bf16(x[i]);
    return ORC_OK;
}

int oracle_attention_backward(const void *q, const void *k, const void *v, const void *dout,
                              int32_t dtype, double *dq, double *dk, double *dv, double *lse,
                              int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                              int32_t causal, int32_t round_o, int32_t nthreads)
{
    if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || D < 1 ||
        (dtype != ORC_BF16 && dtype != ORC_F32 && dtype != ORC_F64))
        return ORC_BAD_ARG;
    if (Hq % Hkv != 0)
        return ORC_NOT_DIVISIBLE;
    const int64_t group = Hq / Hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    const int64_t units = B * Hkv;
    memset(dq, 0, sizeof(double) * (size_t)(B * S * Hq * D));
    memset(dk, 0, sizeof(double) * (size_t)(B * S * Hkv * D));
    memset(dv, 0, sizeof(double) * (size_t)(B * S * Hkv * D));
    int failed = 0;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        if (!s || !o) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t u = 0; u < units; ++u) {
            if (!s || !o)
                continue;
            const int64_t b = u / Hkv, ck = u % Hkv;
            for (int64_t c = ck * group; c < (ck + 1) * group; ++c) {
                for (int64_t i = 0; i < S; ++i) {
                    const int64_t last = causal ? i : S - 1;
                    const int64_t qi = ((b * S + i) * Hq + c) * D;
                    /* scores, their maximum and the log-sum-exp */
                    double m = -INFINITY;
                    for (int64_t kk = 0; kk <= last; ++kk) {
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            dot += load_value(q, dtype, qi + d) *
                                   load_value(k, dtype, ((b * S + kk) * Hkv + ck) * D + d);
                        s[kk] = dot * inv_sqrt_d;
                        if (s[kk] > m)
                            m = s[kk];
                    }
                    double l = 0.0;
                    for (int64_t kk = 0; kk <= last; ++kk)
                        l += exp(s[kk] - m);
                    const double lse_i = m + log(l);
                    if (lse)
                        lse[(b * Hq + c) * S + i] = lse_i;
                    /* output row and delta */
                    for (int64_t d = 0; d < D; ++d)
                        o[d] = 0.0;
                    for (int64_t kk = 0; kk <= last; ++kk) {
                        const double p = exp(s[kk] - lse_i);
                        for (int64_t d = 0; d < D; ++d)
                            o[d] += p * load_value(v, dtype, ((b * S + kk) * Hkv + ck) * D + d);
                    }
                    double delta = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        delta += load_value(dout, dtype, qi + d) * (round_o ? round_bf16(o[d]) : o[d]);
                    /* gradients */
                    for (int64_t kk = 0; kk <= last; ++kk) {
                        const int64_t kj = ((b * S + kk) * Hkv + ck) * D;
                        const double p = exp(s[kk] - lse_i);
                        double dp = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            dp += load_value(dout, dtype, qi + d) * load_value(v, dtype, kj + d);
                        const double ds = p * (dp - delta);
                        for (int64_t d = 0; d < D; ++d) {
                            dq[qi + d] += ds * load_value(k, dtype, kj + d) * inv_sqrt_d;
                            dk[kj + d] += ds * load_value(q, dtype, qi + d) * inv_sqrt_d;
                            dv[kj + d] += p * load_value(dout, dtype, qi + d);
                        }
                    }
                }
            }
        }
        free(s);
        free(o);
    }
    return failed ? ORC_NO_MEMORY : ORC_OK;
}

/*
 * The same gradients on samples, for sizes where the full computation is too
 * slow: dQ at the listed rows, and dK, dV at the listed keys, with the same
 * per-row and per-pair steps as oracle_attention_backward:
 *   1. every row that is listed or sees a listed key: its scores, lse, output
 *      row and delta (as in the full computation);
 *   2. a listed row's dQ: the sum over its keys in increasing key order;
 *   3. a listed key's dK, dV: the sum over the query heads of its group in
 *      increasing order and, within a head, over the rows that see it in
 *      increasing row order -- the order of the full computation, so the
 *      listed elements equal its elements bit for bit.
 * With causal masking only rows i >= k see key k, so keys near the end of the
 * sequence are cheap; without it every row is needed.  Steps 1 and 2 split
 * rows among threads and step 3 keys; no two threads write one element.
 *
 * dq: [B][nrows][Hq][D], dk, dv: [B][nkeys][Hkv][D], fp64.
 */
int oracle_attention_backward_sampled(const void *q, const void *k, const void *v,
                                      const void *dout, int32_t dtype, const int64_t *rows,
                                      int64_t nrows, const int64_t *keys, int64_t nkeys,
                                      double *dq, double *dk, double *dv, int64_t B, int64_t S,
                                      int64_t Hq, int64_t Hkv, int64_t D, int32_t causal,
                                      int32_t round_o, int32_t nthreads)
{
    if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || D < 1 || nrows < 0 || nkeys < 0 ||
        (dtype != ORC_BF16 && dtype != ORC_F32 && dtype != ORC_F64))
        return ORC_BAD_ARG;
    if (Hq % Hkv != 0)
        return ORC_NOT_DIVISIBLE;
    int64_t kmin = S;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= S)
            return ORC_BAD_ARG;
    for (int64_t j = 0; j < nkeys; ++j) {
        if (keys[j] < 0 || keys[j] >= S)
            return ORC_BAD_ARG;
        if (keys[j] < kmin)
            kmin = keys[j];
    }
    const int64_t group = Hq / Hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    memset(dq, 0, sizeof(double) * (size_t)(B * nrows * Hq * D));
    memset(dk, 0, sizeof(double) * (size_t)(B * nkeys * Hkv * D));
    memset(dv, 0, sizeof(double) * (size_t)(B * nkeys * Hkv * D));
    /* first row that can see a listed key */
    const int64_t first = nkeys ? (causal ? kmin : 0) : S;
    /* per (batch, query head, row): lse and delta of the rows step 1 computes */
    double *lse = (double *)malloc(sizeof(double) * (size_t)(B * Hq * S > 0 ? B * Hq * S : 1));
    double *dlt = (double *)malloc(sizeof(double) * (size_t)(B * Hq * S > 0 ? B * Hq * S : 1));
    int64_t *row_slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(S > 0 ? S : 1));
    if (!lse || !dlt || !row_slot) {
        free(lse);
        free(dlt);
        free(row_slot);
        return ORC_NO_MEMORY;
    }
    /* slot of each token in the row list (-1: not listed; the last listing of a
     * repeated index wins) */
    for (int64_t i = 0; i < S; ++i)
        row_slot[i] = -1;
    for (int64_t r = 0; r < nrows; ++r)
        row_slot[rows[r]] = r;
    int failed = 0;
    const int64_t runits = B * Hq * S;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        if (!s || !o) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
        /* steps 1 and 2, one (batch, query head, row) at a time */
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 64)
#endif
        for (int64_t u = 0; u < runits; ++u) {
            if (!s || !o)
                continue;
            const int64_t i = u % S, c = (u / S) % Hq, b = u / (S * Hq);
            const int64_t rslot = row_slot[i];
            if (rslot < 0 && i < first)
                continue;
            const int64_t ck = c / group;
            const int64_t last = causal ? i : S - 1;
            const int64_t qi = ((b * S + i) * Hq + c) * D;
            double m = -INFINITY;
            for (int64_t kk = 0; kk <= last; ++kk) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += load_value(q, dtype, qi + d) *
                           load_value(k, dtype, ((b * S + kk) * Hkv + ck) * D + d);
                s[kk] = dot * inv_sqrt_d;
                if (s[kk] > m)
                    m = s[kk];
            }
            double l = 0.0;
            for (int64_t kk = 0; kk <= last; ++kk)
                l += exp(s[kk] - m);
            const double lse_i = m + log(l);
            for (int64_t d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int64_t kk = 0; kk <= last; ++kk) {
                const double p = exp(s[kk] - lse_i);
                for (int64_t d = 0; d < D; ++d)
                    o[d] += p * load_value(v, dtype, ((b * S + kk) * Hkv + ck) * D + d);
            }
            double delta = 0.0;
            for (int64_t d = 0; d < D; ++d)
                delta += load_value(dout, dtype, qi + d) * (round_o ? round_bf16(o[d]) : o[d]);
            lse[(b * Hq + c) * S + i] = lse_i;
            dlt[(b * Hq + c) * S + i] = delta;
            if (rslot < 0)
                continue;
            for (int64_t kk = 0; kk <= last; ++kk) {
                const int64_t kj = ((b * S + kk) * Hkv + ck) * D;
                const double p = exp(s[kk] - lse_i);
                double dp = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dp += load_value(dout, dtype, qi + d) * load_value(v, dtype, kj + d);
                const double ds = p * (dp - delta);
                for (int64_t d = 0; d < D; ++d)
                    dq[((b * nrows + rslot) * Hq + c) * D + d] +=
                        ds * load_value(k, dtype, kj + d) * inv_sqrt_d;
            }
        }
        /* step 3, one (batch, listed key) at a time, every kv head */
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t u = 0; u < B * nkeys; ++u) {
            const int64_t j = u % nkeys, b = u / nkeys, kk = keys[j];
            for (int64_t ck = 0; ck < Hkv; ++ck) {
                const int64_t kj = ((b * S + kk) * Hkv + ck) * D;
                double *dkj = dk + ((b * nkeys + j) * Hkv + ck) * D;
                double *dvj = dv + ((b * nkeys + j) * Hkv + ck) * D;
                for (int64_t c = ck * group; c < (ck + 1) * group; ++c)
                    for (int64_t i = causal ? kk : 0; i < S; ++i) {
                        const int64_t qi = ((b * S + i) * Hq + c) * D;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            dot += load_value(q, dtype, qi + d) * load_value(k, dtype, kj + d);
                        const double p = exp(dot * inv_sqrt_d - lse[(b * Hq + c) * S + i]);
                        double dp = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            dp += load_value(dout, dtype, qi + d) * load_value(v, dtype, kj + d);
                        const double ds = p * (dp - dlt[(b * Hq + c) * S + i]);
                        for (int64_t d = 0; d < D; ++d) {
                            dkj[d] += ds * load_value(q, dtype, qi + d) * inv_sqrt_d;
                            dvj[d] += p * load_value(dout, dtype, qi + d);
                        }
                    }
            }
        }
        free(s);
        free(o);
    }
    free(lse);
    free(dlt);
    free(row_slot);
    return failed ? ORC_NO_MEMORY : ORC_OK;
}
