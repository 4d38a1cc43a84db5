// C ABI of libulysses.so (declared in include/ulysses.h): argument checks,
// error reporting and kernel dispatch.  Every precondition is checked before
// anything is enqueued; the library allocates nothing and keeps no state
// besides a per-thread error string.
#include "../../include/ulysses.h"
#include "internal.h"

#include <cstdarg>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_last_error;

uly_status_t fail(uly_status_t s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

uly_status_t ok() {
    g_last_error.clear();
    return ULY_OK;
}

int elem_bytes(uly_dtype_t dt) {
    switch (dt) {
        case ULY_DTYPE_BF16: return 2;
        case ULY_DTYPE_FP32: return 4;
        default: return 0;
    }
}

// true if [a, a+na) and [b, b+nb) share a byte
bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

bool aligned(const void *p, uint64_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// n1*n2*... with overflow detection against 2^62
bool mul_ok(uint64_t &acc, int64_t f) {
    if (f < 0) return false;
    if (f && acc > (uint64_t(1) << 62) / uint64_t(f)) return false;
    acc *= uint64_t(f);
    return true;
}

// Checks of one layout change; bytes = the tensor size (0: nothing to do).
uly_status_t layout_check(const char *name, const void *src, const void *dst, int64_t B,
                          int64_t S, int64_t H, int64_t D, int32_t P, uly_dtype_t dtype,
                          uint64_t &bytes) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", name, int(dtype));
    if (B < 0 || S < 0) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: negative B or S", name);
    if (H < 1 || D < 1 || P < 1)
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: n_heads, head_dim and P must be >= 1", name);
    if (P > H)
        return fail(ULY_ERR_NOT_DIVISIBLE, "%s: P=%d exceeds n_heads=%lld (head-count bound)",
                    name, P, (long long)H);
    if (H % P)
        return fail(ULY_ERR_NOT_DIVISIBLE, "%s: n_heads=%lld not divisible by P=%d", name,
                    (long long)H, P);
    if (S % P)
        return fail(ULY_ERR_NOT_DIVISIBLE, "%s: S=%lld not divisible by P=%d", name,
                    (long long)S, P);
    bytes = uint64_t(e);
    if (!mul_ok(bytes, B) || !mul_ok(bytes, S) || !mul_ok(bytes, H) || !mul_ok(bytes, D))
        return fail(ULY_ERR_UNSUPPORTED, "%s: tensor too large", name);
    if (bytes == 0) return ULY_OK;
    if (!src || !dst) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL pointer", name);
    if (!aligned(src, e) || !aligned(dst, e))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: pointers must be %d-byte aligned", name, e);
    if (overlap(src, bytes, dst, bytes))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: source and destination overlap", name);
    if (int64_t(P) * B > 65535)
        return fail(ULY_ERR_UNSUPPORTED, "%s: P*B=%lld exceeds 65535", name,
                    (long long)(int64_t(P) * B));
    // the kernel indexes one (rank, batch) slice with 32-bit arithmetic at the
    // narrowest vector width it may pick (the element size)
    if (uint64_t(S) * uint64_t(H / P) * uint64_t(D) >= (uint64_t(1) << 32))
        return fail(ULY_ERR_UNSUPPORTED, "%s: one (rank, batch) slice exceeds 2^32 elements", name);
    return ULY_OK;
}

uly_status_t layout(const char *name, const void *src, void *dst, int64_t B, int64_t S,
                    int64_t H, int64_t D, int32_t P, uly_dtype_t dtype, void *stream,
                    bool to_head, bool pieces) {
    uint64_t bytes = 0;
    uly_status_t st = layout_check(name, src, dst, B, S, H, D, P, dtype, bytes);
    if (st != ULY_OK) return st;
    if (bytes == 0) return ok();
    hipError_t err = uly::launch_layout(src, dst, B, S, H, D, P, elem_bytes(dtype), to_head,
                                        pieces, static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

// Shape checks shared by the attention calls; byte sizes of q/o and of k/v.
uly_status_t attention_shape(const char *name, int64_t B, int64_t S, int64_t n_q_heads,
                             int64_t n_kv_heads, int64_t head_dim, uly_dtype_t dtype,
                             uint64_t &qbytes, uint64_t &kbytes) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", name, int(dtype));
    if (B < 0 || S < 0) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: negative B or S", name);
    if (n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1)
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: head counts and head_dim must be >= 1", name);
    if (n_q_heads % n_kv_heads)
        return fail(ULY_ERR_NOT_DIVISIBLE, "%s: n_q_heads=%lld not divisible by n_kv_heads=%lld",
                    name, (long long)n_q_heads, (long long)n_kv_heads);
    const bool bf16_ok = dtype == ULY_DTYPE_BF16 && head_dim == 128;
    const bool f32_ok = dtype == ULY_DTYPE_FP32 &&
                        (head_dim == 32 || head_dim == 64 || head_dim == 128);
    if (!bf16_ok && !f32_ok)
        return fail(ULY_ERR_UNSUPPORTED, "%s: no kernel for dtype %d with head_dim %lld", name,
                    int(dtype), (long long)head_dim);
    uint64_t bh = 1;  // B * n_q_heads, formed only once it cannot overflow
    if (S >= (int64_t(1) << 31) || !mul_ok(bh, B) || !mul_ok(bh, n_q_heads) ||
        bh >= (uint64_t(1) << 31))
        return fail(ULY_ERR_UNSUPPORTED, "%s: S or B*n_q_heads too large", name);
    // the bf16 kernels address a 64-row tile with 32-bit lane offsets
    if (bf16_ok && n_kv_heads > 65536)
        return fail(ULY_ERR_UNSUPPORTED, "%s: n_kv_heads=%lld exceeds 65536 for bf16", name,
                    (long long)n_kv_heads);
    qbytes = uint64_t(e);
    kbytes = uint64_t(e);
    if (!mul_ok(qbytes, B) || !mul_ok(qbytes, S) || !mul_ok(qbytes, n_q_heads) ||
        !mul_ok(qbytes, head_dim) || !mul_ok(kbytes, B) || !mul_ok(kbytes, S) ||
        !mul_ok(kbytes, n_kv_heads) || !mul_ok(kbytes, head_dim))
        return fail(ULY_ERR_UNSUPPORTED, "%s: tensor too large", name);
    const int64_t blocks = ((S + 63) / 64) * B * n_q_heads;  // bound for any block size >= 64
    if (qbytes && blocks >= (int64_t(1) << 31))
        return fail(ULY_ERR_UNSUPPORTED, "%s: too many query blocks", name);
    return ULY_OK;
}

// P = 0: q, k, v, o in [B][S][h][D]; P >= 1: in P pieces [P][B][S/P][h][D].
uly_status_t attention_fwd(const char *name, const void *q, const void *k, const void *v, void *o,
                           float *lse, int64_t B, int64_t S, int64_t n_q_heads, int64_t n_kv_heads,
                           int64_t head_dim, int32_t P, int32_t causal, uly_dtype_t dtype,
                           void *stream) {
    uint64_t qbytes = 0, kbytes = 0;
    uly_status_t st = attention_shape(name, B, S, n_q_heads, n_kv_heads, head_dim, dtype, qbytes,
                                      kbytes);
    if (st != ULY_OK) return st;
    if (P < 0) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: P must be >= 1", name);
    if (P && S % P)
        return fail(ULY_ERR_NOT_DIVISIBLE, "%s: S=%lld not divisible by P=%d", name,
                    (long long)S, P);
    // a bf16 key tile (64 rows) must not straddle two pieces
    if (P && B > 1 && dtype == ULY_DTYPE_BF16 && (S / P) % 64)
        return fail(ULY_ERR_UNSUPPORTED, "%s: bf16 with B > 1 needs S/P a multiple of 64 (S/P=%lld)",
                    name, (long long)(S / P));
    if (qbytes == 0) return ok();
    if (!q || !k || !v || !o) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL pointer", name);
    const int al = dtype == ULY_DTYPE_BF16 ? 16 : 4;
    if (!aligned(q, al) || !aligned(k, al) || !aligned(v, al) || !aligned(o, al))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: pointers must be %d-byte aligned", name, al);
    if (lse && !aligned(lse, 4))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: lse must be 4-byte aligned", name);
    if (overlap(o, qbytes, q, qbytes) || overlap(o, qbytes, k, kbytes) ||
        overlap(o, qbytes, v, kbytes))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: output overlaps an input", name);
    const uint64_t lbytes = uint64_t(B) * uint64_t(S) * uint64_t(n_q_heads) * 4;
    if (lse && (overlap(lse, lbytes, q, qbytes) || overlap(lse, lbytes, k, kbytes) ||
                overlap(lse, lbytes, v, kbytes) || overlap(lse, lbytes, o, qbytes)))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: lse overlaps another tensor", name);
    hipStream_t st_ = static_cast<hipStream_t>(stream);
    const bool bf16 = dtype == ULY_DTYPE_BF16;
    const int64_t sp = P ? S / P : 0;
    hipError_t err =
        bf16 ? uly::launch_attention_bf16_d128(q, k, v, o, lse, B, S, n_q_heads, n_kv_heads, sp,
                                               causal != 0, st_)
             : uly::launch_attention_f32(static_cast<const float *>(q),
                                         static_cast<const float *>(k),
                                         static_cast<const float *>(v), static_cast<float *>(o),
                                         lse, B, S, n_q_heads, n_kv_heads, head_dim, sp,
                                         causal != 0, st_);
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

uly_status_t attention_chunk(const char *name, const void *q, const void *k, const void *v, void *o,
                             float *lse, int64_t B, int64_t Sq, int64_t Skv, int64_t n_q_heads,
                             int64_t n_kv_heads, int64_t head_dim, int64_t q_pos0, int64_t k_pos0,
                             int32_t causal, uly_dtype_t dtype, bool accumulate, void *stream) {
    uint64_t qbytes = 0, kbytes = 0, unused = 0;
    uly_status_t st = attention_shape(name, B, Sq, n_q_heads, n_kv_heads, head_dim, dtype, qbytes,
                                      unused);
    if (st != ULY_OK) return st;
    if (accumulate && (dtype != ULY_DTYPE_BF16 || head_dim != 128))
        return fail(ULY_ERR_UNSUPPORTED, "%s: needs ULY_DTYPE_BF16 with head_dim 128", name);
    st = attention_shape(name, B, Skv, n_q_heads, n_kv_heads, head_dim, dtype, unused, kbytes);
    if (st != ULY_OK) return st;
    // block offsets plus the diagonal offset stay inside 32-bit arithmetic
    if (Sq >= (int64_t(1) << 30) || Skv >= (int64_t(1) << 30))
        return fail(ULY_ERR_UNSUPPORTED, "%s: Sq and Skv must be below 2^30", name);
    const int64_t kPosMax = int64_t(1) << 62;
    if (q_pos0 < -kPosMax || q_pos0 > kPosMax || k_pos0 < -kPosMax || k_pos0 > kPosMax)
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: positions beyond +-2^62", name);
    if (qbytes == 0) return ok();
    if (!q || !o || !lse || (kbytes && (!k || !v)))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL pointer", name);
    const int al = dtype == ULY_DTYPE_BF16 ? 16 : 4;
    if (!aligned(q, al) || !aligned(k, al) || !aligned(v, al) || !aligned(o, al) || !aligned(lse, 4))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: tensors must be %d-byte aligned, lse 4-byte", name,
                    al);
    const uint64_t lbytes = uint64_t(B) * uint64_t(Sq) * uint64_t(n_q_heads) * 4;
    if (overlap(o, qbytes, q, qbytes) || overlap(o, qbytes, k, kbytes) ||
        overlap(o, qbytes, v, kbytes))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: output overlaps an input", name);
    if (overlap(lse, lbytes, q, qbytes) || overlap(lse, lbytes, k, kbytes) ||
        overlap(lse, lbytes, v, kbytes) || overlap(lse, lbytes, o, qbytes))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: lse overlaps another tensor", name);
    // key j visible to row i iff k_pos0 + j <= q_pos0 + i, i.e. j <= i + delta;
    // beyond [-Sq, Skv] every row sees no key / every key
    int64_t delta = q_pos0 - k_pos0;
    delta = delta < -Sq ? -Sq : (delta > Skv ? Skv : delta);
    hipStream_t st_ = static_cast<hipStream_t>(stream);
    hipError_t err =
        dtype == ULY_DTYPE_BF16
            ? uly::launch_attention_chunk_bf16_d128(q, k, v, o, lse, B, Sq, Skv, delta, n_q_heads,
                                                    n_kv_heads, causal != 0, accumulate, st_)
            : uly::launch_attention_chunk_f32(static_cast<const float *>(q),
                                              static_cast<const float *>(k),
                                              static_cast<const float *>(v), static_cast<float *>(o),
                                              lse, B, Sq, Skv, delta, n_q_heads, n_kv_heads,
                                              head_dim, causal != 0, st_);
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

// Checks of the gradient calls (with the caller's delta workspace when
// has_delta); empty is set when there is nothing to do.
uly_status_t backward_checks(const char *name, const void *q, const void *k, const void *v,
                             const void *o, const void *dout, const float *lse, float *delta,
                             void *dq, void *dk, void *dv, int64_t B, int64_t S, int64_t n_q_heads,
                             int64_t n_kv_heads, int64_t head_dim, uly_dtype_t dtype,
                             bool has_delta, bool &empty) {
    uint64_t qbytes = 0, kbytes = 0;
    uly_status_t st = attention_shape(name, B, S, n_q_heads, n_kv_heads, head_dim, dtype, qbytes,
                                      kbytes);
    if (st != ULY_OK) return st;
    if (dtype != ULY_DTYPE_BF16 || head_dim != 128)
        return fail(ULY_ERR_UNSUPPORTED, "%s: gradients need ULY_DTYPE_BF16 with head_dim 128", name);
    if (n_q_heads > 65536)
        return fail(ULY_ERR_UNSUPPORTED, "%s: n_q_heads=%lld exceeds 65536", name,
                    (long long)n_q_heads);
    empty = qbytes == 0;
    if (empty) return ok();
    const uint64_t fbytes = uint64_t(B) * uint64_t(S) * uint64_t(n_q_heads) * 4;
    if (!q || !k || !v || !o || !dout || !lse || (has_delta && !delta) || !dq || !dk || !dv)
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL pointer", name);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(lse, 4) || !aligned(delta, 4))
        return fail(ULY_ERR_INVALID_ARGUMENT,
                    "%s: tensors must be 16-byte aligned, lse and delta 4-byte aligned", name);
    const void *in[6] = {q, k, v, o, dout, lse};
    const uint64_t inb[6] = {qbytes, kbytes, kbytes, qbytes, qbytes, fbytes};
    void *out[4] = {dq, dk, dv, delta};
    const uint64_t outb[4] = {qbytes, kbytes, kbytes, has_delta ? fbytes : 0};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(out[i], outb[i], in[j], inb[j]))
                return fail(ULY_ERR_INVALID_ARGUMENT, "%s: an output overlaps an input", name);
        for (int j = i + 1; j < 4; ++j)
            if (overlap(out[i], outb[i], out[j], outb[j]))
                return fail(ULY_ERR_INVALID_ARGUMENT, "%s: two outputs overlap", name);
    }
    return ULY_OK;
}

// seq->head (pieces: seq->pieces) of Q, K and V in one launch
uly_status_t layout_qkv(const char *name, const void *q_seq, const void *k_seq, const void *v_seq,
                        void *q_head, void *k_head, void *v_head, int64_t B, int64_t S,
                        int64_t n_q_heads, int64_t n_kv_heads, int64_t head_dim, int32_t P,
                        uly_dtype_t dtype, void *stream, bool pieces) {
    const void *src[3] = {q_seq, k_seq, v_seq};
    void *dst[3] = {q_head, k_head, v_head};
    uint64_t bytes[3] = {0, 0, 0};
    for (int x = 0; x < 3; ++x) {
        uly_status_t st = layout_check(name, src[x], dst[x], B, S, x == 0 ? n_q_heads : n_kv_heads,
                                       head_dim, P, dtype, bytes[x]);
        if (st != ULY_OK) return st;
    }
    if (bytes[0] == 0) return ok();
    for (int x = 0; x < 3; ++x)
        for (int y = 0; y < 3; ++y) {
            if (overlap(dst[x], bytes[x], src[y], bytes[y]))
                return fail(ULY_ERR_INVALID_ARGUMENT, "%s: a destination overlaps a source", name);
            if (y > x && overlap(dst[x], bytes[x], dst[y], bytes[y]))
                return fail(ULY_ERR_INVALID_ARGUMENT, "%s: two destinations overlap", name);
        }
    hipError_t err = uly::launch_layout_qkv(src, dst, B, S, n_q_heads, n_kv_heads, head_dim, P,
                                            elem_bytes(dtype), pieces,
                                            static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

}  // namespace

extern "C" {

uly_status_t ulysses_seq_to_head(const void *seq_shards, void *head_shards, int64_t B,
                                 int64_t S, int64_t n_heads, int64_t head_dim, int32_t P,
                                 uly_dtype_t dtype, void *stream) {
    return layout("ulysses_seq_to_head", seq_shards, head_shards, B, S, n_heads, head_dim, P,
                  dtype, stream, true, false);
}

uly_status_t ulysses_seq_to_head_qkv(const void *q_seq, const void *k_seq, const void *v_seq,
                                     void *q_head, void *k_head, void *v_head, int64_t B,
                                     int64_t S, int64_t n_q_heads, int64_t n_kv_heads,
                                     int64_t head_dim, int32_t P, uly_dtype_t dtype,
                                     void *stream) {
    return layout_qkv("ulysses_seq_to_head_qkv", q_seq, k_seq, v_seq, q_head, k_head, v_head, B,
                      S, n_q_heads, n_kv_heads, head_dim, P, dtype, stream, false);
}

uly_status_t ulysses_head_to_seq(const void *head_shards, void *seq_shards, int64_t B,
                                 int64_t S, int64_t n_heads, int64_t head_dim, int32_t P,
                                 uly_dtype_t dtype, void *stream) {
    return layout("ulysses_head_to_seq", head_shards, seq_shards, B, S, n_heads, head_dim, P,
                  dtype, stream, false, false);
}

uly_status_t ulysses_attention_local(const void *q, const void *k, const void *v, void *o,
                                     int64_t B, int64_t S, int64_t n_q_heads,
                                     int64_t n_kv_heads, int64_t head_dim, int32_t causal,
                                     uly_dtype_t dtype, void *stream) {
    return attention_fwd("ulysses_attention_local", q, k, v, o, nullptr, B, S, n_q_heads,
                         n_kv_heads, head_dim, 0, causal, dtype, stream);
}

uly_status_t ulysses_attention_local_lse(const void *q, const void *k, const void *v, void *o,
                                         float *lse, int64_t B, int64_t S, int64_t n_q_heads,
                                         int64_t n_kv_heads, int64_t head_dim, int32_t causal,
                                         uly_dtype_t dtype, void *stream) {
    const char *name = "ulysses_attention_local_lse";
    if (B > 0 && S > 0 && !lse) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL lse", name);
    return attention_fwd(name, q, k, v, o, lse, B, S, n_q_heads, n_kv_heads, head_dim, 0, causal,
                         dtype, stream);
}

uly_status_t ulysses_attention_local_split_workspace(int64_t B, int64_t S, int64_t n_q_heads,
                                                    int64_t head_dim, int32_t causal,
                                                    uly_dtype_t dtype, uint64_t *bytes) {
    const char *name = "ulysses_attention_local_split_workspace";
    if (!bytes) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL bytes", name);
    *bytes = 0;
    uint64_t qbytes = 0, kbytes = 0;
    uly_status_t st = attention_shape(name, B, S, n_q_heads, 1, head_dim, dtype, qbytes, kbytes);
    if (st != ULY_OK) return st;
    if (dtype != ULY_DTYPE_BF16 || head_dim != 128)
        return fail(ULY_ERR_UNSUPPORTED, "%s: needs ULY_DTYPE_BF16 with head_dim 128", name);
    if (B * n_q_heads > 65535)
        return fail(ULY_ERR_UNSUPPORTED, "%s: B*n_q_heads=%lld exceeds 65535", name,
                    (long long)(B * n_q_heads));
    if (qbytes) *bytes = uly::attention_bf16_d128_split_workspace(B, S, n_q_heads, causal != 0);
    return ok();
}

uly_status_t ulysses_attention_local_split(const void *q, const void *k, const void *v, void *o,
                                           float *lse, int64_t B, int64_t S, int64_t n_q_heads,
                                           int64_t n_kv_heads, int64_t head_dim, int32_t causal,
                                           uly_dtype_t dtype, void *workspace,
                                           uint64_t workspace_bytes, void *stream) {
    const char *name = "ulysses_attention_local_split";
    uint64_t qbytes = 0, kbytes = 0;
    uly_status_t st = attention_shape(name, B, S, n_q_heads, n_kv_heads, head_dim, dtype, qbytes,
                                      kbytes);
    if (st != ULY_OK) return st;
    if (dtype != ULY_DTYPE_BF16 || head_dim != 128)
        return fail(ULY_ERR_UNSUPPORTED, "%s: needs ULY_DTYPE_BF16 with head_dim 128", name);
    // the merge's grid is (query blocks, B * n_q_heads); the unit grid at most 512 times that
    if (B * n_q_heads > 65535)
        return fail(ULY_ERR_UNSUPPORTED, "%s: B*n_q_heads=%lld exceeds 65535", name,
                    (long long)(B * n_q_heads));
    if (qbytes == 0) return ok();
    if (!q || !k || !v || !o) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL pointer", name);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        (lse && !aligned(lse, 4)))
        return fail(ULY_ERR_INVALID_ARGUMENT,
                    "%s: tensors must be 16-byte aligned, lse 4-byte aligned", name);
    const uint64_t lbytes = lse ? uint64_t(B) * uint64_t(S) * uint64_t(n_q_heads) * 4 : 0;
    if (overlap(o, qbytes, q, qbytes) || overlap(o, qbytes, k, kbytes) ||
        overlap(o, qbytes, v, kbytes))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: output overlaps an input", name);
    if (overlap(lse, lbytes, q, qbytes) || overlap(lse, lbytes, k, kbytes) ||
        overlap(lse, lbytes, v, kbytes) || overlap(lse, lbytes, o, qbytes))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: lse overlaps another tensor", name);
    const uint64_t need = uly::attention_bf16_d128_split_workspace(B, S, n_q_heads, causal != 0);
    if (need) {
        if (!workspace || workspace_bytes < need)
            return fail(ULY_ERR_INVALID_ARGUMENT, "%s: workspace of %llu bytes needed, %llu given",
                        name, (unsigned long long)need,
                        (unsigned long long)(workspace ? workspace_bytes : 0));
        if (!aligned(workspace, 16))
            return fail(ULY_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", name);
        const void *t[5] = {q, k, v, o, lse};
        const uint64_t tb[5] = {qbytes, kbytes, kbytes, qbytes, lbytes};
        for (int i = 0; i < 5; ++i)
            if (overlap(workspace, need, t[i], tb[i]))
                return fail(ULY_ERR_INVALID_ARGUMENT, "%s: workspace overlaps a tensor", name);
    }
    hipError_t err = uly::launch_attention_bf16_d128_split(q, k, v, o, lse, B, S, n_q_heads,
                                                           n_kv_heads, causal != 0, workspace,
                                                           static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

uly_status_t ulysses_seq_to_pieces(const void *seq_shards, void *pieces, int64_t B, int64_t S,
                                   int64_t n_heads, int64_t head_dim, int32_t P, uly_dtype_t dtype,
                                   void *stream) {
    return layout("ulysses_seq_to_pieces", seq_shards, pieces, B, S, n_heads, head_dim, P, dtype,
                  stream, true, true);
}

uly_status_t ulysses_seq_to_pieces_qkv(const void *q_seq, const void *k_seq, const void *v_seq,
                                       void *q_pieces, void *k_pieces, void *v_pieces, int64_t B,
                                       int64_t S, int64_t n_q_heads, int64_t n_kv_heads,
                                       int64_t head_dim, int32_t P, uly_dtype_t dtype,
                                       void *stream) {
    return layout_qkv("ulysses_seq_to_pieces_qkv", q_seq, k_seq, v_seq, q_pieces, k_pieces,
                      v_pieces, B, S, n_q_heads, n_kv_heads, head_dim, P, dtype, stream, true);
}

uly_status_t ulysses_pieces_to_seq(const void *pieces, void *seq_shards, int64_t B, int64_t S,
                                   int64_t n_heads, int64_t head_dim, int32_t P, uly_dtype_t dtype,
                                   void *stream) {
    return layout("ulysses_pieces_to_seq", pieces, seq_shards, B, S, n_heads, head_dim, P, dtype,
                  stream, false, true);
}

uly_status_t ulysses_attention_local_pieces(const void *q, const void *k, const void *v, void *o,
                                            float *lse, int64_t B, int64_t S, int64_t n_q_heads,
                                            int64_t n_kv_heads, int64_t head_dim, int32_t P,
                                            int32_t causal, uly_dtype_t dtype, void *stream) {
    const char *name = "ulysses_attention_local_pieces";
    if (P < 1) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: P must be >= 1", name);
    return attention_fwd(name, q, k, v, o, lse, B, S, n_q_heads, n_kv_heads, head_dim, P, causal,
                         dtype, stream);
}

uly_status_t ulysses_attention_local_backward(const void *q, const void *k, const void *v,
                                              const void *o, const void *dout, const float *lse,
                                              float *delta, void *dq, void *dk, void *dv,
                                              int64_t B, int64_t S, int64_t n_q_heads,
                                              int64_t n_kv_heads, int64_t head_dim,
                                              int32_t causal, uly_dtype_t dtype, void *stream) {
    const char *name = "ulysses_attention_local_backward";
    bool empty = false;
    uly_status_t st = backward_checks(name, q, k, v, o, dout, lse, delta, dq, dk, dv, B, S,
                                      n_q_heads, n_kv_heads, head_dim, dtype, true, empty);
    if (st != ULY_OK || empty) return st;
    hipError_t err = uly::launch_attention_bwd_bf16_d128(q, k, v, o, dout, lse, delta, dq, dk, dv,
                                                         B, S, n_q_heads, n_kv_heads, 0, causal != 0,
                                                         static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

uly_status_t ulysses_attention_local_backward_split_workspace(int64_t B, int64_t S,
                                                             int64_t n_q_heads, int64_t n_kv_heads,
                                                             int64_t head_dim, int32_t causal,
                                                             uly_dtype_t dtype, uint64_t *bytes) {
    const char *name = "ulysses_attention_local_backward_split_workspace";
    if (!bytes) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL bytes", name);
    *bytes = 0;
    uint64_t qbytes = 0, kbytes = 0;
    uly_status_t st = attention_shape(name, B, S, n_q_heads, n_kv_heads, head_dim, dtype, qbytes,
                                      kbytes);
    if (st != ULY_OK) return st;
    if (dtype != ULY_DTYPE_BF16 || head_dim != 128)
        return fail(ULY_ERR_UNSUPPORTED, "%s: needs ULY_DTYPE_BF16 with head_dim 128", name);
    if (qbytes)
        *bytes = uly::attention_bwd_bf16_d128_split_workspace(B, S, n_q_heads, n_kv_heads, causal != 0);
    return ok();
}

uly_status_t ulysses_attention_local_backward_split(
    const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
    float *delta, void *dq, void *dk, void *dv, int64_t B, int64_t S, int64_t n_q_heads,
    int64_t n_kv_heads, int64_t head_dim, int32_t causal, uly_dtype_t dtype, void *workspace,
    uint64_t workspace_bytes, void *stream) {
    const char *name = "ulysses_attention_local_backward_split";
    bool empty = false;
    uly_status_t st = backward_checks(name, q, k, v, o, dout, lse, delta, dq, dk, dv, B, S,
                                      n_q_heads, n_kv_heads, head_dim, dtype, true, empty);
    if (st != ULY_OK || empty) return st;
    const uint64_t need =
        uly::attention_bwd_bf16_d128_split_workspace(B, S, n_q_heads, n_kv_heads, causal != 0);
    if (need) {
        if (!workspace || workspace_bytes < need)
            return fail(ULY_ERR_INVALID_ARGUMENT, "%s: workspace of %llu bytes needed, %llu given",
                        name, (unsigned long long)need,
                        (unsigned long long)(workspace ? workspace_bytes : 0));
        if (!aligned(workspace, 256))
            return fail(ULY_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", name);
        const uint64_t qb = uint64_t(B) * uint64_t(S) * uint64_t(n_q_heads) * 256;
        const uint64_t kb = uint64_t(B) * uint64_t(S) * uint64_t(n_kv_heads) * 256;
        const uint64_t lb = uint64_t(B) * uint64_t(S) * uint64_t(n_q_heads) * 4;
        const void *t[11] = {q, k, v, o, dout, lse, delta, dq, dk, dv, nullptr};
        const uint64_t tb[10] = {qb, kb, kb, qb, qb, lb, lb, qb, kb, kb};
        for (int i = 0; i < 10; ++i)
            if (overlap(workspace, need, t[i], tb[i]))
                return fail(ULY_ERR_INVALID_ARGUMENT, "%s: workspace overlaps a tensor", name);
    }
    hipError_t err = uly::launch_attention_bwd_bf16_d128_split(
        q, k, v, o, dout, lse, delta, dq, dk, dv, B, S, n_q_heads, n_kv_heads, causal != 0,
        need ? workspace : nullptr, static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

uly_status_t ulysses_attention_local_backward_noalloc(const void *q, const void *k, const void *v,
                                                      const void *o, const void *dout,
                                                      const float *lse, void *dq, void *dk,
                                                      void *dv, int64_t B, int64_t S,
                                                      int64_t n_q_heads, int64_t n_kv_heads,
                                                      int64_t head_dim, int32_t causal,
                                                      uly_dtype_t dtype, void *stream) {
    const char *name = "ulysses_attention_local_backward_noalloc";
    bool empty = false;
    uly_status_t st = backward_checks(name, q, k, v, o, dout, lse, nullptr, dq, dk, dv, B, S,
                                      n_q_heads, n_kv_heads, head_dim, dtype, false, empty);
    if (st != ULY_OK || empty) return st;
    // delta ([B][n_q_heads][S] floats) lives in the GPU's scratch array
    if (uint64_t(B) * uint64_t(n_q_heads) * uint64_t(S) > uint64_t(uly::kScratchFloats))
        return fail(ULY_ERR_UNSUPPORTED,
                    "%s: B*n_q_heads*S = %lld exceeds the %lld rows of the library's scratch", name,
                    (long long)(B * n_q_heads * S), (long long)uly::kScratchFloats);
    float *delta = nullptr;
    hipError_t err = uly::scratch_floats(stream, &delta);
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: scratch lookup failed: %s", name, hipGetErrorString(err));
    err = uly::launch_attention_bwd_bf16_d128(q, k, v, o, dout, lse, delta, dq, dk, dv, B, S,
                                              n_q_heads, n_kv_heads, 0, causal != 0,
                                              static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

uly_status_t ulysses_attention_local_backward_pieces(
    const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
    float *delta, void *dq, void *dk, void *dv, int64_t B, int64_t S, int64_t n_q_heads,
    int64_t n_kv_heads, int64_t head_dim, int32_t P, int32_t causal, uly_dtype_t dtype,
    void *stream) {
    const char *name = "ulysses_attention_local_backward_pieces";
    bool empty = false;
    uly_status_t st = backward_checks(name, q, k, v, o, dout, lse, delta, dq, dk, dv, B, S,
                                      n_q_heads, n_kv_heads, head_dim, dtype, true, empty);
    if (st != ULY_OK) return st;
    if (P < 1) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: P must be >= 1", name);
    if (S % P)
        return fail(ULY_ERR_NOT_DIVISIBLE, "%s: S=%lld not divisible by P=%d", name,
                    (long long)S, P);
    // a 64-row tile must not straddle two pieces
    if (B > 1 && (S / P) % 64)
        return fail(ULY_ERR_UNSUPPORTED, "%s: B > 1 needs S/P a multiple of 64 (S/P=%lld)", name,
                    (long long)(S / P));
    if (empty) return ok();
    hipError_t err = uly::launch_attention_bwd_bf16_d128(q, k, v, o, dout, lse, delta, dq, dk, dv,
                                                         B, S, n_q_heads, n_kv_heads, S / P,
                                                         causal != 0,
                                                         static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

uly_status_t ulysses_attention_chunk(const void *q, const void *k, const void *v, void *o,
                                     float *lse, int64_t B, int64_t Sq, int64_t Skv,
                                     int64_t n_q_heads, int64_t n_kv_heads, int64_t head_dim,
                                     int64_t q_pos0, int64_t k_pos0, int32_t causal,
                                     uly_dtype_t dtype, void *stream) {
    return attention_chunk("ulysses_attention_chunk", q, k, v, o, lse, B, Sq, Skv, n_q_heads,
                           n_kv_heads, head_dim, q_pos0, k_pos0, causal, dtype, false, stream);
}

uly_status_t ulysses_attention_chunk_accumulate(const void *q, const void *k, const void *v, void *o,
                                                float *lse, int64_t B, int64_t Sq, int64_t Skv,
                                                int64_t n_q_heads, int64_t n_kv_heads,
                                                int64_t head_dim, int64_t q_pos0, int64_t k_pos0,
                                                int32_t causal, uly_dtype_t dtype, void *stream) {
    return attention_chunk("ulysses_attention_chunk_accumulate", q, k, v, o, lse, B, Sq, Skv,
                           n_q_heads, n_kv_heads, head_dim, q_pos0, k_pos0, causal, dtype, true,
                           stream);
}

uly_status_t ulysses_attention_merge(const void *o_a, const float *lse_a, const void *o_b,
                                     const float *lse_b, void *o, float *lse, int64_t B, int64_t S,
                                     int64_t n_heads, int64_t head_dim, uly_dtype_t dtype,
                                     void *stream) {
    const char *name = "ulysses_attention_merge";
    const int e = elem_bytes(dtype);
    if (!e) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", name, int(dtype));
    if (B < 0 || S < 0) return fail(ULY_ERR_INVALID_ARGUMENT, "%s: negative B or S", name);
    if (n_heads < 1 || head_dim < 1)
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: n_heads and head_dim must be >= 1", name);
    const int64_t row = head_dim * e;
    if (row < 16 || row > 1024 || (row & (row - 1)))
        return fail(ULY_ERR_UNSUPPORTED, "%s: head_dim * element size = %lld bytes is not a power "
                    "of two in [16, 1024]", name, (long long)row);
    uint64_t rows = 1;
    if (!mul_ok(rows, B) || !mul_ok(rows, S) || !mul_ok(rows, n_heads) || rows >= (uint64_t(1) << 32))
        return fail(ULY_ERR_UNSUPPORTED, "%s: B*S*n_heads must be below 2^32", name);
    if (rows == 0) return ok();
    if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse)
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL pointer", name);
    if (!aligned(o_a, 16) || !aligned(o_b, 16) || !aligned(o, 16) || !aligned(lse_a, 4) ||
        !aligned(lse_b, 4) || !aligned(lse, 4))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: outputs must be 16-byte aligned, lse 4-byte",
                    name);
    const uint64_t ob = rows * uint64_t(row), lb = rows * 4;
    // in place is allowed: o may be exactly o_a or o_b, lse exactly lse_a or lse_b
    if ((o != o_a && overlap(o, ob, o_a, ob)) || (o != o_b && overlap(o, ob, o_b, ob)) ||
        (lse != lse_a && overlap(lse, lb, lse_a, lb)) || (lse != lse_b && overlap(lse, lb, lse_b, lb)))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: an output partly overlaps its input", name);
    if (overlap(o, ob, lse_a, lb) || overlap(o, ob, lse_b, lb) || overlap(o, ob, lse, lb) ||
        overlap(lse, lb, o_a, ob) || overlap(lse, lb, o_b, ob))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: outputs overlap the other tensors", name);
    hipError_t err = uly::launch_merge(o_a, lse_a, o_b, lse_b, o, lse, B, S, n_heads, head_dim, e,
                                       static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

uly_status_t ulysses_attention_chunk_backward(const void *q, const void *k, const void *v,
                                              const void *o, const void *dout, const float *lse,
                                              float *delta, void *dq, void *dk, void *dv, int64_t B,
                                              int64_t Sq, int64_t Skv, int64_t n_q_heads,
                                              int64_t n_kv_heads, int64_t head_dim, int64_t q_pos0,
                                              int64_t k_pos0, int32_t causal, int32_t accumulate_dq,
                                              int32_t accumulate_dkv, uly_dtype_t dtype,
                                              void *stream) {
    const char *name = "ulysses_attention_chunk_backward";
    uint64_t qbytes = 0, kbytes = 0, unused = 0;
    uly_status_t st = attention_shape(name, B, Sq, n_q_heads, n_kv_heads, head_dim, dtype, qbytes,
                                      unused);
    if (st != ULY_OK) return st;
    st = attention_shape(name, B, Skv, n_q_heads, n_kv_heads, head_dim, dtype, unused, kbytes);
    if (st != ULY_OK) return st;
    if (dtype != ULY_DTYPE_BF16 || head_dim != 128)
        return fail(ULY_ERR_UNSUPPORTED, "%s: gradients need ULY_DTYPE_BF16 with head_dim 128", name);
    if (n_q_heads > 65536)
        return fail(ULY_ERR_UNSUPPORTED, "%s: n_q_heads=%lld exceeds 65536", name,
                    (long long)n_q_heads);
    if (Sq >= (int64_t(1) << 30) || Skv >= (int64_t(1) << 30))
        return fail(ULY_ERR_UNSUPPORTED, "%s: Sq and Skv must be below 2^30", name);
    const int64_t kPosMax = int64_t(1) << 62;
    if (q_pos0 < -kPosMax || q_pos0 > kPosMax || k_pos0 < -kPosMax || k_pos0 > kPosMax)
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: positions beyond +-2^62", name);
    if (qbytes == 0 && kbytes == 0) return ok();
    const uint64_t fbytes = uint64_t(B) * uint64_t(Sq) * uint64_t(n_q_heads) * 4;
    const bool qside = qbytes != 0, kside = kbytes != 0;
    if ((qside && (!q || !o || !dout || !lse || !delta || !dq)) || (kside && (!k || !v || !dk || !dv)))
        return fail(ULY_ERR_INVALID_ARGUMENT, "%s: NULL pointer", name);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(lse, 4) || !aligned(delta, 4))
        return fail(ULY_ERR_INVALID_ARGUMENT,
                    "%s: tensors must be 16-byte aligned, lse and delta 4-byte aligned", name);
    const void *in[6] = {q, k, v, o, dout, lse};
    const uint64_t inb[6] = {qbytes, kbytes, kbytes, qbytes, qbytes, fbytes};
    void *out[4] = {dq, dk, dv, delta};
    const uint64_t outb[4] = {qbytes, kbytes, kbytes, fbytes};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(out[i], outb[i], in[j], inb[j]))
                return fail(ULY_ERR_INVALID_ARGUMENT, "%s: an output overlaps an input", name);
        for (int j = i + 1; j < 4; ++j)
            if (overlap(out[i], outb[i], out[j], outb[j]))
                return fail(ULY_ERR_INVALID_ARGUMENT, "%s: two outputs overlap", name);
    }
    // key j visible to row i iff k_pos0 + j <= q_pos0 + i, i.e. j <= i + dpos;
    // a chunk whose every key precedes every row needs no mask
    int64_t dpos = q_pos0 - k_pos0;
    dpos = dpos < -Sq ? -Sq : (dpos > Skv ? Skv : dpos);
    const bool masked = causal != 0 && dpos < Skv - 1;
    hipError_t err = uly::launch_attention_chunk_bwd_bf16_d128(
        q, k, v, o, dout, lse, delta, dq, dk, dv, B, Sq, Skv, dpos, accumulate_dq != 0,
        accumulate_dkv != 0, n_q_heads, n_kv_heads, masked, static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(ULY_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return ok();
}

const char *ulysses_status_string(uly_status_t s) {
    switch (s) {
        case ULY_OK: return "ok";
        case ULY_ERR_INVALID_ARGUMENT: return "invalid argument";
        case ULY_ERR_NOT_DIVISIBLE: return "not divisible";
        case ULY_ERR_UNSUPPORTED: return "unsupported";
        case ULY_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char *ulysses_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
