// One rank's local attention in fp32 (small head_dim, correctness-first path):
// softmax(Q K^T / sqrt(D)) V per head ("Comparing Ulysses and Megatron Sequence
// Parallelism", attention skeleton in the Introduction), grouped key/value
// heads, optional causal triangle ("Sequence Parallelism II: DeepSpeed Ulysses
// and All-to-All Attention", section 8).
//
// One thread owns one query row; key/value rows are staged through LDS in
// tiles of KT and read back as broadcasts.  The softmax is the online
// (running max / running sum) form: per tile the row maximum is updated, the
// accumulator and the running sum are rescaled by exp2(m_old - m_new), then
// the tile's weights are accumulated.  Exponentials are taken base 2 on
// scores pre-multiplied by log2(e)/sqrt(D).
#include "internal.h"

#include <cmath>

namespace uly {
namespace {

constexpr int kRows = 128;  // query rows (threads) per workgroup

// PIECES (full sequence only): q, k, v, o in the order the exchange delivers
// and sends them, [P][B][sp][h][D] with sp = S/P rows per peer piece: token s
// of batch entry b is row b*sp + s + (s / sp) * gap, gap = (B-1)*sp.
template <int D, int KT, bool PIECES>
__global__ __launch_bounds__(kRows) void attention_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    float *__restrict__ o, float *__restrict__ lse, int S, int Skv, int delta, int Hq, int Hkv,
    int group, int causal, float scale_log2, FastDiv by_sp, int64_t gap) {
    // S query rows, Skv key rows; under the causal mask key j is visible to
    // row i iff j <= i + delta (delta = 0 and Skv = S for the full sequence)
    __shared__ float ks[KT][D];
    __shared__ float vs[KT][D];
    const int nblk = (S + kRows - 1) / kRows;
    const int bh = blockIdx.x / nblk;
    const int b = bh / Hq, c = bh - b * Hq, ck = c / group;
    const int row0 = (blockIdx.x - bh * nblk) * kRows;
    const int row = row0 + threadIdx.x;
    const bool live = row < S;
    const int64_t qstride = int64_t(Hq) * D, kstride = int64_t(Hkv) * D;
    // first row of batch entry b, and the row of its token s past that
    const int64_t qb0 = int64_t(b) * (PIECES ? int64_t(by_sp.d) : int64_t(S));
    const int64_t kb0 = int64_t(b) * (PIECES ? int64_t(by_sp.d) : int64_t(Skv));
    auto row_of = [&](int s) -> int64_t {
        return PIECES ? int64_t(s) + int64_t(by_sp.div(uint32_t(s))) * gap : int64_t(s);
    };
    const float *qb = q + qb0 * qstride + int64_t(c) * D;
    const float *kb = k + kb0 * kstride + int64_t(ck) * D;
    const float *vb = v + kb0 * kstride + int64_t(ck) * D;

    float qr[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        qr[d] = live ? qb[row_of(row) * qstride + d] : 0.f;
        acc[d] = 0.f;
    }
    float m = -1e30f, l = 0.f;
    const int last_row = min(S - 1, row0 + kRows - 1);
    const int kend = causal ? min(Skv, max(0, last_row + 1 + delta)) : Skv;

    for (int k0 = 0; k0 < kend; k0 += KT) {
        for (int e = threadIdx.x; e < KT * D; e += kRows) {
            const int j = e / D, d = e - j * D, key = k0 + j;
            const bool in = key < Skv;
            const int64_t kr = row_of(in ? key : 0) * kstride;
            ks[j][d] = in ? kb[kr + d] : 0.f;
            vs[j][d] = in ? vb[kr + d] : 0.f;
        }
        __syncthreads();
        if (live) {
            float s[KT];
            float tmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                const int key = k0 + j;
                float dot = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) dot = fmaf(qr[d], ks[j][d], dot);
                const bool visible = key < Skv && (!causal || key <= row + delta);
                s[j] = visible ? dot * scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, s[j]);
            }
            const float mnew = fmaxf(m, tmax);
            const float alpha = exp2f(m - mnew);
            l *= alpha;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
            for (int j = 0; j < KT; ++j) {
                const float p = exp2f(s[j] - mnew);
                l += p;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
            }
            m = mnew;
        }
        __syncthreads();
    }
    if (live && lse)  // natural log of the row's sum of exp(scores)
        lse[int64_t(bh) * S + row] = (m + log2f(l)) * 0.69314718055994531f;
    if (live) {
        const float inv = l > 0.f ? 1.f / l : 0.f;  // a row with no visible key: o = 0
        float *ob = o + (qb0 + row_of(row)) * qstride + int64_t(c) * D;
#pragma unroll
        for (int d = 0; d < D; ++d) ob[d] = acc[d] * inv;
    }
}

template <int D, int KT>
hipError_t launch_d(const float *q, const float *k, const float *v, float *o, float *lse,
                    int64_t B, int64_t S, int64_t Skv, int64_t delta, int64_t Hq, int64_t Hkv,
                    int64_t sp, bool causal, hipStream_t st) {
    dim3 grid(uint32_t((S + kRows - 1) / kRows * B * Hq));
    const float scale_log2 = float(1.4426950408889634 / std::sqrt(double(D)));
    if (sp)
        hipLaunchKernelGGL((attention_f32_kernel<D, KT, true>), grid, dim3(kRows), 0, st, q, k, v,
                           o, lse, int(S), int(Skv), int(delta), int(Hq), int(Hkv), int(Hq / Hkv),
                           int(causal), scale_log2, FastDiv(uint32_t(sp)), (B - 1) * sp);
    else
        hipLaunchKernelGGL((attention_f32_kernel<D, KT, false>), grid, dim3(kRows), 0, st, q, k, v,
                           o, lse, int(S), int(Skv), int(delta), int(Hq), int(Hkv), int(Hq / Hkv),
                           int(causal), scale_log2, FastDiv(), int64_t(0));
    return hipGetLastError();
}

hipError_t launch_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                      int64_t B, int64_t Sq, int64_t Skv, int64_t delta, int64_t Hq, int64_t Hkv,
                      int64_t D, int64_t sp, bool causal, hipStream_t st) {
    switch (D) {
        case 32: return launch_d<32, 32>(q, k, v, o, lse, B, Sq, Skv, delta, Hq, Hkv, sp, causal, st);
        case 64: return launch_d<64, 16>(q, k, v, o, lse, B, Sq, Skv, delta, Hq, Hkv, sp, causal, st);
        case 128: return launch_d<128, 8>(q, k, v, o, lse, B, Sq, Skv, delta, Hq, Hkv, sp, causal, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attention_chunk_f32(const float *q, const float *k, const float *v, float *o,
                                      float *lse, int64_t B, int64_t Sq, int64_t Skv,
                                      int64_t delta, int64_t Hq, int64_t Hkv, int64_t D,
                                      bool causal, hipStream_t st) {
    return launch_f32(q, k, v, o, lse, B, Sq, Skv, delta, Hq, Hkv, D, 0, causal, st);
}

hipError_t launch_attention_f32(const float *q, const float *k, const float *v, float *o,
                                float *lse, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                int64_t D, int64_t sp, bool causal, hipStream_t st) {
    // with one batch entry the pieces are the plain sequence order
    return launch_f32(q, k, v, o, lse, B, S, S, 0, Hq, Hkv, D, B > 1 ? sp : 0, causal, st);
}

}  // namespace uly
