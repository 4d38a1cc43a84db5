// Merge of two partial attention results over disjoint key sets, the step
// that combines the visits of circulating key/value blocks once the sequence
// degree passes the head count ("Sequence Parallelism II: DeepSpeed Ulysses
// and All-to-All Attention", section 8).  With lse_x the natural log of a
// row's exp-sum over key set x and o_x its normalised output:
//
//   lse = log(exp(lse_a) + exp(lse_b))
//   o   = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b
//
// evaluated against m = max(lse_a, lse_b) so that no exponential overflows; a
// row empty on both sides (m = -inf) stays empty (o = 0, lse = -inf).
//
// Bound: HBM.  Per row of head_dim elements the kernel reads o_a and o_b and
// writes o (3 * head_dim * e bytes) plus three 4-byte lse values.  One lane
// moves 16 bytes of a row; the lanes of one row are consecutive and lie in
// one wavefront (head_dim * e is a power of two <= 1024, so a row is at most
// 64 lanes and rows never straddle a wavefront), which is what makes the
// in-place form (o = o_a or o_b, lse = lse_a or lse_b) safe: every lane of
// the row has read both lse values before any lane writes the merged one.
#include "internal.h"

#include <cmath>

namespace uly {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec16;
template <>
struct Vec16<short> {  // 8 bf16
    static constexpr int n = 8;
    typedef short raw __attribute__((ext_vector_type(8)));
    static __device__ float get(const raw &r, int i) { return __uint_as_float(uint32_t(uint16_t(r[i])) << 16); }
    static __device__ void set(raw &r, int i, float x) {
        // round to nearest, ties to even (NaN kept quiet)
        const uint32_t u = __float_as_uint(x);
        const uint32_t rnd = (u & 0x7FFFFFFFu) > 0x7F800000u ? (u | 0x00400000u) : u + 0x7FFFu + ((u >> 16) & 1u);
        r[i] = short(rnd >> 16);
    }
};
template <>
struct Vec16<float> {  // 4 fp32
    static constexpr int n = 4;
    typedef float raw __attribute__((ext_vector_type(4)));
    static __device__ float get(const raw &r, int i) { return r[i]; }
    static __device__ void set(raw &r, int i, float x) { r[i] = x; }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void merge_kernel(const T *oa, const float *lse_a, const T *ob,
                                                         const float *lse_b, T *o, float *lse,
                                                         uint64_t nvec, uint32_t vpr_shift,
                                                         FastDiv heads, FastDiv seq) {
    // no __restrict__: o may be o_a or o_b, lse may be lse_a or lse_b
    using V = Vec16<T>;
    using raw = typename V::raw;
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;  // a multiple of 64
    for (uint64_t x = uint64_t(blockIdx.x) * kThreads + threadIdx.x; x < nvec; x += stride) {
        // vector x -> row r = (b*S + s)*H + h  ->  lse index (b*H + h)*S + s
        const uint32_t r = uint32_t(x >> vpr_shift);  // rows < 2^32 (checked by the caller)
        const uint32_t bs = heads.div(r), h = r - bs * heads.d;
        const uint32_t b = seq.div(bs), s = bs - b * seq.d;
        const uint64_t li = (uint64_t(b) * heads.d + h) * seq.d + s;
        const float la = lse_a[li], lb = lse_b[li];
        const raw va = *reinterpret_cast<const raw *>(oa + x * V::n);
        const raw vb = *reinterpret_cast<const raw *>(ob + x * V::n);
        const float m = fmaxf(la, lb);
        float wa = 0.f, wb = 0.f, l = -INFINITY;
        if (m != -INFINITY) {
            const float ea = expf(la - m), eb = expf(lb - m);
            const float tot = ea + eb;
            wa = ea / tot;
            wb = eb / tot;
            l = m + logf(tot);
        }
        raw out;
#pragma unroll
        for (int i = 0; i < V::n; ++i) V::set(out, i, fmaf(wa, V::get(va, i), wb * V::get(vb, i)));
        *reinterpret_cast<raw *>(o + x * V::n) = out;
        if ((uint32_t(x) & ((1u << vpr_shift) - 1)) == 0) lse[li] = l;
    }
}

}  // namespace

hipError_t launch_merge(const void *oa, const float *lse_a, const void *ob, const float *lse_b,
                        void *o, float *lse, int64_t B, int64_t S, int64_t H, int64_t D, int32_t elem,
                        hipStream_t st) {
    const uint32_t vpr = uint32_t(D * elem / 16);  // 16-byte vectors per row, a power of two <= 64
    const uint64_t nvec = uint64_t(B) * uint64_t(S) * uint64_t(H) * vpr;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const uint64_t want = (nvec + kThreads - 1) / kThreads;
    const uint32_t blocks = uint32_t(want < uint64_t(cus) * 16 ? want : uint64_t(cus) * 16);
    uint32_t shift = 0;
    while ((1u << shift) < vpr) ++shift;
    const FastDiv fh{uint32_t(H)}, fs{uint32_t(S)};
    if (elem == 2)
        hipLaunchKernelGGL(merge_kernel<short>, dim3(blocks), dim3(kThreads), 0, st,
                           static_cast<const short *>(oa), lse_a, static_cast<const short *>(ob),
                           lse_b, static_cast<short *>(o), lse, nvec, shift, fh, fs);
    else
        hipLaunchKernelGGL(merge_kernel<float>, dim3(blocks), dim3(kThreads), 0, st,
                           static_cast<const float *>(oa), lse_a, static_cast<const float *>(ob),
                           lse_b, static_cast<float *>(o), lse, nvec, shift, fh, fs);
    return hipGetLastError();
}

}  // namespace uly
