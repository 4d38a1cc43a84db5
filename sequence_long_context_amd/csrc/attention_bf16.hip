// One rank's local attention, bf16 in / bf16 out, head_dim 128, on gfx950
// matrix cores: softmax(Q K^T / sqrt(D)) V per head ("Comparing Ulysses and
// Megatron Sequence Parallelism", attention skeleton in the Introduction),
// grouped key/value heads, optional causal triangle ("Sequence Parallelism II:
// DeepSpeed Ulysses and All-to-All Attention", section 8).
//
// Flash-style fused kernel.  A workgroup is 8 wavefronts and owns 256 query
// rows of one head (32 rows per wavefront; 4 wavefronts and 128 rows when the
// 8-wavefront grid would leave CUs idle, as for short sequences); it streams the head's keys and
// values in tiles of 64 rows through LDS (two stages: tile n+1 is requested
// straight into the free stage while tile n is computed) and keeps a running
// row maximum and row sum (online softmax), so the S x S score matrix never
// leaves registers.  The running maximum is only moved when a tile raises it
// by more than 8 (base-2 units): until then the weights exp2(s - m) stay
// below 2^8, which fp32 sums and bf16 weights carry without loss, and the
// output and row sum need no rescaling (the final division uses the same m).
//
// Orientation.  Each wavefront computes the transposed score tile
// S^T[key][query] = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
// B = the wavefront's Q rows, held in registers for the whole kernel).  In the
// 32x32 accumulator layout lane l holds query row l%32 and 16 of the 32 keys,
// the other 16 sitting in lane l^32, so
//   * a row maximum is a register reduction plus one v_permlane32_swap,
//   * the rescale of the output by exp2(m_old - m_new) is a per-lane scalar,
//   * the bf16 probabilities are already in the B-operand layout of the next
//     product O^T[d][query] += V^T P^T: no LDS round trip for P.
// The A operand V^T needs, per lane, four consecutive keys of one d column:
// ds_read_b64_tr_b16 returns exactly that from row-major V in LDS.  The key
// order inside each 16-key MFMA step is permuted identically in P and V
// (a sum over keys does not depend on their order).
//
// Row sums on the matrix core.  The normaliser is the sum of the same bf16
// weights that multiply V, accumulated by one v_mfma_f32_16x16x32_bf16 per
// 16-key step: read as a 16x16x32 B operand, the P register holds, in lane
// group g = l/16, 8 keys of query (l%16) + 16*(g%2); an A operand with
// A[m][k] = 1 exactly when (k/8)%2 == (m/4)%2 sums, into output row block
// m/4 = g, all 16 keys of that lane's own query.  This replaces 32 vector
// adds per tile and makes the division consistent with the rounded weights.
//
// Tile copies are LDS DMA (buffer_load_dwordx4 ... lds: each lane's 16 bytes
// go from global memory straight to LDS), which costs neither registers nor
// ds_write instructions; writing tiles through registers kept the LDS write
// queue full and cost about a tenth of the kernel's time.  Each request holds
// the issuing wavefront for a few tens of cycles, so a wavefront's requests
// for tile n+1 are spread over its Q.K products of tile n, where the other
// wavefront of the SIMD keeps the matrix core busy.  The buffer resource of a
// tile spans only its rows inside the sequence; the rows of a ragged last
// tile past the end read as zero (their scores are masked; the V stages are
// zeroed once at the start so that no stale LDS content can reach the sum).
// The DMA is issued as inline assembly: the compiler models an LDS DMA as an
// access that may alias every LDS read and would then wait for all
// outstanding LDS operations before each fragment read.  Each wavefront orders
// its own requests with an explicit vmcnt wait before the barrier that
// publishes the tile; the hazard wait states an LDS DMA needs (after a vector
// write of a scalar operand, after the write of M0) are part of the assembly.
//
// Issue order.  The scheduler would read K fragments only about two products
// ahead; sched_group_barrier pins four reads ahead of each Q.K product.
//
// LDS rows are 256 bytes; the 16-byte chunk c of row r is stored at chunk
// c ^ swz(r) with swz(r) = (r%4)*4 + (r/4)%4, which keeps both the K reads
// (16 consecutive rows, one chunk) and the V transpose reads (8 rows, 4
// chunks) free of bank conflicts.
//
// Work order: workgroup e takes head e % (B*Hq) and, for causal, query block
// nqb-1 - e/(B*Hq), so the longest blocks start first; consecutive workgroups
// go round-robin to the 8 XCDs, so each XCD works on a fixed subset of heads
// and their keys/values stay in its L2.
//
// Algorithmic work: 4*D flops per visible (query, key) pair.
#include "internal.h"

namespace uly {
namespace {

typedef __attribute__((__vector_size__(16))) short s16x8;
typedef __attribute__((__vector_size__(8))) short s16x4;
typedef __attribute__((__vector_size__(64))) float f32x16;
typedef __attribute__((__vector_size__(16))) float f32x4;
#define LDS_AS __attribute__((address_space(3)))

// Workgroups of NW wavefronts own 32*NW query rows: NW = 8 where the grid
// fills the GPU, NW = 4 (twice the workgroups) for short sequences.
constexpr int kBN = 64;              // keys per tile
constexpr int kD = 128;              // head_dim
constexpr float kRescaleSlack = 8.f; // base-2 headroom before the running max moves
constexpr int kRowB = kD * 2;        // bytes per K/V row
constexpr int kTileB = kBN * kRowB;  // 16 KiB
constexpr int kStageB = 2 * kTileB;  // K tile + V tile
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ float pair_max(float x) {  // max over lanes l and l^32
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ short to_bf16(float f) {  // round to nearest even
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(short, h);
}

// LDS DMA through a buffer resource: this lane's 16 bytes at (resource base
// + voff) land at LDS byte address m0 + 16 * lane; offsets at or past the
// resource's byte count read as zero.  s_nop 4 gives the five wait states a
// vector memory instruction needs after a vector instruction wrote one of its
// scalar operands (and the one after a write of M0): the compiler's hazard
// checks do not see inside inline assembly.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16(const i32x4 &rsrc, uint32_t voff, uint32_t m0) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}
// Raw buffer resource (stride 0) over the first rows_valid rows of a tile
// whose rows are rstride elements apart: byte count (rows_valid-1)*row pitch
// + 256, so exactly the rows inside the sequence are in range.
__device__ __forceinline__ i32x4 tile_resource(const short *tile0, int rows_valid, int64_t rstride) {
    const uint64_t a = reinterpret_cast<uint64_t>(tile0);
    const uint32_t bytes = uint32_t(int64_t(rows_valid - 1) * rstride * 2 + kRowB);
    return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xFFFFu), int(bytes), 0x00020000};
}
// This wavefront's share of a 64-row tile (16 quads of 4 rows, 1 KiB each):
// quads QPW*w .. QPW*w + QPW-1 with QPW = 16 / NW; lane l of quad q lands in
// slot l%16 of row 4q + l/16 and so loads the global chunk (l%16) ^ swz(row).
template <int QPW> struct TileDma {
    uint32_t goff[QPW];  // per-lane byte offsets from the tile's first row
    uint32_t m0[QPW];    // LDS byte offsets of this wavefront's quads (uniform)
};
template <int QPW>
__device__ __forceinline__ void tile_dma_setup(TileDma<QPW> &td, int w, int lane, int64_t rstride) {
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
        const int row = (QPW * w + u) * 4 + (lane >> 4), chunk = (lane & 15) ^ swz(row);
        td.goff[u] = uint32_t(int64_t(row) * rstride * 2 + chunk * 16);
        td.m0[u] = __builtin_amdgcn_readfirstlane((QPW * w + u) * 4 * kRowB);
    }
}

struct Frag {
    s16x8 q[8];          // this wavefront's 32 query rows, B-operand layout
    f32x16 o[4];         // O^T accumulators, d blocks of 32
    f32x4 lsum;          // row sums of the bf16 weights (each element: this lane's row)
    s16x8 ones;          // 16x16x32 A operand summing weights per query row
    float m;             // running max (scaled, base 2)
    int koff[8];         // per-lane LDS byte offsets of the K reads, per 16-wide d chunk
    int voff[2][4];      // per-lane LDS byte offsets of the V transpose reads
};

// K fragment i (d chunk i/2, key chain i%2) and V operand i (key step
// (i/8, i/4 % 2), d block i % 4) of this lane, from the LDS tiles.
__device__ __forceinline__ s16x8 read_k(const Frag &f, const LDS_AS char *kt, int i) {
    return *reinterpret_cast<const LDS_AS s16x8 *>(kt + f.koff[i >> 1] + (i & 1) * 32 * kRowB);
}
__device__ __forceinline__ s16x8 read_v(const Frag &f, const LDS_AS char *vt, int i) {
    const int t = i >> 3, h = (i >> 2) & 1, mt = i & 3;
    const int rowoff = (32 * t + 16 * h) * kRowB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(vt + f.voff[0][mt] + rowoff));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(vt + f.voff[1][mt] + rowoff));
    return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// One tile for one wavefront; req(r), r < NREQ, issues this wavefront's
// requests for the next tile, spread over the Q.K products.
template <bool CAUSAL, int NREQ, typename Req>
__device__ __forceinline__ void tile_step(Frag &f, const LDS_AS char *kt, const LDS_AS char *vt,
                                          int key0, int wrow0, int qrow, int S, float scale_log2,
                                          int lane, Req &&req) {
    if (CAUSAL && key0 > wrow0 + 31) {  // every key of the tile is after every row
#pragma unroll
        for (int r = 0; r < NREQ; ++r) req(r);
        return;
    }
    constexpr int kReqStride = 16 / NREQ;

    // S^T = K Q^T for keys key0 .. key0+63: 16 products (d chunk i/2, 32-key
    // chain i%2), each K fragment read four products ahead of its use.
    constexpr int kAhead = 4;
    f32x16 s[2] = {f32x16{}, f32x16{}};
    {
        s16x8 kf[16];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) kf[i] = read_k(f, kt, i);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + kAhead < 16) kf[i + kAhead] = read_k(f, kt, i + kAhead);
            s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], f.q[i >> 1], s[i & 1], 0, 0, 0);
            if (i % kReqStride == kReqStride / 2) req(i / kReqStride);
        }
    }
    // The first V operands of O^T += V^T P^T do not depend on the softmax:
    // read them now so they arrive while the vector work runs.
    s16x8 vf[16];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) vf[i] = read_v(f, vt, i);
    // Issue order: kAhead K reads, then one product and one further read at a
    // time, then the V reads.
#pragma unroll
    for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);

    const bool need_mask = (CAUSAL && key0 + kBN - 1 > wrow0) || key0 + kBN > S;
    if (need_mask) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * t + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const bool hidden = key >= S || (CAUSAL && key > qrow);
                s[t][r] = hidden ? -INFINITY : s[t][r];
            }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = pair_max(mx) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > f.m + kRescaleSlack)) {  // wavefront-uniform
        const float mnew = fmaxf(f.m, mx);
        const float alpha = __builtin_amdgcn_exp2f(f.m - mnew);
        f.m = mnew;
#pragma unroll
        for (int r = 0; r < 4; ++r) f.lsum[r] *= alpha;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) f.o[mt][r] *= alpha;
    }
    const float mnew = f.m;

    s16x8 pk[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            pk[t][r >> 3][r & 7] = to_bf16(__builtin_amdgcn_exp2f(fmaf(s[t][r], scale_log2, -mnew)));

    // O^T += V^T P^T: 16 products, key step (t, h) = (i/8, i/4 % 2) and d block
    // mt = i % 4, operands read four ahead; a row-sum product ends each key step.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i + kAhead < 16) vf[i + kAhead] = read_v(f, vt, i + kAhead);
        const int t = i >> 3, h = (i >> 2) & 1, mt = i & 3;
        f.o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pk[t][h], f.o[mt], 0, 0, 0);
        if (mt == 3)
            f.lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.ones, pk[t][h], f.lsum, 0, 0, 0);
    }
}

template <bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attention_bf16_d128_kernel(
    const short *__restrict__ q, const short *__restrict__ k, const short *__restrict__ v,
    short *__restrict__ o, float *__restrict__ lse, int S, int Hq, int Hkv, int group, int nqb,
    int htot, float scale_log2) {
    __shared__ __attribute__((aligned(1024))) char smem0[kStageB];
    __shared__ __attribute__((aligned(1024))) char smem1[kStageB];
    LDS_AS char *lds0 = (LDS_AS char *)smem0;
    LDS_AS char *lds1 = (LDS_AS char *)smem1;

    const int e = blockIdx.x;
    const int hh = e % htot;
    constexpr int kBM = 32 * NW;  // query rows per workgroup
    const int qb = CAUSAL ? nqb - 1 - e / htot : e / htot;
    const int b = hh / Hq, c = hh - b * Hq, ck = c / group;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int q0 = qb * kBM;
    const int wrow0 = q0 + 32 * w;
    const int qrow = wrow0 + (lane & 31);
    const int64_t qstride = int64_t(Hq) * kD, kstride = int64_t(Hkv) * kD;
    const short *qh = q + int64_t(b) * S * qstride + int64_t(c) * kD;
    const short *kh = k + int64_t(b) * S * kstride + int64_t(ck) * kD;
    const short *vh = v + int64_t(b) * S * kstride + int64_t(ck) * kD;

    const int kend = CAUSAL ? min(S, q0 + kBM) : S;
    const int ntiles = (kend + kBN - 1) / kBN;

    constexpr int QPW = 16 / NW;
    TileDma<QPW> td;
    tile_dma_setup(td, w, lane, kstride);
    // requests of this wavefront's share of tile n (K and V) into stage dst
    auto tile_req = [&](int n, const LDS_AS char *dst, int r) __attribute__((always_inline)) {
        const int row0 = n * kBN;
        const int valid = min(S - row0, kBN);
        const uint32_t d = uint32_t(reinterpret_cast<uintptr_t>(dst));
        if (r < QPW) dma16(tile_resource(kh + int64_t(row0) * kstride, valid, kstride), td.goff[r], d + td.m0[r]);
        else dma16(tile_resource(vh + int64_t(row0) * kstride, valid, kstride), td.goff[r - QPW],
                   d + kTileB + td.m0[r - QPW]);
    };
    if (S % kBN != 0) {  // ragged last tile: start both V stages at zero
#pragma unroll
        for (int i = 0; i < kTileB / (16 * 64 * NW); ++i) {
            const int off = (i * 64 * NW + int(threadIdx.x)) * 16;
            *reinterpret_cast<LDS_AS s16x8 *>(lds0 + kTileB + off) = s16x8{};
            *reinterpret_cast<LDS_AS s16x8 *>(lds1 + kTileB + off) = s16x8{};
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 2 * QPW; ++r) tile_req(0, lds0, r);

    Frag f;
    {
        const short *qp = qh + int64_t(min(qrow, S - 1)) * qstride + 8 * (lane >> 5);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) f.q[cc] = *reinterpret_cast<const s16x8 *>(qp + 16 * cc);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) f.o[mt] = f32x16{};
        f.m = -1e30f;
        f.lsum = f32x4{};
        const short one = ((lane >> 4) & 1) == ((lane & 15) >> 2 & 1) ? short(0x3F80) : short(0);
#pragma unroll
        for (int i = 0; i < 8; ++i) f.ones[i] = one;
        const int kr = lane & 31;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc)
            f.koff[cc] = kr * kRowB + (((2 * cc + (lane >> 5)) ^ swz(kr)) << 4);
        const int sl = lane & 15;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int vr = 8 * rr + 4 * (lane >> 5) + (sl >> 2);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int dcol = 32 * mt + 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
                f.voff[rr][mt] = vr * kRowB + (((dcol >> 3) ^ swz(vr)) << 4) + ((dcol & 7) << 1);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and tile 0 have landed
    __syncthreads();

    auto step = [&](int n, LDS_AS char *cur, LDS_AS char *nxt) __attribute__((always_inline)) -> bool {
        const bool more = n + 1 < ntiles;
        // tile n+1 into the other stage (after the last tile: the last tile
        // again, into the stage nobody reads any more)
        const int n1 = min(n + 1, ntiles - 1);
        auto req = [&](int r) __attribute__((always_inline)) { tile_req(n1, nxt, r); };
        tile_step<CAUSAL, 2 * QPW>(f, cur, cur + kTileB, n * kBN, wrow0, qrow, S, scale_log2, lane, req);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's DMA of tile n+1
        __syncthreads();
        return more;
    };
    for (int n = 0;; n += 2) {
        if (!step(n, lds0, lds1)) break;
        if (!step(n + 1, lds1, lds0)) break;
    }

    if (lse && qrow < S && lane < 32)  // natural log of the row's sum of exp(scores)
        lse[int64_t(hh) * S + qrow] = (f.m + __log2f(f.lsum[0])) * kLn2;
    if (qrow < S) {
        const float inv = 1.f / f.lsum[0];
        short *op = o + int64_t(b) * S * qstride + int64_t(c) * kD + int64_t(qrow) * qstride;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                s16x4 pv;
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[i] = to_bf16(f.o[mt][4 * g + i] * inv);
                *reinterpret_cast<s16x4 *>(op + 32 * mt + 8 * g + 4 * (lane >> 5)) = pv;
            }
    }
}

}  // namespace

namespace {
template <int NW>
hipError_t launch_nw(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                     int64_t S, int64_t Hq, int64_t Hkv, bool causal, hipStream_t st) {
    const int nqb = int((S + 32 * NW - 1) / (32 * NW));
    const int htot = int(B * Hq);
    const float scale_log2 = float(1.4426950408889634 / 11.313708498984761);  // log2(e)/sqrt(128)
    dim3 grid(uint32_t(int64_t(nqb) * htot)), block(NW * 64);
    if (causal)
        hipLaunchKernelGGL((attention_bf16_d128_kernel<true, NW>), grid, block, 0, st,
                           static_cast<const short *>(q), static_cast<const short *>(k),
                           static_cast<const short *>(v), static_cast<short *>(o), lse, int(S),
                           int(Hq), int(Hkv), int(Hq / Hkv), nqb, htot, scale_log2);
    else
        hipLaunchKernelGGL((attention_bf16_d128_kernel<false, NW>), grid, block, 0, st,
                           static_cast<const short *>(q), static_cast<const short *>(k),
                           static_cast<const short *>(v), static_cast<short *>(o), lse, int(S),
                           int(Hq), int(Hkv), int(Hq / Hkv), nqb, htot, scale_log2);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_attention_bf16_d128(const void *q, const void *k, const void *v, void *o,
                                      float *lse, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                      bool causal, hipStream_t st) {
    // 8-wavefront workgroups when they cover every CU at least once, else 4
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t wg8 = ((S + 255) / 256) * B * Hq;
    return wg8 >= cus ? launch_nw<8>(q, k, v, o, lse, B, S, Hq, Hkv, causal, st)
                      : launch_nw<4>(q, k, v, o, lse, B, S, Hq, Hkv, causal, st);
}

// ---------------------------------------------------------------------------
// Gradients.  The backward pass runs the layout changes in reverse ("Sequence
// Parallelism II...", section 6); between them sits the derivative of the
// local attention above.  With lse_i the natural log of row i's sum of
// exp(scores) (written by the forward), p = exp(s - lse_i), and
// delta_i = sum_d dO[i,d] O[i,d]:
//   dS = p (dO.v - delta_i),  dQ += dS k / sqrt(D),  dK += dS q / sqrt(D),  dV += p dO.
// Three kernels: delta (one pass over O and dO), dQ (each wavefront owns 32
// query rows and streams the key/value tiles, as the forward), and dK/dV
// (each wavefront owns 32 key rows and streams the query, dO, lse and delta
// tiles of every query head of its kv head).  The products reuse the forward's
// operand forms: a row-major LDS tile read as an A operand whose rows are the
// tile rows (read_k), or transposed so that its rows are the 128 columns
// (read_v), and score-layout weights packed to bf16 as the B operand.
namespace {

__device__ __forceinline__ float bf16_to_f32(short x) {
    return __uint_as_float(uint32_t(uint16_t(x)) << 16);
}

// delta[b][c][i] = sum_d dO[b][i][c][d] * O[b][i][c][d]; 16 lanes per row.
__global__ __launch_bounds__(256) void attention_delta_kernel(const short *__restrict__ o,
                                                              const short *__restrict__ dout,
                                                              float *__restrict__ delta, int S,
                                                              int Hq, int64_t rows) {
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t row = t >> 4;  // (b, i, c) in memory order
    const int part = int(t & 15);
    float acc = 0.f;
    if (row < rows) {
        const s16x8 a = *reinterpret_cast<const s16x8 *>(o + row * kD + part * 8);
        const s16x8 g = *reinterpret_cast<const s16x8 *>(dout + row * kD + part * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(bf16_to_f32(a[j]), bf16_to_f32(g[j]), acc);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (row < rows && part == 0) {
        const int64_t bi = row / Hq;
        const int c = int(row - bi * Hq);
        const int64_t b = bi / S;
        const int i = int(bi - b * S);
        delta[(b * Hq + c) * S + i] = acc;
    }
}

struct LdsOff {
    int koff[8];     // A operand from tile rows (read_k form)
    int voff[2][4];  // A operand from tile columns (read_v form)
};
__device__ __forceinline__ void lds_offsets(LdsOff &f, int lane) {
    const int kr = lane & 31;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) f.koff[cc] = kr * kRowB + (((2 * cc + (lane >> 5)) ^ swz(kr)) << 4);
    const int sl = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int vr = 8 * rr + 4 * (lane >> 5) + (sl >> 2);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int dcol = 32 * mt + 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
            f.voff[rr][mt] = vr * kRowB + (((dcol >> 3) ^ swz(vr)) << 4) + ((dcol & 7) << 1);
        }
    }
}
// tile rows 32*(i&1) .. +31, columns 16*(i>>1) .. +15
__device__ __forceinline__ s16x8 rows_op(const LdsOff &f, const LDS_AS char *t, int i) {
    return *reinterpret_cast<const LDS_AS s16x8 *>(t + f.koff[i >> 1] + (i & 1) * 32 * kRowB);
}
// tile columns 32*(i&3) .. +31 as rows, tile rows 32*(i>>3) + 16*((i>>2)&1) .. +15 as k
__device__ __forceinline__ s16x8 cols_op(const LdsOff &f, const LDS_AS char *t, int i) {
    const int tt = i >> 3, h = (i >> 2) & 1, mt = i & 3;
    const int rowoff = (32 * tt + 16 * h) * kRowB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(t + f.voff[0][mt] + rowoff));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(t + f.voff[1][mt] + rowoff));
    return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// this lane's row (lane % 32) of a [rows][128] bf16 matrix as 8 B operands
__device__ __forceinline__ void load_row_operand(s16x8 (&r)[8], const short *row, int lane) {
    const short *p = row + 8 * (lane >> 5);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) r[cc] = *reinterpret_cast<const s16x8 *>(p + 16 * cc);
}
// 32x32 accumulators (4 blocks of 32 columns; lane: column l%32) scaled, to
// bf16, into row (lane % 32) of a [rows][128] matrix
__device__ __forceinline__ void store_acc_row(short *row, const f32x16 (&a)[4], float scale, int lane) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            s16x4 pv;
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = to_bf16(a[mt][4 * g + i] * scale);
            *reinterpret_cast<s16x4 *>(row + 32 * mt + 8 * g + 4 * (lane >> 5)) = pv;
        }
}

// dQ: workgroup of 8 wavefronts = 256 query rows of one head; the key/value
// tiles stream through two LDS stages as in the forward.
template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attention_bwd_dq_kernel(
    const short *__restrict__ q, const short *__restrict__ k, const short *__restrict__ v,
    const short *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    short *__restrict__ dq, int S, int Hq, int Hkv, int group, int nqb, int htot, float scale_log2,
    float inv_sqrt_d) {
    constexpr int NW = 8, QPW = 2, kBM = 256;
    __shared__ __attribute__((aligned(1024))) char smem0[kStageB];
    __shared__ __attribute__((aligned(1024))) char smem1[kStageB];
    LDS_AS char *lds0 = (LDS_AS char *)smem0;
    LDS_AS char *lds1 = (LDS_AS char *)smem1;

    const int e = blockIdx.x;
    const int hh = e % htot;
    const int qb = CAUSAL ? nqb - 1 - e / htot : e / htot;
    const int b = hh / Hq, c = hh - b * Hq, ck = c / group;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int q0 = qb * kBM, wrow0 = q0 + 32 * w, qrow = wrow0 + (lane & 31);
    const int64_t qstride = int64_t(Hq) * kD, kstride = int64_t(Hkv) * kD;
    const int64_t qoff = int64_t(b) * S * qstride + int64_t(c) * kD;
    const short *kh = k + int64_t(b) * S * kstride + int64_t(ck) * kD;
    const short *vh = v + int64_t(b) * S * kstride + int64_t(ck) * kD;
    const int kend = CAUSAL ? min(S, q0 + kBM) : S;
    const int ntiles = (kend + kBN - 1) / kBN;

    TileDma<QPW> td;
    tile_dma_setup(td, w, lane, kstride);
    auto tile_req = [&](int n, const LDS_AS char *dst, int r) __attribute__((always_inline)) {
        const int row0 = n * kBN, valid = min(S - row0, kBN);
        const uint32_t d = uint32_t(reinterpret_cast<uintptr_t>(dst));
        if (r < QPW) dma16(tile_resource(kh + int64_t(row0) * kstride, valid, kstride), td.goff[r], d + td.m0[r]);
        else dma16(tile_resource(vh + int64_t(row0) * kstride, valid, kstride), td.goff[r - QPW],
                   d + kTileB + td.m0[r - QPW]);
    };
    if (S % kBN != 0) {  // ragged last tile: K and V rows past the end start at zero
#pragma unroll
        for (int i = 0; i < kStageB / (16 * 64 * NW); ++i) {
            const int off = (i * 64 * NW + int(threadIdx.x)) * 16;
            *reinterpret_cast<LDS_AS s16x8 *>(lds0 + off) = s16x8{};
            *reinterpret_cast<LDS_AS s16x8 *>(lds1 + off) = s16x8{};
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 2 * QPW; ++r) tile_req(0, lds0, r);

    LdsOff lo;
    lds_offsets(lo, lane);
    s16x8 qr[8], dor[8];
    const int crow = min(qrow, S - 1);
    load_row_operand(qr, q + qoff + int64_t(crow) * qstride, lane);
    load_row_operand(dor, dout + qoff + int64_t(crow) * qstride, lane);
    const float lse2 = lse[int64_t(hh) * S + crow] * kLog2e;
    const float dlt = delta[int64_t(hh) * S + crow];
    f32x16 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x16{};
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    auto step = [&](int n, LDS_AS char *cur, LDS_AS char *nxt) __attribute__((always_inline)) -> bool {
        const bool more = n + 1 < ntiles;
        const int n1 = min(n + 1, ntiles - 1);
        const int key0 = n * kBN;
        const LDS_AS char *kt = cur, *vt = cur + kTileB;
        if (CAUSAL && key0 > wrow0 + 31) {
#pragma unroll
            for (int r = 0; r < 2 * QPW; ++r) tile_req(n1, nxt, r);
        } else {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // S^T and dP^T for keys key0 + 32t .. +31 (lane: query row);
                // operands read kA products ahead, the first kB of dQ before the
                // vector work
                constexpr int kA = 4, kB = 4;
                auto opA = [&](int i) __attribute__((always_inline)) {  // i = 2*cc + (0: K rows, 1: V rows)
                    return rows_op(lo, (i & 1) ? vt : kt, 2 * (i >> 1) + t);
                };
                f32x16 sc = f32x16{}, dp = f32x16{};
                s16x8 a[16], bo[8];
#pragma unroll
                for (int i = 0; i < kA; ++i) a[i] = opA(i);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (i + kA < 16) a[i + kA] = opA(i + kA);
                    if (i & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], dor[i >> 1], dp, 0, 0, 0);
                    else sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qr[i >> 1], sc, 0, 0, 0);
                    if (t == 0 && (i & 3) == 3) tile_req(n1, nxt, i >> 2);
                }
#pragma unroll
                for (int i = 0; i < kB; ++i) bo[i] = cols_op(lo, kt, 8 * t + i);
#pragma unroll
                for (int i = 0; i < kA; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + kA < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * kB, 0);
                s16x8 dsb[2];
                // keys past the end, or after this wavefront's first row (causal), need the mask
                const bool need_mask = key0 + 32 * t + 31 >= S || (CAUSAL && key0 + 32 * t + 31 > wrow0);
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key0 + 32 * t + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                        const bool vis = key < S && (!CAUSAL || key <= qrow);
                        const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, -lse2));
                        dsb[r >> 3][r & 7] = to_bf16(vis ? p * (dp[r] - dlt) : 0.f);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, -lse2));
                        dsb[r >> 3][r & 7] = to_bf16(p * (dp[r] - dlt));
                    }
                }
                // dQ^T += K^T dS^T over these 32 keys
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (i + kB < 8) bo[i + kB] = cols_op(lo, kt, 8 * t + i + kB);
                    acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bo[i], dsb[i >> 2], acc[i & 3], 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i + kB < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's DMA of tile n+1
        __syncthreads();
        return more;
    };
    for (int n = 0;; n += 2) {
        if (!step(n, lds0, lds1)) break;
        if (!step(n + 1, lds1, lds0)) break;
    }
    if (qrow < S) store_acc_row(dq + qoff + int64_t(qrow) * qstride, acc, inv_sqrt_d, lane);
}

// dK, dV: workgroup of 4 wavefronts = 128 key rows of one kv head; for every
// query head of the group, the query tiles (Q, dO: 64 rows each; lse and
// delta: 64 values each) stream through two LDS stages.
constexpr int kBwdStageB = 2 * kTileB + 2 * 64 * 4;
template <bool CAUSAL>
__global__ __launch_bounds__(256, 1) void attention_bwd_dkdv_kernel(
    const short *__restrict__ q, const short *__restrict__ k, const short *__restrict__ v,
    const short *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    short *__restrict__ dk, short *__restrict__ dv, int S, int Hq, int Hkv, int group, int nkb,
    int hkvtot, float scale_log2, float inv_sqrt_d) {
    constexpr int NW = 4, QPW = 4, kBK = 128;
    __shared__ __attribute__((aligned(1024))) char smem0[kBwdStageB];
    __shared__ __attribute__((aligned(1024))) char smem1[kBwdStageB];
    LDS_AS char *lds0 = (LDS_AS char *)smem0;
    LDS_AS char *lds1 = (LDS_AS char *)smem1;

    const int e = blockIdx.x;
    const int hk = e % hkvtot;
    const int kb = e / hkvtot;  // causal: the first key blocks have the most queries
    const int b = hk / Hkv, ck = hk - b * Hkv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int k0 = kb * kBK, wkey0 = k0 + 32 * w, key = wkey0 + (lane & 31);
    const int64_t qstride = int64_t(Hq) * kD, kstride = int64_t(Hkv) * kD;
    const int64_t koff = int64_t(b) * S * kstride + int64_t(ck) * kD;
    const int ntiles = (S + kBN - 1) / kBN;
    const int m0 = CAUSAL ? k0 / kBN : 0;  // first query tile with a visible pair

    TileDma<QPW> td;
    tile_dma_setup(td, w, lane, qstride);
    // requests of this wavefront's share of query tile m of query head c
    auto tile_req = [&](int c, int m, const LDS_AS char *dst, int r) __attribute__((always_inline)) {
        const int row0 = m * kBN, valid = min(S - row0, kBN);
        const int64_t off = int64_t(b) * S * qstride + int64_t(c) * kD + int64_t(row0) * qstride;
        const uint32_t d = uint32_t(reinterpret_cast<uintptr_t>(dst));
        if (r < QPW) dma16(tile_resource(q + off, valid, qstride), td.goff[r], d + td.m0[r]);
        else dma16(tile_resource(dout + off, valid, qstride), td.goff[r - QPW], d + kTileB + td.m0[r - QPW]);
    };
    // lse (base 2) and delta of query tile m of head c: lanes 0..31 of wavefront 0
    auto side_load = [&](int c, int m, f32x4 &x) __attribute__((always_inline)) {
        const int j = (lane & 15) * 4, row = m * kBN + j;
        const float *src = (lane < 16 ? lse : delta) + (int64_t(b) * Hq + c) * S;
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = row + u < S ? src[row + u] : 0.f;
        if (lane < 16) x *= kLog2e;
    };
    auto side_store = [&](const f32x4 &x, LDS_AS char *dst) __attribute__((always_inline)) {
        *reinterpret_cast<LDS_AS f32x4 *>(dst + 2 * kTileB + (lane >> 4) * 256 + (lane & 15) * 16) = x;
    };
    if (S % kBN != 0) {  // ragged last tile: Q and dO rows past the end start at zero
#pragma unroll
        for (int i = 0; i < 2 * kTileB / (16 * 64 * NW); ++i) {
            const int off = (i * 64 * NW + int(threadIdx.x)) * 16;
            *reinterpret_cast<LDS_AS s16x8 *>(lds0 + off) = s16x8{};
            *reinterpret_cast<LDS_AS s16x8 *>(lds1 + off) = s16x8{};
        }
        __syncthreads();
    }

    LdsOff lo;
    lds_offsets(lo, lane);
    s16x8 kr[8], vr[8];
    const int crow = min(key, S - 1);
    load_row_operand(kr, k + koff + int64_t(crow) * kstride, lane);
    load_row_operand(vr, v + koff + int64_t(crow) * kstride, lane);
    f32x16 dka[4], dva[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) { dka[mt] = f32x16{}; dva[mt] = f32x16{}; }

    // steps run over (query head c of the group, query tile m), m fastest,
    // stages alternating; (c, m) advance by increments (no division, so the
    // tile addresses stay scalar)
    const int clast = ck * group + group - 1;
    int c = ck * group, m = m0;
#pragma unroll
    for (int r = 0; r < 2 * QPW; ++r) tile_req(c, m, lds0, r);
    if (w == 0 && lane < 32) {
        f32x4 x;
        side_load(c, m, x);
        side_store(x, lds0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    auto step = [&](LDS_AS char *cur, LDS_AS char *nxt) __attribute__((always_inline)) -> bool {
        const bool last_m = m + 1 == ntiles;
        const bool more = !(last_m && c == clast);
        // the next step's tile (the current one again after the last step)
        const int c1 = more && last_m ? c + 1 : c;
        const int m1 = !more ? m : last_m ? m0 : m + 1;
        // the next tile's resources first, so that its addresses are formed
        // outside the single-wavefront branch below; the requests themselves
        // are spread over the first half's products (one per two products)
        const int nrow0 = m1 * kBN, nvalid = min(S - nrow0, kBN);
        const int64_t noff = int64_t(b) * S * qstride + int64_t(c1) * kD + int64_t(nrow0) * qstride;
        const i32x4 rq = tile_resource(q + noff, nvalid, qstride);
        const i32x4 rd = tile_resource(dout + noff, nvalid, qstride);
        const uint32_t nd = uint32_t(reinterpret_cast<uintptr_t>(nxt));
        auto req = [&](int r) __attribute__((always_inline)) {
            if (r < QPW) dma16(rq, td.goff[r], nd + td.m0[r]);
            else dma16(rd, td.goff[r - QPW], nd + kTileB + td.m0[r - QPW]);
        };
        f32x4 side;
        if (w == 0 && lane < 32) side_load(c1, m1, side);
        const LDS_AS char *qt = cur, *dt = cur + kTileB;
        const LDS_AS float *ls = (const LDS_AS float *)(cur + 2 * kTileB);
        const LDS_AS float *dl = ls + 64;
        const int qt0 = m * kBN;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (CAUSAL && qt0 + 32 * t + 31 < wkey0) {  // every query of the half before every key
                if (t == 0) {
#pragma unroll
                    for (int r = 0; r < 2 * QPW; ++r) req(r);
                }
                continue;
            }
            // S and dP for queries qt0 + 32t .. +31 (lane: key row).  One
            // wavefront per SIMD: operands are read kA products ahead, and the
            // first kB operands of dV/dK are read before the vector work.
            constexpr int kA = 8, kB = 8;
            auto opA = [&](int i) __attribute__((always_inline)) {  // i = 2*cc + (0: Q rows, 1: dO rows)
                return rows_op(lo, (i & 1) ? dt : qt, 2 * (i >> 1) + t);
            };
            auto opB = [&](int i) __attribute__((always_inline)) {  // i = 2*(4h + mt) + (0: dO^T, 1: Q^T)
                return cols_op(lo, (i & 1) ? qt : dt, 8 * t + (i >> 1));
            };
            f32x16 sc = f32x16{}, dp = f32x16{};
            s16x8 a[16], bo[16];
#pragma unroll
            for (int i = 0; i < kA; ++i) a[i] = opA(i);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i + kA < 16) a[i + kA] = opA(i + kA);
                if (i & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], vr[i >> 1], dp, 0, 0, 0);
                else sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], kr[i >> 1], sc, 0, 0, 0);
                if (t == 0 && (i & 1)) req(i >> 1);
            }
#pragma unroll
            for (int i = 0; i < kB; ++i) bo[i] = opB(i);
#pragma unroll
            for (int i = 0; i < kA; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i + kA < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kB, 0);
            s16x8 pb[2], dsb[2];
            // queries past the end, or before this wavefront's last key (causal), need the mask
            const bool need_mask = qt0 + 32 * t + 31 >= S || (CAUSAL && qt0 + 32 * t < wkey0 + 31);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int j = 32 * t + 8 * g + 4 * (lane >> 5);
                const f32x4 l4 = *reinterpret_cast<const LDS_AS f32x4 *>(ls + j);
                const f32x4 d4 = *reinterpret_cast<const LDS_AS f32x4 *>(dl + j);
                if (need_mask) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = 4 * g + u, qi = qt0 + j + u;
                        const bool vis = qi < S && (!CAUSAL || qi >= key);
                        const float p = vis ? __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, -l4[u])) : 0.f;
                        pb[r >> 3][r & 7] = to_bf16(p);
                        dsb[r >> 3][r & 7] = to_bf16(vis ? p * (dp[r] - d4[u]) : 0.f);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = 4 * g + u;
                        const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, -l4[u]));
                        pb[r >> 3][r & 7] = to_bf16(p);
                        dsb[r >> 3][r & 7] = to_bf16(p * (dp[r] - d4[u]));
                    }
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS over these 32 queries
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i + kB < 16) bo[i + kB] = opB(i + kB);
                const int h = i >> 3, mt = (i >> 1) & 3;
                if (i & 1) dka[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bo[i], dsb[h], dka[mt], 0, 0, 0);
                else dva[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bo[i], pb[h], dva[mt], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i + kB < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
        if (w == 0 && lane < 32) side_store(side, nxt);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's DMA of the next tile
        __syncthreads();
        c = c1;
        m = m1;
        return more;
    };
    for (;;) {
        if (!step(lds0, lds1)) break;
        if (!step(lds1, lds0)) break;
    }
    if (key < S) {
        store_acc_row(dk + koff + int64_t(key) * kstride, dka, inv_sqrt_d, lane);
        store_acc_row(dv + koff + int64_t(key) * kstride, dva, 1.f, lane);
    }
}

}  // namespace

hipError_t launch_attention_bwd_bf16_d128(const void *q, const void *k, const void *v,
                                          const void *o, const void *dout, const float *lse,
                                          float *delta, void *dq, void *dk, void *dv, int64_t B,
                                          int64_t S, int64_t Hq, int64_t Hkv, bool causal,
                                          hipStream_t st) {
    const float scale_log2 = float(1.4426950408889634 / 11.313708498984761);  // log2(e)/sqrt(128)
    const float inv_sqrt_d = float(1.0 / 11.313708498984761);
    const auto *qs = static_cast<const short *>(q), *ks = static_cast<const short *>(k),
               *vs = static_cast<const short *>(v), *os = static_cast<const short *>(o),
               *ds = static_cast<const short *>(dout);
    const int64_t rows = B * S * Hq;
    hipLaunchKernelGGL(attention_delta_kernel, dim3(uint32_t((rows * 16 + 255) / 256)), dim3(256), 0, st,
                       os, ds, delta, int(S), int(Hq), rows);
    const int nqb = int((S + 255) / 256), htot = int(B * Hq);
    const dim3 gq(uint32_t(int64_t(nqb) * htot));
    if (causal)
        hipLaunchKernelGGL(attention_bwd_dq_kernel<true>, gq, dim3(512), 0, st, qs, ks, vs, ds, lse,
                           delta, static_cast<short *>(dq), int(S), int(Hq), int(Hkv), int(Hq / Hkv),
                           nqb, htot, scale_log2, inv_sqrt_d);
    else
        hipLaunchKernelGGL(attention_bwd_dq_kernel<false>, gq, dim3(512), 0, st, qs, ks, vs, ds, lse,
                           delta, static_cast<short *>(dq), int(S), int(Hq), int(Hkv), int(Hq / Hkv),
                           nqb, htot, scale_log2, inv_sqrt_d);
    const int nkb = int((S + 127) / 128), hkvtot = int(B * Hkv);
    const dim3 gk(uint32_t(int64_t(nkb) * hkvtot));
    if (causal)
        hipLaunchKernelGGL(attention_bwd_dkdv_kernel<true>, gk, dim3(256), 0, st, qs, ks, vs, ds, lse,
                           delta, static_cast<short *>(dk), static_cast<short *>(dv), int(S), int(Hq),
                           int(Hkv), int(Hq / Hkv), nkb, hkvtot, scale_log2, inv_sqrt_d);
    else
        hipLaunchKernelGGL(attention_bwd_dkdv_kernel<false>, gk, dim3(256), 0, st, qs, ks, vs, ds, lse,
                           delta, static_cast<short *>(dk), static_cast<short *>(dv), int(S), int(Hq),
                           int(Hkv), int(Hq / Hkv), nkb, hkvtot, scale_log2, inv_sqrt_d);
    return hipGetLastError();
}

}  // namespace uly
