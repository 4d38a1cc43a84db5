// The bf16 attention kernel template and its launch helpers, shared by
// attention_bf16.hip (256-row and key-split blocks, the launch choice, the
// split plan and merge) and attention_bf16_chs.hip (the chain-split
// instantiations, built with their own instruction-scheduler setting).
// The design notes are at the top of attention_bf16.hip.
#pragma once

#include <algorithm>
#include <functional>
#include <cmath>
#include <mutex>
#include <queue>
#include <type_traits>
#include <vector>
#include "attn_tiles.h"

namespace uly {

// Unit table of the split forward, passed by value as a kernel argument:
// entry i = query block << 16 | unit << 8 | units of that block.
constexpr int kSplitMaxUnits = 512;     // entries per head
constexpr int kSplitRows = 64;          // query rows per block (chain split)
constexpr int kSplitSlot = kSplitRows * (tiles::kD + 1);  // floats per unit: o rows, then lse
struct SplitTable {
    float *ws;  // workspace: [B*Hq][nqb][umax] slots
    int umax;   // slots per query block
    uint32_t unit[kSplitMaxUnits];
};

namespace {

using namespace tiles;

// Workgroups of 8 wavefronts own 256 query rows where the grid fills the GPU,
// or 128 rows with the key split (KS = 2, twice the workgroups) for short
// sequences and for causal grids that 256-row blocks would leave unbalanced,
// or 64 rows with the key and chain splits (four wavefronts per 32 rows)
// where even 128-row blocks leave CUs idle (launch_any).
constexpr float kRescaleSlack = 8.f; // base-2 headroom before the running max moves

struct NoSplit {  // the same members, never read
    float *ws = nullptr;
    int umax = 0;
};
template <bool SPLIT> using SplitArg = typename std::conditional<SPLIT, SplitTable, NoSplit>::type;

struct Frag {
    s16x8 q[8];          // this wavefront's 32 query rows, B-operand layout
    f32x16 o[4];         // O^T accumulators, d blocks of 32
    float lsum;          // this lane's share of its row's sum of bf16 weights
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
// requests for the next tile, spread over the Q.K products.  PIN: the issue
// order of reads and products below; otherwise the compiler's own
// interleaving of matrix products and LDS reads (iglp_opt(0)).  Measured on
// MI355X, alternating libraries, same outputs bit for bit: for 256-row
// blocks the compiler's order is faster (32768 tokens, 4 heads: causal 910.6
// vs 915.5 us, non-causal 1743.4 vs 1763.6; 65536 with one key/value head
// 3577.3 vs 3602.3), for the key split's 128-row blocks slower (16384
// tokens, causal: 258.6 vs 255.4 us).
template <bool CAUSAL, int NREQ, bool PIN, typename Req>
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
    if constexpr (PIN) {
#pragma unroll
        for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i + kAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
    } else {
        __builtin_amdgcn_iglp_opt(0);
    }

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
        f.lsum *= alpha;
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
    // the row sum of the same bf16 weights, two per instruction
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const s16x2 ones2 = {short(0x3F80), short(0x3F80)};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                f.lsum = __builtin_amdgcn_fdot2_f32_bf16(s16x2{pk[t][h][2 * j], pk[t][h][2 * j + 1]}, ones2, f.lsum, false);

    // O^T += V^T P^T: 16 products, key step (t, h) = (i/8, i/4 % 2) and d block
    // mt = i % 4, operands read four ahead.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i + kAhead < 16) vf[i + kAhead] = read_v(f, vt, i + kAhead);
        const int t = i >> 3, h = (i >> 2) & 1, mt = i & 3;
        f.o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pk[t][h], f.o[mt], 0, 0, 0);
    }
}

// K fragment (d chunk cc) and V operand i (key step h = i/4 % 2, d block
// mt = i % 4) of 32-key chain `chain`: register indices stay compile-time
// constants (a run-time index would move the offset arrays to scratch).
__device__ __forceinline__ s16x8 read_k_chain(const Frag &f, const LDS_AS char *kt, int cc, int chain) {
    return *reinterpret_cast<const LDS_AS s16x8 *>(kt + f.koff[cc] + chain * 32 * kRowB);
}
__device__ __forceinline__ s16x8 read_v_chain(const Frag &f, const LDS_AS char *vt, int i, int chain) {
    const int h = (i >> 2) & 1, mt = i & 3;
    const int rowoff = (32 * chain + 16 * h) * kRowB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(vt + f.voff[0][mt] + rowoff));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(vt + f.voff[1][mt] + rowoff));
    return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// tile_step for one of the tile's two 32-key chains (keys key0 + 32 * chain
// .. +31): 8 products for S^T and 8 for O^T, the softmax over those keys only.
// Two wavefronts that share their query rows take the two chains of every
// tile; their states are combined at the end like the key split's halves.
template <bool CAUSAL, int NREQ, typename Req>
__device__ __forceinline__ void tile_step_chain(Frag &f, const LDS_AS char *kt, const LDS_AS char *vt,
                                                int key0, int chain, int wrow0, int qrow, int S,
                                                float scale_log2, int lane, Req &&req) {
    const int ckey0 = key0 + 32 * chain;
    if (CAUSAL && ckey0 > wrow0 + 31) {  // every key of the chain is after every row
#pragma unroll
        for (int r = 0; r < NREQ; ++r) req(r);
        return;
    }
    constexpr int kReqStride = 8 / NREQ > 0 ? 8 / NREQ : 1;
    constexpr int kAhead = 4;
    f32x16 s = f32x16{};
    {
        s16x8 kf[8];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) kf[i] = read_k_chain(f, kt, i, chain);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i + kAhead < 8) kf[i + kAhead] = read_k_chain(f, kt, i + kAhead, chain);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], f.q[i], s, 0, 0, 0);
            if (i % kReqStride == 0 && i / kReqStride < NREQ) req(i / kReqStride);
        }
    }
    s16x8 vf[8];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) vf[i] = read_v_chain(f, vt, i, chain);
#pragma unroll
    for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kAhead < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);

    const bool need_mask = (CAUSAL && ckey0 + 31 > wrow0) || ckey0 + 32 > S;
    if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = ckey0 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            const bool hidden = key >= S || (CAUSAL && key > qrow);
            s[r] = hidden ? -INFINITY : s[r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > f.m + kRescaleSlack)) {  // wavefront-uniform
        const float mnew = fmaxf(f.m, mx);
        const float alpha = __builtin_amdgcn_exp2f(f.m - mnew);
        f.m = mnew;
        f.lsum *= alpha;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) f.o[mt][r] *= alpha;
    }
    const float mnew = f.m;
    s16x8 pk[2];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        pk[r >> 3][r & 7] = to_bf16(__builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -mnew)));
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const s16x2 ones2 = {short(0x3F80), short(0x3F80)};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            f.lsum = __builtin_amdgcn_fdot2_f32_bf16(s16x2{pk[h][2 * j], pk[h][2 * j + 1]}, ones2, f.lsum, false);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i + kAhead < 8) vf[i + kAhead] = read_v_chain(f, vt, i + kAhead, chain);
        const int h = (i >> 2) & 1, mt = i & 3;
        f.o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pk[h], f.o[mt], 0, 0, 0);
    }
}

// CHUNK: queries (Sq rows) and keys (skv rows) of different lengths, key j
// visible to row i under the causal mask iff j <= i + delta (delta = the
// query block's global position minus the key chunk's); rows with no visible
// key get o = 0 and lse = -inf.  Without CHUNK, skv = Sq and delta = 0 are
// compile-time facts.
//
// KS = 2 (key split): the NW wavefronts own 32*NW/2 query rows, wavefronts w
// and w + NW/2 the same 32; the first half takes the even key tiles, the
// second the odd ones (each half streams its own two LDS stages), and the two
// partial states (running max, row sum, unnormalised output) are combined
// through LDS at the end.  Twice the blocks of the same size at two
// wavefronts per SIMD, and half the serial tile chain per block.
//
// ACC (chunk calls only): o and lse hold a running result over earlier key
// chunks; the epilogue merges this chunk's rows into it (weights by each
// side's share of the total exp-sum) instead of overwriting, and leaves rows
// this chunk does not reach untouched.
//
// PIECES (full-sequence calls only): q, k, v are read and o is written in
// the order the exchange delivers and sends them, [P][B][S/P][h][D] (one
// piece of S/P token rows per peer rank, batch entries inside each piece),
// instead of [B][S][h][D]: token s of batch entry b is row
// b*sp + s + (s / sp) * gap with sp = S/P and gap = (B-1)*sp.  Key tiles
// never straddle two pieces (sp is a multiple of the tile height), so a tile
// is still one strided block.
//
// SPLIT (with CHS, full sequence): the key tiles of a 64-row query block may
// be cut into units of consecutive tiles, one workgroup per unit.  Workgroup
// e takes head e mod (B*Hq) and entry e / (B*Hq) of the unit table (longest
// unit first): query block, unit index and unit count.  A block of one unit
// writes o (and lse) as usual; the units of a longer block write their rows'
// normalised fp32 output and log-sum-exp to the workspace, for the merge
// (split_merge_kernel, the next launch).
template <bool CAUSAL, int NW, bool CHUNK, int KS, bool ACC, bool PIECES = false, bool CHS = false,
          bool SPLIT = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attention_bf16_d128_kernel(
    const short *__restrict__ q, const short *__restrict__ k, const short *__restrict__ v,
    short *__restrict__ o, float *__restrict__ lse, int Sq, int skv, int delta_arg, int Hq,
    int Hkv, int group, int nqb, int htot, int paired, float scale_log2, FastDiv by_sp,
    int64_t gap, SplitArg<SPLIT> spl) {
    const int S = Sq;                        // query rows
    const int Skv = CHUNK ? skv : Sq;        // key rows
    const int delta = CHUNK ? delta_arg : 0; // causal diagonal offset
    __shared__ __attribute__((aligned(1024))) char smem0[kStageB];
    __shared__ __attribute__((aligned(1024))) char smem1[kStageB];
    __shared__ __attribute__((aligned(1024))) char smem2[KS == 2 ? kStageB : 16];
    __shared__ __attribute__((aligned(1024))) char smem3[KS == 2 ? kStageB : 16];
    LDS_AS char *lds0 = (LDS_AS char *)smem0;
    LDS_AS char *lds1 = (LDS_AS char *)smem1;
    LDS_AS char *lds2 = (LDS_AS char *)smem2;
    LDS_AS char *lds3 = (LDS_AS char *)smem3;
    constexpr int WH = NW / KS;  // wavefronts per key half
    // CHS (chain split, with the key split): the two 32-key chains of every
    // tile go to two wavefronts that share their query rows, so a key half has
    // WH / 2 row slots of 32 rows
    static_assert(!CHS || (KS == 2 && NW == 8), "chain split: 8 wavefronts with the key split");
    static_assert(!SPLIT || (CHS && !CHUNK && !ACC && !PIECES), "split: chain-split full-sequence blocks");
    constexpr int RS = CHS ? WH / 2 : WH;  // row slots

    const int e = blockIdx.x;
    const int hh = e % htot;
    constexpr int kBM = 32 * RS;  // query rows per workgroup
    static_assert(!SPLIT || kBM == kSplitRows, "split: 64-row blocks");
    // Causal, paired: workgroup i takes query blocks nqb-1-i and then i, so
    // that every workgroup streams the same number of tiles.
    const int pi = e / htot;
    const int npass = CAUSAL && paired && nqb - 1 - pi != pi ? 2 : 1;
    // ragged last tile: the V stages start at zero, so that no stale LDS
    // content can reach a sum through the rows past the end
    auto zero_v_stages = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kTileB / (16 * 64 * NW); ++i) {
            const int off = (i * 64 * NW + int(threadIdx.x)) * 16;
            *reinterpret_cast<LDS_AS s16x8 *>(lds0 + kTileB + off) = s16x8{};
            *reinterpret_cast<LDS_AS s16x8 *>(lds1 + kTileB + off) = s16x8{};
            if (KS == 2) {
                *reinterpret_cast<LDS_AS s16x8 *>(lds2 + kTileB + off) = s16x8{};
                *reinterpret_cast<LDS_AS s16x8 *>(lds3 + kTileB + off) = s16x8{};
            }
        }
        __syncthreads();
    };
    if (Skv % kBN != 0) zero_v_stages();
    for (int pass = 0; pass < npass; ++pass) {
        int qb = CAUSAL ? (pass == 0 ? nqb - 1 - pi : pi) : pi;
        int unit = 0, nunits = 1;  // split: this workgroup's unit of its block
        if constexpr (SPLIT) {
            const uint32_t u = spl.unit[pi];
            qb = int(u >> 16);
            unit = int((u >> 8) & 255u);
            nunits = int(u & 255u);
        }
        const int b = hh / Hq, c = hh - b * Hq, ck = c / group;
        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        const int wh = KS == 2 ? wv % WH : wv;    // wavefront within its key half
        const int w = CHS ? wh % RS : wh;         // row slot of this wavefront
        const int chain = CHS ? __builtin_amdgcn_readfirstlane(wh / RS) : 0;  // key chain (CHS)
        // key tiles half, half + KS, ... (wavefront-uniform: scalar, so that the
        // DMA's LDS address can go to M0)
        const int half = KS == 2 ? __builtin_amdgcn_readfirstlane(wv / WH) : 0;
        LDS_AS char *st0 = half ? lds2 : lds0;    // this half's two stages
        LDS_AS char *st1 = half ? lds3 : lds1;
        const int q0 = qb * kBM;
        const int wrow0 = q0 + 32 * w;
        const int qrow = wrow0 + (lane & 31);
        const int64_t qstride = int64_t(Hq) * kD, kstride = int64_t(Hkv) * kD;
        // first row of batch entry b, and the row of its token s past that
        const int64_t qb0 = int64_t(b) * (PIECES ? int64_t(by_sp.d) : int64_t(S));
        const int64_t kb0 = int64_t(b) * (PIECES ? int64_t(by_sp.d) : int64_t(Skv));
        auto row_of = [&](int s) __attribute__((always_inline)) -> int64_t {
            return PIECES ? int64_t(s) + int64_t(by_sp.div(uint32_t(s))) * gap : int64_t(s);
        };
        const short *qh = q + qb0 * qstride + int64_t(c) * kD;
        const short *kh = k + kb0 * kstride + int64_t(ck) * kD;
        const short *vh = v + kb0 * kstride + int64_t(ck) * kD;
        short *oh = o + qb0 * qstride + int64_t(c) * kD;

        const int kend = CAUSAL ? min(Skv, max(0, q0 + kBM + delta)) : Skv;
        const int ntiles = (kend + kBN - 1) / kBN;
        // this workgroup's tiles t_lo .. t_lo + span - 1 (all of them unless split)
        const int t_lo = SPLIT ? unit * ntiles / nunits : 0;
        const int span = SPLIT ? (unit + 1) * ntiles / nunits - t_lo : ntiles;
        if (CHUNK && ntiles == 0) {  // no key of the chunk is visible to any row of the block
            if (!ACC && qrow < S && half == 0 && chain == 0) {
                if (lse && lane < 32) lse[int64_t(hh) * S + qrow] = -INFINITY;
                short *op = oh + row_of(qrow) * qstride;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<s16x4 *>(op + 32 * mt + 8 * g + 4 * (lane >> 5)) = s16x4{};
            }
            continue;  // uniform over the workgroup
        }

        constexpr int QPW = 16 / WH;
        TileDma<QPW> td;
        tile_dma_setup(td, wh, lane, kstride);
        // requests of this wavefront's share of tile n (K and V) into stage dst
        auto tile_req = [&](int n, const LDS_AS char *dst, int r) __attribute__((always_inline)) {
            const int row0 = n * kBN;
            const int valid = min(Skv - row0, kBN);
            const uint32_t d = uint32_t(reinterpret_cast<uintptr_t>(dst));
            const int64_t roff = row_of(row0) * kstride;
            if (r < QPW) dma16(tile_resource(kh + roff, valid, kstride), td.goff[r], d + td.m0[r]);
            else dma16(tile_resource(vh + roff, valid, kstride), td.goff[r - QPW],
                       d + kTileB + td.m0[r - QPW]);
        };
        // the second block of a pair walks its keys downwards: it starts as
        // many tiles after the first blocks of the other workgroups as its
        // diagonal lies further along, so they all read the same tile at once
        const bool down = pass == 1;
        // this half's i-th tile (with the key split clamped into range, so a
        // half without tiles still requests a valid one, which nobody reads)
        const int nt = (span - half + KS - 1) / KS;  // tiles of this half
        auto tile_of = [&](int i) __attribute__((always_inline)) {
            int n = KS * i + half;
            if (KS > 1) n = max(0, min(n, span - 1));
            return down ? ntiles - 1 - n : t_lo + n;
        };
#pragma unroll
        for (int r = 0; r < 2 * QPW; ++r) tile_req(tile_of(0), st0, r);

        Frag f;
        {
            const short *qp = qh + row_of(min(qrow, S - 1)) * qstride + 8 * (lane >> 5);
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) f.q[cc] = *reinterpret_cast<const s16x8 *>(qp + 16 * cc);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) f.o[mt] = f32x16{};
            f.m = -1e30f;
            f.lsum = 0.f;
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

        const int nsteps = (span + KS - 1) / KS;  // = nt of the first half
        auto step = [&](int n, LDS_AS char *cur, LDS_AS char *nxt) __attribute__((always_inline)) -> bool {
            const bool more = n + 1 < nsteps;
            // tile n+1 into the other stage (after the last tile: the last tile
            // again, into the stage nobody reads any more)
            const int n1 = tile_of(min(n + 1, nt - 1));
            auto req = [&](int r) __attribute__((always_inline)) { tile_req(n1, nxt, r); };
            if (CHS && n < nt)
                tile_step_chain<CAUSAL, 2 * QPW>(f, cur, cur + kTileB, tile_of(n) * kBN, chain, wrow0 + delta,
                                                 qrow + delta, Skv, scale_log2, lane, req);
            else if (!CHS && (KS == 1 || n < nt))
                tile_step<CAUSAL, 2 * QPW, KS == 2>(f, cur, cur + kTileB, tile_of(n) * kBN, wrow0 + delta,
                                                    qrow + delta, Skv, scale_log2, lane, req);
            else  // the second half past its last tile
#pragma unroll
                for (int r = 0; r < 2 * QPW; ++r) req(r);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's DMA of tile n+1
            __syncthreads();
            return more;
        };
        for (int n = 0;; n += 2) {
            if (!step(n, st0, st1)) break;
            if (!step(n + 1, st1, st0)) break;
        }

        if (KS == 2) {
            // combine partial states: the parking wavefronts write their output
            // accumulators, max and row sum to LDS (every tile read and every
            // DMA has completed before the last barrier), the merging ones add
            // them in.  Key split: the second half parks for the first.  Chain
            // split: first chain 1 parks for chain 0 in each half, then the
            // halves as before.
            auto park_at = [&](int i) __attribute__((always_inline)) {
                return reinterpret_cast<LDS_AS float *>(i == 0 ? lds0 : i == 1 ? lds1 : i == 2 ? lds2 : lds3);
            };
            // (16-byte LDS accesses, lane-contiguous: four accumulators per instruction)
            auto combine = [&](bool parker, bool merger, LDS_AS float *park) __attribute__((always_inline)) {
                LDS_AS f32x4 *pk = reinterpret_cast<LDS_AS f32x4 *>(park);
                if (parker) {
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        pk[j * 64 + lane] = f32x4{f.o[j >> 2][4 * (j & 3)], f.o[j >> 2][4 * (j & 3) + 1],
                                                  f.o[j >> 2][4 * (j & 3) + 2], f.o[j >> 2][4 * (j & 3) + 3]};
                    park[64 * 64 + lane] = f.m;
                    park[65 * 64 + lane] = f.lsum;
                }
                __syncthreads();
                if (merger) {
                    const float m1 = park[64 * 64 + lane], l1 = park[65 * 64 + lane];
                    const float mn = fmaxf(f.m, m1);
                    const float a0 = __builtin_amdgcn_exp2f(f.m - mn), a1 = __builtin_amdgcn_exp2f(m1 - mn);
                    f.m = mn;
                    f.lsum = f.lsum * a0 + l1 * a1;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const f32x4 p = pk[j * 64 + lane];
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            f.o[j >> 2][4 * (j & 3) + t] = f.o[j >> 2][4 * (j & 3) + t] * a0 + p[t] * a1;
                    }
                }
            };
            if (CHS) {
                combine(chain == 1, chain == 0, park_at(2 * half + w));
                __syncthreads();  // the first round's parks are read before the second's
                combine(chain == 0 && half == 1, chain == 0 && half == 0, park_at(w));
            } else {
                combine(half == 1, half == 0, park_at(w));
            }
        }

        // lanes l and l^32 hold the same row's two halves of the keys
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(f.lsum), __float_as_uint(f.lsum),
                                                         false, false);
        const float lrow = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if (ACC) {
            if (qrow < S && half == 0 && chain == 0 && lrow > 0.f) {
                // merge with the running result: lse = log(e^lse_old + e^lse_new),
                // o = e^(lse_old - lse) o_old + e^(lse_new - lse) o_new
                const float lnew = (f.m + __log2f(lrow)) * kLn2;
                const float lold = lse[int64_t(hh) * S + qrow];  // both lanes of the row read it first
                const float mx = fmaxf(lold, lnew);
                const float eo = expf(lold - mx), en = expf(lnew - mx);
                const float tot = eo + en;
                const float wo = eo / tot, wn = en / (tot * lrow);
                short *op = oh + row_of(qrow) * qstride;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        s16x4 *pp = reinterpret_cast<s16x4 *>(op + 32 * mt + 8 * g + 4 * (lane >> 5));
                        const s16x4 old = *pp;
                        s16x4 pv;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            pv[i] = to_bf16(fmaf(wo, bf16_to_f32(old[i]), wn * f.o[mt][4 * g + i]));
                        *pp = pv;
                    }
                if (lane < 32) lse[int64_t(hh) * S + qrow] = mx + logf(tot);
            }
        } else if (SPLIT && nunits > 1) {
            // this unit's rows for the merge: normalised fp32 output, then the
            // rows' natural-log sums of exp(scores)
            if (qrow < S && half == 0 && chain == 0) {
                float *slot = spl.ws + ((int64_t(hh) * nqb + qb) * spl.umax + unit) * kSplitSlot;
                float *orow = slot + (qrow - q0) * kD;
                const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<f32x4 *>(orow + 32 * mt + 8 * g + 4 * (lane >> 5)) =
                            f32x4{f.o[mt][4 * g] * inv, f.o[mt][4 * g + 1] * inv,
                                  f.o[mt][4 * g + 2] * inv, f.o[mt][4 * g + 3] * inv};
                if (lane < 32)
                    slot[kSplitRows * kD + (qrow - q0)] = lrow > 0.f ? (f.m + __log2f(lrow)) * kLn2 : -INFINITY;
            }
        } else {
        if (lse && qrow < S && lane < 32 && half == 0 && chain == 0)  // natural log of the row's sum of exp(scores)
            lse[int64_t(hh) * S + qrow] = (f.m + __log2f(lrow)) * kLn2;
        if (qrow < S && half == 0 && chain == 0) {
            const float inv = CHUNK && lrow == 0.f ? 0.f : 1.f / lrow;  // a row with no visible key: o = 0
            short *op = oh + row_of(qrow) * qstride;
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
        if (pass + 1 < npass) {
            __syncthreads();  // both stages are refilled for the next block
            // the key split's combine parked fp32 sums over the first V rows
            if (KS == 2 && Skv % kBN != 0) zero_v_stages();
        }
    }
}

}  // namespace

namespace {
template <bool CAUSAL, int NW, bool CHUNK, int KS, bool ACC = false, bool PIECES = false,
          bool CHS = false, bool SPLIT = false>
void launch_one(dim3 grid, hipStream_t st, const void *q, const void *k, const void *v, void *o,
                float *lse, int Sq, int Skv, int delta, int Hq, int Hkv, int nqb, int htot,
                int paired, float scale_log2, FastDiv by_sp = FastDiv(), int64_t gap = 0,
                const SplitArg<SPLIT> &spl = SplitArg<SPLIT>()) {
    hipLaunchKernelGGL((attention_bf16_d128_kernel<CAUSAL, NW, CHUNK, KS, ACC, PIECES, CHS, SPLIT>),
                       grid, dim3(NW * 64), 0, st, static_cast<const short *>(q),
                       static_cast<const short *>(k), static_cast<const short *>(v),
                       static_cast<short *>(o), lse, Sq, Skv, delta, Hq, Hkv, Hq / Hkv, nqb, htot,
                       paired, scale_log2, by_sp, gap, spl);
}

template <int NW, int KS, bool CHS = false>
hipError_t launch_nw(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                     int64_t Sq, int64_t Skv, int64_t delta, int64_t Hq, int64_t Hkv, bool causal,
                     bool chunk, bool acc, int64_t sp, int cus, hipStream_t st) {
    constexpr int rows = 32 * NW / KS / (CHS ? 2 : 1);  // query rows per block
    const int nqb = int((Sq + rows - 1) / rows);
    const int htot = int(B * Hq);
    const float scale_log2 = float(1.4426950408889634 / 11.313708498984761);  // log2(e)/sqrt(128)
    // causal: pair a long and a short query block per workgroup while the
    // pairs still cover every CU (one tail instead of a spread of lengths)
    const int paired = causal && int64_t((nqb + 1) / 2) * htot >= cus ? 1 : 0;
    const dim3 grid(uint32_t(int64_t(paired ? (nqb + 1) / 2 : nqb) * htot));
    const int sq = int(Sq), skv = int(Skv), dl = int(delta), hq = int(Hq), hkv = int(Hkv);
    if (acc) {
        if (causal)
            launch_one<true, NW, true, KS, true, false, CHS>(grid, st, q, k, v, o, lse, sq, skv, dl, hq, hkv, nqb, htot, paired, scale_log2);
        else
            launch_one<false, NW, true, KS, true, false, CHS>(grid, st, q, k, v, o, lse, sq, skv, dl, hq, hkv, nqb, htot, paired, scale_log2);
    } else if (chunk) {
        if (causal)
            launch_one<true, NW, true, KS, false, false, CHS>(grid, st, q, k, v, o, lse, sq, skv, dl, hq, hkv, nqb, htot, paired, scale_log2);
        else
            launch_one<false, NW, true, KS, false, false, CHS>(grid, st, q, k, v, o, lse, sq, skv, dl, hq, hkv, nqb, htot, paired, scale_log2);
    } else if (sp) {
        const FastDiv by_sp{uint32_t(sp)};
        const int64_t gap = (B - 1) * sp;
        if (causal)
            launch_one<true, NW, false, KS, false, true, CHS>(grid, st, q, k, v, o, lse, sq, sq, 0, hq, hkv, nqb, htot, paired, scale_log2, by_sp, gap);
        else
            launch_one<false, NW, false, KS, false, true, CHS>(grid, st, q, k, v, o, lse, sq, sq, 0, hq, hkv, nqb, htot, paired, scale_log2, by_sp, gap);
    } else {
        if (causal)
            launch_one<true, NW, false, KS, false, false, CHS>(grid, st, q, k, v, o, lse, sq, sq, 0, hq, hkv, nqb, htot, paired, scale_log2);
        else
            launch_one<false, NW, false, KS, false, false, CHS>(grid, st, q, k, v, o, lse, sq, sq, 0, hq, hkv, nqb, htot, paired, scale_log2);
    }
    return hipGetLastError();
}
}  // namespace

// chain-split launches and the split forward's merge (attention_bf16_chs.hip)
hipError_t launch_chain_split(const void *q, const void *k, const void *v, void *o, float *lse,
                              int64_t B, int64_t Sq, int64_t Skv, int64_t delta, int64_t Hq,
                              int64_t Hkv, bool causal, bool chunk, bool acc, int64_t sp, int cus,
                              hipStream_t st);
hipError_t launch_split_units(dim3 grid, hipStream_t st, const void *q, const void *k, const void *v,
                              void *o, float *lse, int S, int Hq, int Hkv, int nqb, int htot,
                              bool causal, const SplitTable &t);
hipError_t launch_split_merge(const float *ws, void *o, float *lse, int S, int Hq, int nqb, int umax,
                              int ctiles, int first, int htot, bool causal, hipStream_t st);

}  // namespace uly
