// Gradients of one rank's local attention, bf16 in / bf16 out, head_dim 128,
// on gfx950 matrix cores.
//
// The backward pass runs the layout changes in reverse ("Sequence Parallelism
// II: DeepSpeed Ulysses and All-to-All Attention", section 6); between them
// sits the derivative of the local attention (attention_bf16.hip).  With lse_i the natural log of row i's sum of
// exp(scores) (written by the forward), p = exp(s - lse_i), and
// delta_i = sum_d dO[i,d] O[i,d]:
//   dS = p (dO.v - delta_i),  dQ += dS k / sqrt(D),  dK += dS q / sqrt(D),  dV += p dO.
// Three kernels: delta (one pass over O and dO), dQ (each wavefront owns 32
// query rows and streams the key/value tiles, as the forward), and dK/dV
// (two wavefronts per 32 key rows, each taking one half of every query tile,
// streaming the query, dO, lse and delta tiles of every query head of its kv
// head).  The products reuse the forward's
// operand forms: a row-major LDS tile read as an A operand whose rows are the
// tile rows (rows_op), or transposed so that its rows are the 128 columns
// (cols_op), and score-layout weights packed to bf16 as the B operand.
//
// PIECES (full sequence): every tensor in the order the exchanges deliver
// and send it, [P][B][S/P][h][D]; token s of batch entry b is row
// b*sp + s + (s / sp) * gap (sp = S/P, gap = (B-1)*sp), mapped once per row
// and once per 64-row tile (sp is a multiple of 64, so a tile never spans
// two pieces), as in the forward.
//
// The same kernels give the gradient contributions of one key/value chunk
// visit past the head-count bound (section 8 of the same page): query rows
// and keys counted separately, the causal diagonal moved by the two blocks'
// position offset, the merged lse and output of the whole ring, and the
// results written or added to the gradients of earlier visits.
//
// Split gradients (ulysses_attention_local_backward_split): at short lengths
// or with grouped heads the longest dK/dV blocks bound the single launch, so
// their query streams are cut into units on several workgroups (DkdvUnit),
// whose fp32 sums a short second launch (dkdv_split_sum_kernel) adds in unit
// order.
#include <algorithm>
#include <cmath>
#include <functional>
#include <queue>
#include <vector>

#include "attn_tiles.h"

namespace uly {
namespace {

using namespace tiles;

// delta[b][c][i] = sum_d dO[b][i][c][d] * O[b][i][c][d]; 16 lanes per row.
template <bool PIECES>
__global__ __launch_bounds__(256) void attention_delta_kernel(const short *__restrict__ o,
                                                              const short *__restrict__ dout,
                                                              float *__restrict__ delta, int S,
                                                              int Hq, int64_t rows, int B, int sp) {
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
        int64_t b;
        int i;
        if (PIECES) {  // bi = (piece * B + b) * sp + t
            const int64_t pb = bi / sp;
            const int t = int(bi - pb * sp);
            const int64_t piece = pb / B;
            b = pb - piece * B;
            i = int(piece * sp + t);
        } else {
            b = bi / S;
            i = int(bi - b * S);
        }
        delta[(b * Hq + c) * S + i] = acc;
    }
}

// As store_acc_row, but added to the bf16 values already in the row (fp32
// sum, rounded once): the contributions of successive key/value chunks.
__device__ __forceinline__ void add_acc_row(short *row, const f32x16 (&a)[4], float scale, int lane) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            s16x4 *p = reinterpret_cast<s16x4 *>(row + 32 * mt + 8 * g + 4 * (lane >> 5));
            const s16x4 old = *p;
            s16x4 pv;
#pragma unroll
            for (int u = 0; u < 4; ++u) pv[u] = to_bf16(fmaf(a[mt][4 * g + u], scale, bf16_to_f32(old[u])));
            *p = pv;
        }
}

// dQ: workgroup of 8 wavefronts = 256 query rows of one head (128 rows with
// the key split); the key/value tiles stream through two LDS stages as in the
// forward.
// (The body takes its workgroup index e and its LDS stages, so that one launch
// can also run dQ and dK/dV workgroups side by side: attention_bwd_fused_kernel.)
template <bool CAUSAL, bool CHUNK, int KS, bool PIECES>
__device__ __forceinline__ void dq_body(
    int e, LDS_AS char *lds0, LDS_AS char *lds1, LDS_AS char *lds2, LDS_AS char *lds3,
    const short *__restrict__ q, const short *__restrict__ k, const short *__restrict__ v,
    const short *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    short *__restrict__ dq, int S, int skv, int delta_arg, int acc_arg, int Hq, int Hkv, int group,
    int nqb, int htot, int paired, float scale_log2, float inv_sqrt_d, FastDiv by_sp, int64_t gap) {
    // CHUNK: S query rows against skv keys, key j visible to row i under the
    // causal mask iff j <= i + dpos; with accumulate the result is added to dq
    const int Skv = CHUNK ? skv : S;
    const int dpos = CHUNK ? delta_arg : 0;
    const bool accum = CHUNK && acc_arg != 0;
    // KS = 2 (key split, as in the forward): wavefronts w and w + 4 own the
    // same 32 rows of a 128-row block and take the even / odd key tiles through
    // their own two LDS stages; their dQ sums are added through LDS at the end
    constexpr int NW = 8, WH = NW / KS, QPW = 16 / WH, kBM = 32 * WH;
    // ragged last tile: K and V rows past the end start at zero
    auto zero_stages = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kStageB / (16 * 64 * NW); ++i) {
            const int off = (i * 64 * NW + int(threadIdx.x)) * 16;
            *reinterpret_cast<LDS_AS s16x8 *>(lds0 + off) = s16x8{};
            *reinterpret_cast<LDS_AS s16x8 *>(lds1 + off) = s16x8{};
            if (KS == 2) {
                *reinterpret_cast<LDS_AS s16x8 *>(lds2 + off) = s16x8{};
                *reinterpret_cast<LDS_AS s16x8 *>(lds3 + off) = s16x8{};
            }
        }
        __syncthreads();
    };
    if (Skv % kBN != 0) zero_stages();

    const int hh = e % htot;
    // causal, paired: workgroup i takes query blocks nqb-1-i and then i
    const int pi = e / htot;
    const int npass = CAUSAL && paired && nqb - 1 - pi != pi ? 2 : 1;
    for (int pass = 0; pass < npass; ++pass) {
        const int qb = CAUSAL ? (pass == 0 ? nqb - 1 - pi : pi) : pi;
        const int b = hh / Hq, c = hh - b * Hq, ck = c / group;
        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        const int w = KS == 2 ? wv % WH : wv;  // row slot of this wavefront
        // key tiles half, half + KS, ... (scalar, so that the DMA's LDS address can go to M0)
        const int half = KS == 2 ? __builtin_amdgcn_readfirstlane(wv / WH) : 0;
        LDS_AS char *st0 = half ? lds2 : lds0;  // this half's two stages
        LDS_AS char *st1 = half ? lds3 : lds1;
        const int q0 = qb * kBM, wrow0 = q0 + 32 * w, qrow = wrow0 + (lane & 31);
        const int64_t qstride = int64_t(Hq) * kD, kstride = int64_t(Hkv) * kD;
        // first row of batch entry b, and the row of its token s past that
        auto row_of = [&](int s_) __attribute__((always_inline)) -> int64_t {
            return PIECES ? int64_t(s_) + int64_t(by_sp.div(uint32_t(s_))) * gap : int64_t(s_);
        };
        const int64_t bq = int64_t(b) * (PIECES ? int64_t(by_sp.d) : int64_t(S));
        const int64_t bk = int64_t(b) * (PIECES ? int64_t(by_sp.d) : int64_t(Skv));
        const int64_t qoff = bq * qstride + int64_t(c) * kD;
        const short *kh = k + bk * kstride + int64_t(ck) * kD;
        const short *vh = v + bk * kstride + int64_t(ck) * kD;
        const int kend = CAUSAL ? min(Skv, max(0, q0 + kBM + dpos)) : Skv;
        const int ntiles = (kend + kBN - 1) / kBN;
        if (CHUNK && ntiles == 0) {  // no key of the chunk reaches the block: a zero contribution
            if (qrow < S && !accum && half == 0) {
                f32x16 zero[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
                store_acc_row(dq + qoff + row_of(qrow) * qstride, zero, 1.f, lane);
            }
            continue;  // uniform over the workgroup
        }

        TileDma<QPW> td;
        tile_dma_setup(td, w, lane, kstride);
        auto tile_req = [&](int n, const LDS_AS char *dst, int r) __attribute__((always_inline)) {
            const int row0 = n * kBN, valid = min(Skv - row0, kBN);
            const uint32_t d = uint32_t(reinterpret_cast<uintptr_t>(dst));
            const int64_t roff = row_of(row0) * kstride;
            if (r < QPW) dma16(tile_resource(kh + roff, valid, kstride), td.goff[r], d + td.m0[r]);
            else dma16(tile_resource(vh + roff, valid, kstride), td.goff[r - QPW],
                       d + kTileB + td.m0[r - QPW]);
        };
        // the second block of a pair walks its keys downwards, in step with
        // the second blocks of the other workgroups (as in the forward); this
        // half's i-th tile, clamped into range with the key split
        const bool down = pass == 1;
        const int nt = (ntiles - half + KS - 1) / KS;  // tiles of this half
        auto tile_of = [&](int i) __attribute__((always_inline)) {
            int n = KS * i + half;
            if (KS > 1) n = max(0, min(n, ntiles - 1));
            return down ? ntiles - 1 - n : n;
        };
#pragma unroll
        for (int r = 0; r < 2 * QPW; ++r) tile_req(tile_of(0), st0, r);

        LdsOff lo;
        lds_offsets(lo, lane);
        s16x8 qr[8], dor[8];
        const int crow = min(qrow, S - 1);
        load_row_operand(qr, q + qoff + row_of(crow) * qstride, lane);
        load_row_operand(dor, dout + qoff + row_of(crow) * qstride, lane);
        const float lse2 = lse[int64_t(hh) * S + crow] * kLog2e;
        const float dlt = delta[int64_t(hh) * S + crow];
        f32x16 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x16{};
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();

        const int nsteps = (ntiles + KS - 1) / KS;
        auto step = [&](int n, LDS_AS char *cur, LDS_AS char *nxt) __attribute__((always_inline)) -> bool {
            const bool more = n + 1 < nsteps;
            const int n1 = tile_of(min(n + 1, nt - 1));
            const int key0 = tile_of(n) * kBN;
            const LDS_AS char *kt = cur, *vt = cur + kTileB;
            const bool mine = KS == 1 || n < nt;  // the second half may have one tile fewer
            if (!mine || (CAUSAL && key0 > wrow0 + 31 + dpos)) {
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
                        // this wavefront's 2*QPW requests for the next tile, spread over the products
                        constexpr int kSpread = 16 / (2 * QPW);
                        if (t == 0 && i % kSpread == kSpread - 1) tile_req(n1, nxt, i / kSpread);
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
                    const bool need_mask = key0 + 32 * t + 31 >= Skv || (CAUSAL && key0 + 32 * t + 31 > wrow0 + dpos);
                    if (need_mask) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = key0 + 32 * t + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                            const bool vis = key < Skv && (!CAUSAL || key <= qrow + dpos);
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
            if (!step(n, st0, st1)) break;
            if (!step(n + 1, st1, st0)) break;
        }
        if (KS == 2) {
            // the second half parks its sums in LDS (every tile read and DMA has
            // completed before the last barrier); the first adds them
            LDS_AS float *park = reinterpret_cast<LDS_AS float *>(w == 0 ? lds0 : w == 1 ? lds1 : w == 2 ? lds2 : lds3);
            if (half == 1) {
#pragma unroll
                for (int i = 0; i < 64; ++i) park[i * 64 + lane] = acc[i >> 4][i & 15];
            }
            __syncthreads();
            if (half == 0) {
#pragma unroll
                for (int i = 0; i < 64; ++i) acc[i >> 4][i & 15] += park[i * 64 + lane];
            }
        }
        if (qrow < S && half == 0) {
            if (accum) add_acc_row(dq + qoff + row_of(qrow) * qstride, acc, inv_sqrt_d, lane);
            else store_acc_row(dq + qoff + row_of(qrow) * qstride, acc, inv_sqrt_d, lane);
        }
        if (pass + 1 < npass) {
            __syncthreads();  // both stages are refilled for the next block
            // the key split's combine parked fp32 sums over the K tiles
            if (KS == 2 && Skv % kBN != 0) zero_stages();
        }
    }
}

// dK, dV: workgroup of 8 wavefronts (two per SIMD) = 128 key rows of one kv
// head.  The block's K and V rows sit in LDS for the whole kernel (holding
// them in registers, as the B operands of S and dP, would need about 350
// registers and allow only one wavefront per SIMD, whose vector work then
// leaves the matrix core idle); for every
// query head of the group, the query tiles (Q, dO: 64 rows each; lse and
// delta: 64 values each) stream through two LDS stages.  Wavefront w takes
// keys 32*(w%4) .. +31 of the block and query half w/4 of every tile, so the
// wavefronts w and w+4 hold the same keys and add their dK and dV once at the
// end, through LDS.
constexpr int kBwdStageB = 2 * kTileB + 2 * 64 * 4;
constexpr int kBwdKvB = 4 * kTileB;  // K rows 0..127, then V rows 0..127
// Split gradients: the step stream of a key block (query head of the group,
// query tile; the tile fastest) cut into n units of consecutive steps, unit u
// taking steps u*L/n .. (u+1)*L/n - 1.  Each unit of a split block leaves its
// fp32 sums in a slot of the workspace, in the accumulators' own lane order;
// a second launch (dkdv_split_sum_kernel) adds the n slots in unit order and
// writes dK and dV.  Split blocks are the first ones of the grid (e below
// the number of split blocks).
constexpr int kDkdvSlot = 2 * 128 * kD;  // floats per (block, unit): dK sums, then dV sums
struct DkdvUnit {
    float *ws = nullptr;  // kDkdvSlot floats per (split block, unit)
    int u = 0, n = 1, umax = 1;
};
template <bool CAUSAL, bool CHUNK, bool PIECES, bool SPLIT = false>
__device__ __forceinline__ void dkdv_body(
    int e, LDS_AS char *lds0, LDS_AS char *lds1, LDS_AS char *ldskv,
    const short *__restrict__ q, const short *__restrict__ k, const short *__restrict__ v,
    const short *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    short *__restrict__ dk, short *__restrict__ dv, int S, int skv, int delta_arg, int acc_arg,
    int Hq, int Hkv, int group, int nkb, int hkvtot, float scale_log2, float inv_sqrt_d,
    FastDiv by_sp, int64_t gap, DkdvUnit du = DkdvUnit()) {
    constexpr int NW = 8, QPW = 2, kBK = 128;
    // CHUNK: S query rows against skv keys, key j visible to query i under the
    // causal mask iff i + dpos >= j; with accumulate the results are added to
    // dk and dv
    const int Skv = CHUNK ? skv : S;
    const int dpos = CHUNK ? delta_arg : 0;
    const bool accum = CHUNK && acc_arg != 0;

    const int hk = e % hkvtot;
    const int kb = e / hkvtot;  // causal: the first key blocks have the most queries
    const int b = hk / Hkv, ck = hk - b * Hkv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = w >> 2, kw = w & 3;  // query half, key group
    const int k0 = kb * kBK, wkey0 = k0 + 32 * kw, key = wkey0 + (lane & 31);
    const int64_t qstride = int64_t(Hq) * kD, kstride = int64_t(Hkv) * kD;
    // first row of batch entry b, and the row of its token s past that
    auto row_of = [&](int s_) __attribute__((always_inline)) -> int64_t {
        return PIECES ? int64_t(s_) + int64_t(by_sp.div(uint32_t(s_))) * gap : int64_t(s_);
    };
    const int64_t bq = int64_t(b) * (PIECES ? int64_t(by_sp.d) : int64_t(S));
    const int64_t koff = int64_t(b) * (PIECES ? int64_t(by_sp.d) : int64_t(Skv)) * kstride + int64_t(ck) * kD;
    const int ntiles = (S + kBN - 1) / kBN;
    const int m0 = CAUSAL ? max(0, k0 - dpos) / kBN : 0;  // first query tile with a visible pair
    if (CHUNK && m0 >= ntiles) {  // no query of the block reaches these keys: a zero contribution
        if (t == 0 && key < Skv && !accum) {
            f32x16 zero[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
            store_acc_row(dk + koff + row_of(key) * kstride, zero, 1.f, lane);
            store_acc_row(dv + koff + row_of(key) * kstride, zero, 1.f, lane);
        }
        return;  // uniform over the workgroup
    }

    TileDma<QPW> td;
    tile_dma_setup(td, w, lane, qstride);
    // requests of this wavefront's share of query tile m of query head c
    auto tile_req = [&](int c, int m, const LDS_AS char *dst, int r) __attribute__((always_inline)) {
        const int row0 = m * kBN, valid = min(S - row0, kBN);
        const int64_t off = bq * qstride + int64_t(c) * kD + row_of(row0) * qstride;
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
    // the block's K and V rows (two 64-row tiles each; rows past the end read
    // as zero and only reach the accumulators of keys that are never stored)
    {
        TileDma<QPW> tk;
        tile_dma_setup(tk, w, lane, kstride);
        const uint32_t d = uint32_t(reinterpret_cast<uintptr_t>(ldskv));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row0 = k0 + j * kBN, valid = min(Skv - row0, kBN);
            i32x4 rk = tile_resource(k + koff + row_of(max(row0, 0)) * kstride, valid, kstride);
            i32x4 rv = tile_resource(v + koff + row_of(max(row0, 0)) * kstride, valid, kstride);
            if (valid <= 0) rk[2] = rv[2] = 0;
#pragma unroll
            for (int u = 0; u < QPW; ++u) {
                dma16(rk, tk.goff[u], d + j * kTileB + tk.m0[u]);
                dma16(rv, tk.goff[u], d + (2 + j) * kTileB + tk.m0[u]);
            }
        }
    }
    LdsOff lo;
    lds_offsets(lo, lane);
    const LDS_AS char *kt = ldskv + 32 * kw * kRowB, *vt = ldskv + 2 * kTileB + 32 * kw * kRowB;
    f32x16 dka[4], dva[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) { dka[mt] = f32x16{}; dva[mt] = f32x16{}; }

    // steps run over (query head c of the group, query tile m), m fastest,
    // stages alternating; (c, m) advance by increments (no division, so the
    // tile addresses stay scalar)
    const int clast = ck * group + group - 1;
    int c = ck * group, m = m0;
    int nsteps = 0, sidx = 0;  // split: this unit's steps, and the steps taken
    if constexpr (SPLIT) {
        const int64_t nm = ntiles - m0, L = int64_t(group) * nm;
        const int64_t s_lo = du.u * L / du.n;
        nsteps = int((du.u + 1) * L / du.n - s_lo);
        c += int(s_lo / nm);
        m = m0 + int(s_lo % nm);
    }
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
        const bool more = SPLIT ? sidx + 1 < nsteps : !(last_m && c == clast);
        // the next step's tile (the current one again after the last step)
        const int c1 = more && last_m ? c + 1 : c;
        const int m1 = !more ? m : last_m ? m0 : m + 1;
        // the next tile's resources first, so that its addresses are formed
        // outside the single-wavefront branch below; the requests themselves
        // are spread over the first products
        const int nrow0 = m1 * kBN, nvalid = min(S - nrow0, kBN);
        const int64_t noff = bq * qstride + int64_t(c1) * kD + row_of(nrow0) * qstride;
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
        if (CAUSAL && qt0 + 32 * t + 31 + dpos < wkey0) {  // every query of the half before every key
#pragma unroll
            for (int r = 0; r < 2 * QPW; ++r) req(r);
        } else {
            // S and dP for queries qt0 + 32t .. +31 (lane: key row): A = the
            // Q / dO tile rows, B = this wavefront's K / V rows, both from
            // LDS, read kA products ahead; the first kB operands of dV/dK are
            // read before the vector work.
            constexpr int kA = 4, kB = 4;
            const int thalf = 32 * t * kRowB;  // this wavefront's 32 query rows of the tile
            auto opA = [&](int i) __attribute__((always_inline)) {  // i = 2*cc + (0: Q rows, 1: dO rows)
                return rows_op(lo, ((i & 1) ? dt : qt) + thalf, 2 * (i >> 1));
            };
            auto opK = [&](int i) __attribute__((always_inline)) {  // i = 2*cc + (0: K rows, 1: V rows)
                return rows_op(lo, (i & 1) ? vt : kt, 2 * (i >> 1));
            };
            auto opB = [&](int i) __attribute__((always_inline)) {  // i = 2*(4h + mt) + (0: dO^T, 1: Q^T)
                return cols_op(lo, ((i & 1) ? qt : dt) + thalf, i >> 1);
            };
            f32x16 sc = f32x16{}, dp = f32x16{};
            s16x8 a[16], kv[16], bo[16];
#pragma unroll
            for (int i = 0; i < kA; ++i) { a[i] = opA(i); kv[i] = opK(i); }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i + kA < 16) { a[i + kA] = opA(i + kA); kv[i + kA] = opK(i + kA); }
                if (i & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], kv[i], dp, 0, 0, 0);
                else sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], kv[i], sc, 0, 0, 0);
                if ((i & 3) == 1) req(i >> 2);
            }
#pragma unroll
            for (int i = 0; i < kB; ++i) bo[i] = opB(i);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kA, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i + kA < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kB, 0);
            s16x8 pb[2], dsb[2];
            // queries past the end, or before this wavefront's last key (causal), need the mask
            const bool need_mask = qt0 + 32 * t + 31 >= S || (CAUSAL && qt0 + 32 * t + dpos < wkey0 + 31);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int j = 32 * t + 8 * g + 4 * (lane >> 5);
                const f32x4 l4 = *reinterpret_cast<const LDS_AS f32x4 *>(ls + j);
                const f32x4 d4 = *reinterpret_cast<const LDS_AS f32x4 *>(dl + j);
                if (need_mask) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = 4 * g + u, qi = qt0 + j + u;
                        const bool vis = qi < S && (!CAUSAL || qi + dpos >= key);
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
        ++sidx;
        return more;
    };
    for (;;) {
        if (!step(lds0, lds1)) break;
        if (!step(lds1, lds0)) break;
    }

    // wavefront w+4 hands its sums for the same keys to wavefront w (the K/V
    // rows are no longer read: 16 KiB per key group, one accumulator set at a
    // time)
    LDS_AS f32x4 *red = reinterpret_cast<LDS_AS f32x4 *>(ldskv) + kw * 1024 + lane;
    auto reduce = [&](f32x16 (&acc)[4]) __attribute__((always_inline)) {
        if (t == 1) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    red[(4 * mt + g) * 64] = f32x4{acc[mt][4 * g], acc[mt][4 * g + 1], acc[mt][4 * g + 2], acc[mt][4 * g + 3]};
        }
        __syncthreads();
        if (t == 0) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 x = red[(4 * mt + g) * 64];
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[mt][4 * g + u] += x[u];
                }
        }
        __syncthreads();
    };
    reduce(dva);
    reduce(dka);
    if (SPLIT && du.n > 1) {  // this unit's sums (16-byte stores, lane-contiguous)
        if (t == 0) {
            f32x4 *sl = reinterpret_cast<f32x4 *>(du.ws + (int64_t(e) * du.umax + du.u) * int64_t(kDkdvSlot)) +
                        kw * 1024 + lane;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    sl[(4 * mt + g) * 64] = f32x4{dka[mt][4 * g], dka[mt][4 * g + 1], dka[mt][4 * g + 2],
                                                  dka[mt][4 * g + 3]};
                    sl[4096 + (4 * mt + g) * 64] = f32x4{dva[mt][4 * g], dva[mt][4 * g + 1],
                                                         dva[mt][4 * g + 2], dva[mt][4 * g + 3]};
                }
        }
        return;
    }
    if (t == 0 && key < Skv) {
        if (accum) {
            add_acc_row(dk + koff + row_of(key) * kstride, dka, inv_sqrt_d, lane);
            add_acc_row(dv + koff + row_of(key) * kstride, dva, 1.f, lane);
        } else {
            store_acc_row(dk + koff + row_of(key) * kstride, dka, inv_sqrt_d, lane);
            store_acc_row(dv + koff + row_of(key) * kstride, dva, 1.f, lane);
        }
    }
}

// The kernels: each declares its LDS and runs its body for its workgroup.
template <bool CAUSAL, bool CHUNK, int KS, bool PIECES = false>
__global__ __launch_bounds__(512, 1) void attention_bwd_dq_kernel(
    const short *__restrict__ q, const short *__restrict__ k, const short *__restrict__ v,
    const short *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    short *__restrict__ dq, int S, int skv, int delta_arg, int acc_arg, int Hq, int Hkv, int group,
    int nqb, int htot, int paired, float scale_log2, float inv_sqrt_d, FastDiv by_sp, int64_t gap) {
    __shared__ __attribute__((aligned(1024))) char smem0[kStageB];
    __shared__ __attribute__((aligned(1024))) char smem1[kStageB];
    __shared__ __attribute__((aligned(1024))) char smem2[KS == 2 ? kStageB : 16];
    __shared__ __attribute__((aligned(1024))) char smem3[KS == 2 ? kStageB : 16];
    dq_body<CAUSAL, CHUNK, KS, PIECES>(int(blockIdx.x), (LDS_AS char *)smem0, (LDS_AS char *)smem1,
                                       (LDS_AS char *)smem2, (LDS_AS char *)smem3, q, k, v, dout, lse,
                                       delta, dq, S, skv, delta_arg, acc_arg, Hq, Hkv, group, nqb, htot,
                                       paired, scale_log2, inv_sqrt_d, by_sp, gap);
}

template <bool CAUSAL, bool CHUNK, bool PIECES = false>
__global__ __launch_bounds__(512, 1) void attention_bwd_dkdv_kernel(
    const short *__restrict__ q, const short *__restrict__ k, const short *__restrict__ v,
    const short *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    short *__restrict__ dk, short *__restrict__ dv, int S, int skv, int delta_arg, int acc_arg,
    int Hq, int Hkv, int group, int nkb, int hkvtot, float scale_log2, float inv_sqrt_d,
    FastDiv by_sp, int64_t gap) {
    __shared__ __attribute__((aligned(1024))) char smem0[kBwdStageB];
    __shared__ __attribute__((aligned(1024))) char smem1[kBwdStageB];
    __shared__ __attribute__((aligned(1024))) char smemkv[kBwdKvB];
    dkdv_body<CAUSAL, CHUNK, PIECES>(int(blockIdx.x), (LDS_AS char *)smem0, (LDS_AS char *)smem1,
                                     (LDS_AS char *)smemkv, q, k, v, dout, lse, delta, dk, dv, S, skv,
                                     delta_arg, acc_arg, Hq, Hkv, group, nkb, hkvtot, scale_log2,
                                     inv_sqrt_d, by_sp, gap);
}

// dQ (key split, 128-row blocks) and dK/dV workgroups in one launch: the two
// roles share one LDS buffer (1024-byte aligned parts), and a host-built order
// (passed by value) lists the workgroups of both, longest first: entry i is
// role << 15 | the workgroup's index in its own grid (role 0 dQ, 1 dK/dV).
constexpr int kFusedKv0 = (kBwdStageB + 1023) / 1024 * 1024;  // dK/dV: stage 1
constexpr int kFusedKv1 = 2 * kFusedKv0;                        // dK/dV: K and V rows
constexpr int kFusedB = kFusedKv1 + kBwdKvB > 4 * kStageB ? kFusedKv1 + kBwdKvB : 4 * kStageB;
constexpr int kFusedMaxWg = 1024;
struct FusedOrder {
    uint16_t wg[kFusedMaxWg];
};
// SPLIT: a dK/dV entry is 1 << 15 | (units - 1) << 12 | unit << 9 | the
// block's index (below 512).
template <bool CAUSAL, bool CHUNK, bool PIECES = false, bool SPLIT = false>
__global__ __launch_bounds__(512, 1) void attention_bwd_fused_kernel(
    const short *__restrict__ q, const short *__restrict__ k, const short *__restrict__ v,
    const short *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    short *__restrict__ dq, short *__restrict__ dk, short *__restrict__ dv, int S, int skv,
    int delta_arg, int acc_q, int acc_kv, int Hq, int Hkv, int group, int nqb, int htot, int paired,
    int nkb, int hkvtot, float scale_log2, float inv_sqrt_d, FastDiv by_sp, int64_t gap,
    FusedOrder order, float *ws, int umax) {
    __shared__ __attribute__((aligned(1024))) char smem[kFusedB];
    LDS_AS char *base = (LDS_AS char *)smem;
    const uint32_t u = order.wg[blockIdx.x];
    const int e = int(u & 0x7FFFu);
    if ((u >> 15) == 0)
        dq_body<CAUSAL, CHUNK, 2, PIECES>(e, base, base + kStageB, base + 2 * kStageB, base + 3 * kStageB,
                                          q, k, v, dout, lse, delta, dq, S, skv, delta_arg, acc_q, Hq, Hkv,
                                          group, nqb, htot, paired, scale_log2, inv_sqrt_d, by_sp, gap);
    else if (SPLIT)
        dkdv_body<CAUSAL, CHUNK, PIECES, true>(
            int(u & 511u), base, base + kFusedKv0, base + kFusedKv1, q, k, v, dout, lse, delta, dk, dv, S,
            skv, delta_arg, acc_kv, Hq, Hkv, group, nkb, hkvtot, scale_log2, inv_sqrt_d, by_sp, gap,
            DkdvUnit{ws, int((u >> 9) & 7u), int((u >> 12) & 7u) + 1, umax});
    else
        dkdv_body<CAUSAL, CHUNK, PIECES>(e, base, base + kFusedKv0, base + kFusedKv1, q, k, v, dout, lse,
                                         delta, dk, dv, S, skv, delta_arg, acc_kv, Hq, Hkv, group, nkb,
                                         hkvtot, scale_log2, inv_sqrt_d, by_sp, gap);
}

// Split gradients, second launch: workgroup i adds the unit slots of split
// block i (units[kb] of them, in unit order) and writes its dK (times
// 1/sqrt(D)) and dV rows in bf16.  Chunk j of a slot (16 bytes) holds key
// row 32*(j/1024) + j%32 and columns 32*mt + 8*g + 4*((j%64)/32) .. +3 with
// (4*mt + g) = (j%1024)/64, the accumulators' lane order.
struct SplitUnits {
    uint8_t n[512];
};
__global__ __launch_bounds__(512) void dkdv_split_sum_kernel(const float *__restrict__ ws,
                                                             short *__restrict__ dk, short *__restrict__ dv,
                                                             int S, int Hkv, int hkvtot, int umax,
                                                             float inv_sqrt_d, SplitUnits units) {
    const int e = blockIdx.x, kb = e / hkvtot, hk = e - kb * hkvtot;
    const int b = hk / Hkv, ck = hk - b * Hkv, n = units.n[kb];
    const int64_t kstride = int64_t(Hkv) * kD;
    const int64_t koff = int64_t(b) * S * kstride + int64_t(ck) * kD;
    const f32x4 *base = reinterpret_cast<const f32x4 *>(ws + int64_t(e) * umax * kDkdvSlot);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int j = r * 512 + int(threadIdx.x);  // 0 .. 8191: dK chunks, then dV chunks
        const int jj = j & 4095, lane = jj & 63, blk = (jj >> 6) & 15;
        const int key = kb * 128 + 32 * (jj >> 10) + (lane & 31);
        const int col = 32 * (blk >> 2) + 8 * (blk & 3) + 4 * (lane >> 5);
        f32x4 acc = base[j];
        for (int u = 1; u < n; ++u) acc += base[int64_t(u) * (kDkdvSlot / 4) + j];
        if (key < S) {
            const float sc = j < 4096 ? inv_sqrt_d : 1.f;
            s16x4 pv;
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = to_bf16(acc[i] * sc);
            *reinterpret_cast<s16x4 *>((j < 4096 ? dk : dv) + koff + int64_t(key) * kstride + col) = pv;
        }
    }
}

// Order of a fused launch: every workgroup of both grids with its work in
// tile products (128 x 64 tiles: dQ three products per 128 rows x 64 keys,
// dK/dV four per 128 keys x 64 queries of each head of its group, the same
// tiles the kernels walk), plus kFusedWgCost for its start and stores, listed
// longest first so that the CUs drain both grids together.  Each grid is
// already longest first in its own order (dQ: unpaired blocks from the last
// query block down; dK/dV: key blocks from the first up), so one merge of the
// two lists sorts them.
constexpr double kFusedWgCost = 36.0;  // about 12 64-key tiles of the forward (three products each)
void fused_order(FusedOrder &ord, int ngq, int ngk, bool causal, int S, int Skv, int dpos, int nqb,
                 int htot, int hkvtot, int group) {
    const int ntq = (S + kBN - 1) / kBN;
    auto dq_cost = [&](int e) {
        const int qb = causal ? nqb - 1 - e / htot : e / htot;
        const int kend = causal ? std::min(Skv, std::max(0, (qb + 1) * 128 + dpos)) : Skv;
        return 3.0 * double((kend + kBN - 1) / kBN) + kFusedWgCost;
    };
    auto dkdv_cost = [&](int e) {
        const int kb = e / hkvtot;
        const int m0 = causal ? std::max(0, kb * 128 - dpos) / kBN : 0;
        return 4.0 * double(std::max(0, ntq - m0)) * group + kFusedWgCost;
    };
    int a = 0, b = 0, n = 0;
    while (a < ngq || b < ngk) {
        if (b >= ngk || (a < ngq && dq_cost(a) >= dkdv_cost(b)))
            ord.wg[n++] = uint16_t(a++);
        else
            ord.wg[n++] = uint16_t(0x8000u | uint32_t(b++));
    }
}

// Split gradients (full sequence, fused launch, at most 512 dK/dV blocks):
// the dK/dV blocks whose work exceeds a cap are cut into units (units[kb]
// per key block, at most 8), so that the longest workgroup comes
// down towards dQ's longest and the mean per CU.  The cap is chosen with a
// longest-first list schedule of every workgroup's cost (as fused_order, plus
// kSplitSumCost per unit of a split block for its slot and the second launch);
// no split unless the span drops by kBwdSplitGain.
constexpr double kSplitSumCost = 6.0;
constexpr double kBwdSplitGain = 0.9;
struct BwdSplit {
    int ksplit = 0;  // key blocks cut (the first ones)
    int umax = 1;    // units of the first key block
    std::vector<int> units;  // per key block
};
double list_span(std::vector<double> cost, int cus) {
    std::sort(cost.begin(), cost.end(), std::greater<double>());
    std::priority_queue<double, std::vector<double>, std::greater<double>> load;
    for (int i = 0; i < cus; ++i) load.push(0.0);
    double span = 0.0;
    for (double c : cost) {
        const double e = load.top() + c;
        load.pop();
        load.push(e);
        span = std::max(span, e);
    }
    return span;
}
BwdSplit bwd_split_plan(int S, int nqb, int htot, int nkb, int hkvtot, int group, bool causal, int cus,
                        int ngq) {
    BwdSplit best;
    // every dK/dV entry of a split launch carries its block index in 9 bits
    if (int64_t(nkb) * hkvtot > 512) return best;
    const int ntq = (S + kBN - 1) / kBN;
    std::vector<double> dq;
    for (int e = 0; e < ngq; ++e) {
        const int qb = causal ? nqb - 1 - e / htot : e / htot;
        const int kend = causal ? std::min(S, (qb + 1) * 128) : S;
        dq.push_back(3.0 * double((kend + kBN - 1) / kBN) + kFusedWgCost);
    }
    std::vector<int> steps(nkb);
    for (int kb = 0; kb < nkb; ++kb) steps[kb] = group * (ntq - (causal ? kb * 128 / kBN : 0));
    auto costs = [&](const std::vector<int> &units) {
        std::vector<double> c = dq;
        for (int kb = 0; kb < nkb; ++kb)
            for (int u = 0; u < units[kb]; ++u) {
                const int n = units[kb], st = (u + 1) * steps[kb] / n - u * steps[kb] / n;
                for (int h = 0; h < hkvtot; ++h)
                    c.push_back(4.0 * st + kFusedWgCost + (n > 1 ? kSplitSumCost : 0.0));
            }
        return c;
    };
    const std::vector<int> ones(nkb, 1);
    const std::vector<double> c0 = costs(ones);
    double total = 0.0, dqmax = 0.0;
    for (double x : c0) total += x;
    for (double x : dq) dqmax = std::max(dqmax, x);
    double span = list_span(c0, cus) * kBwdSplitGain;
    for (double f : {1.0, 1.15, 1.3, 1.5, 2.0}) {
        const double cap = std::max(dqmax, f * total / cus);
        std::vector<int> units(nkb, 1);
        int nwg = ngq, ksplit = 0;
        for (int kb = 0; kb < nkb; ++kb) {
            const double w = 4.0 * steps[kb];
            int n = w + kFusedWgCost > cap ? int(std::ceil(w / std::max(1.0, cap - kFusedWgCost))) : 1;
            n = std::max(1, std::min({n, 8, steps[kb]}));
            if (kb > 0 && units[kb - 1] == 1) n = 1;  // split blocks first
            units[kb] = n;
            nwg += n * hkvtot;
            if (n > 1) ksplit = kb + 1;
        }
        if (ksplit == 0 || nwg > kFusedMaxWg) continue;
        const double sp = list_span(costs(units), cus);
        if (sp < span) {
            span = sp;
            best.ksplit = ksplit;
            best.umax = units[0];
            best.units = units;
        }
    }
    return best;
}

// The fused order with split dK/dV blocks: every workgroup longest first (dQ
// before dK/dV on equal costs).
void fused_order_split(FusedOrder &ord, const BwdSplit &plan, int ngq, int S, int nqb, int htot, int nkb,
                       int hkvtot, int group, bool causal) {
    const int ntq = (S + kBN - 1) / kBN;
    struct W { double cost; int role; uint16_t code; };
    std::vector<W> all;
    for (int e = 0; e < ngq; ++e) {
        const int qb = causal ? nqb - 1 - e / htot : e / htot;
        const int kend = causal ? std::min(S, (qb + 1) * 128) : S;
        all.push_back({3.0 * double((kend + kBN - 1) / kBN), 0, uint16_t(e)});
    }
    for (int kb = 0; kb < nkb; ++kb) {
        const int steps = group * (ntq - (causal ? kb * 128 / kBN : 0)), n = plan.units[kb];
        for (int u = 0; u < n; ++u)
            for (int h = 0; h < hkvtot; ++h) {
                const int e = kb * hkvtot + h;
                const uint32_t code = n > 1 ? 0x8000u | uint32_t(n - 1) << 12 | uint32_t(u) << 9 | uint32_t(e)
                                            : 0x8000u | uint32_t(e);
                all.push_back({4.0 * ((u + 1) * steps / n - u * steps / n), 1, uint16_t(code)});
            }
    }
    std::stable_sort(all.begin(), all.end(), [](const W &a, const W &b) {
        return a.cost != b.cost ? a.cost > b.cost : a.role < b.role;
    });
    for (size_t i = 0; i < all.size(); ++i) ord.wg[i] = all[i].code;
}

// Workspace of the split gradients: umax slots per split block.
uint64_t bwd_split_bytes(const BwdSplit &p, int hkvtot) {
    return p.ksplit ? uint64_t(p.ksplit) * uint64_t(hkvtot) * uint64_t(p.umax) * kDkdvSlot * 4 : 0;
}

int device_cus() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return cus;
}

// dQ's block choice, shared by the launch and the split plan
struct DqGrid {
    bool use8;
    int nqb, paired;
};
DqGrid dq_grid(int64_t S, int htot, bool causal, int cus) {
    // dQ block size as in the forward: 256-row blocks where they cover every CU
    // (causal: as long-with-short pairs, or unpaired while the longest-first
    // schedule keeps the mean work per CU at 0.6 of the longest block), else
    // the key split on 128-row blocks
    const int64_t nqb8 = (S + 255) / 256;
    bool use8 = nqb8 * htot >= cus;
    if (causal && use8 && (nqb8 + 1) / 2 * htot < cus)
        use8 = double(htot) * double(nqb8) * double(nqb8 + 1) / 2 / cus >= 0.6 * double(nqb8);
    const int nqb = int(use8 ? nqb8 : (S + 127) / 128);
    // causal: a long and a short query block per workgroup while the pairs
    // still cover every CU (as in the forward)
    const int paired = causal && int64_t((nqb + 1) / 2) * htot >= cus ? 1 : 0;
    return {use8, nqb, paired};
}

// The split plan for a full-sequence call, or none where the call does not
// take the fused launch.
BwdSplit split_plan_for(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, bool causal) {
    const int cus = device_cus(), htot = int(B * Hq), hkvtot = int(B * Hkv);
    const DqGrid g = dq_grid(S, htot, causal, cus);
    const int64_t ngq = int64_t(g.paired ? (g.nqb + 1) / 2 : g.nqb) * htot;
    const int nkb = int((S + 127) / 128);
    if (B * S * Hq == 0 || g.use8 || g.paired || ngq + int64_t(nkb) * hkvtot > kFusedMaxWg) return {};
    return bwd_split_plan(int(S), g.nqb, htot, nkb, hkvtot, int(Hq / Hkv), causal, cus, int(ngq));
}
}  // namespace

namespace {
template <bool CHUNK, bool PIECES = false>
hipError_t launch_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                      const float *lse, float *delta, void *dq, void *dk, void *dv, int64_t B,
                      int64_t S, int64_t Skv, int64_t dpos, bool acc_dq, bool acc_dkv, int64_t Hq,
                      int64_t Hkv, bool causal, hipStream_t st, int64_t sp = 0, void *ws = nullptr) {
    const float scale_log2 = float(1.4426950408889634 / 11.313708498984761);  // log2(e)/sqrt(128)
    const float inv_sqrt_d = float(1.0 / 11.313708498984761);
    const auto *qs = static_cast<const short *>(q), *ks = static_cast<const short *>(k),
               *vs = static_cast<const short *>(v), *os = static_cast<const short *>(o),
               *ds = static_cast<const short *>(dout);
    const int64_t rows = B * S * Hq;
    const FastDiv by_sp = PIECES ? FastDiv(uint32_t(sp)) : FastDiv();
    const int64_t gap = PIECES ? (B - 1) * sp : 0;
    const int htot = int(B * Hq);
    const int cus = device_cus();
    const DqGrid dg = dq_grid(S, htot, causal, cus);
    const bool use8 = dg.use8;
    const int nqb = dg.nqb, paired = dg.paired;
    const dim3 gq(uint32_t(int64_t(paired ? (nqb + 1) / 2 : nqb) * htot));
    const int accq = acc_dq ? 1 : 0, acck = acc_dkv ? 1 : 0;
    const int nkb = int((Skv + 127) / 128), hkvtot = int(B * Hkv);
    const dim3 gk(uint32_t(int64_t(nkb) * hkvtot));
    // dQ's key-split blocks and the dK/dV blocks in one launch, longest first
    // across both, where dQ's blocks are neither 256 rows high nor paired (so
    // its grid alone leaves CUs idle or unbalanced) and the two grids drain
    // together instead of one after the other.  Measured on MI355X against two
    // launches (whole gradient call, causal): S = 4096 with 4 heads 193 -> 130
    // us, 6144 271 -> 192, 8192 361 -> 259, 12288 596 -> 523, 4096 with 8 heads
    // 193 -> 140; with paired dQ blocks it was slower (S = 16384 with 4 heads
    // 889 -> 927, 8192 with 8 heads 461 -> 487), so those keep two launches.
    const bool fuse = rows > 0 && int64_t(nkb) * hkvtot > 0 && !use8 && !paired &&
                      int64_t(gq.x) + int64_t(gk.x) <= kFusedMaxWg;
    // split gradients (workspace given, full sequence): the plan of these sizes
    BwdSplit plan;
    if (!CHUNK && !PIECES && ws && fuse)
        plan = bwd_split_plan(int(S), nqb, htot, nkb, hkvtot, int(Hq / Hkv), causal, cus, int(gq.x));
    float *slots = plan.ksplit ? static_cast<float *>(ws) : nullptr;
    if (rows > 0)
        hipLaunchKernelGGL((attention_delta_kernel<PIECES>), dim3(uint32_t((rows * 16 + 255) / 256)), dim3(256),
                           0, st, os, ds, delta, int(S), int(Hq), rows, int(B), int(PIECES ? sp : S));
    if (fuse) {
        FusedOrder ord;
        uint32_t nwg = gq.x + gk.x;
        if (plan.ksplit) {
            fused_order_split(ord, plan, int(gq.x), int(S), nqb, htot, nkb, hkvtot, int(Hq / Hkv), causal);
            nwg = gq.x;
            for (int u : plan.units) nwg += uint32_t(u * hkvtot);
        } else {
            fused_order(ord, int(gq.x), int(gk.x), causal, int(S), int(Skv), int(dpos), nqb, htot, hkvtot,
                        int(Hq / Hkv));
        }
        auto fused = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, dim3(nwg), dim3(512), 0, st, qs, ks, vs, ds, lse, delta,
                               static_cast<short *>(dq), static_cast<short *>(dk), static_cast<short *>(dv),
                               int(S), int(Skv), int(dpos), accq, acck, int(Hq), int(Hkv), int(Hq / Hkv), nqb,
                               htot, paired, nkb, hkvtot, scale_log2, inv_sqrt_d, by_sp, gap, ord, slots,
                               plan.umax);
        };
        if (plan.ksplit && !CHUNK && !PIECES) {
            causal ? fused(attention_bwd_fused_kernel<true, false, false, true>)
                   : fused(attention_bwd_fused_kernel<false, false, false, true>);
            SplitUnits un{};
            for (int kb = 0; kb < plan.ksplit; ++kb) un.n[kb] = uint8_t(plan.units[kb]);
            hipLaunchKernelGGL(dkdv_split_sum_kernel, dim3(uint32_t(plan.ksplit * hkvtot)), dim3(512), 0, st, slots,
                               static_cast<short *>(dk), static_cast<short *>(dv), int(S), int(Hkv), hkvtot,
                               plan.umax, inv_sqrt_d, un);
        } else
            causal ? fused(attention_bwd_fused_kernel<true, CHUNK, PIECES>)
                   : fused(attention_bwd_fused_kernel<false, CHUNK, PIECES>);
        return hipGetLastError();
    }
    auto dq_launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, gq, dim3(512), 0, st, qs, ks, vs, ds, lse, delta,
                           static_cast<short *>(dq), int(S), int(Skv), int(dpos), accq, int(Hq),
                           int(Hkv), int(Hq / Hkv), nqb, htot, paired, scale_log2, inv_sqrt_d, by_sp, gap);
    };
    if (rows == 0) {  // (chunk calls with no query rows) only the key side has outputs
    } else if (causal)
        use8 ? dq_launch(attention_bwd_dq_kernel<true, CHUNK, 1, PIECES>)
             : dq_launch(attention_bwd_dq_kernel<true, CHUNK, 2, PIECES>);
    else
        use8 ? dq_launch(attention_bwd_dq_kernel<false, CHUNK, 1, PIECES>)
             : dq_launch(attention_bwd_dq_kernel<false, CHUNK, 2, PIECES>);
    if (int64_t(nkb) * hkvtot == 0) {  // (chunk calls with no keys) nothing on the key side
    } else if (causal)
        hipLaunchKernelGGL((attention_bwd_dkdv_kernel<true, CHUNK, PIECES>), gk, dim3(512), 0, st, qs, ks, vs,
                           ds, lse, delta, static_cast<short *>(dk), static_cast<short *>(dv), int(S),
                           int(Skv), int(dpos), acck, int(Hq), int(Hkv), int(Hq / Hkv), nkb, hkvtot,
                           scale_log2, inv_sqrt_d, by_sp, gap);
    else
        hipLaunchKernelGGL((attention_bwd_dkdv_kernel<false, CHUNK, PIECES>), gk, dim3(512), 0, st, qs, ks, vs,
                           ds, lse, delta, static_cast<short *>(dk), static_cast<short *>(dv), int(S),
                           int(Skv), int(dpos), acck, int(Hq), int(Hkv), int(Hq / Hkv), nkb, hkvtot,
                           scale_log2, inv_sqrt_d, by_sp, gap);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_attention_bwd_bf16_d128(const void *q, const void *k, const void *v,
                                          const void *o, const void *dout, const float *lse,
                                          float *delta, void *dq, void *dk, void *dv, int64_t B,
                                          int64_t S, int64_t Hq, int64_t Hkv, int64_t sp,
                                          bool causal, hipStream_t st) {
    // with one batch entry the pieces are the plain sequence order
    if (sp > 0 && B > 1)
        return launch_bwd<false, true>(q, k, v, o, dout, lse, delta, dq, dk, dv, B, S, S, 0, false, false,
                                       Hq, Hkv, causal, st, sp);
    return launch_bwd<false>(q, k, v, o, dout, lse, delta, dq, dk, dv, B, S, S, 0, false, false, Hq,
                             Hkv, causal, st);
}

uint64_t attention_bwd_bf16_d128_split_workspace(int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                                 bool causal) {
    return bwd_split_bytes(split_plan_for(B, S, Hq, Hkv, causal), int(B * Hkv));
}

hipError_t launch_attention_bwd_bf16_d128_split(const void *q, const void *k, const void *v,
                                                const void *o, const void *dout, const float *lse,
                                                float *delta, void *dq, void *dk, void *dv, int64_t B,
                                                int64_t S, int64_t Hq, int64_t Hkv, bool causal,
                                                void *workspace, hipStream_t st) {
    return launch_bwd<false>(q, k, v, o, dout, lse, delta, dq, dk, dv, B, S, S, 0, false, false, Hq,
                             Hkv, causal, st, 0, workspace);
}

hipError_t launch_attention_chunk_bwd_bf16_d128(const void *q, const void *k, const void *v,
                                                const void *o, const void *dout, const float *lse,
                                                float *delta, void *dq, void *dk, void *dv,
                                                int64_t B, int64_t Sq, int64_t Skv, int64_t dpos,
                                                bool acc_dq, bool acc_dkv, int64_t Hq, int64_t Hkv,
                                                bool causal, hipStream_t st) {
    return launch_bwd<true>(q, k, v, o, dout, lse, delta, dq, dk, dv, B, Sq, Skv, dpos, acc_dq,
                            acc_dkv, Hq, Hkv, causal, st);
}

}  // namespace uly
