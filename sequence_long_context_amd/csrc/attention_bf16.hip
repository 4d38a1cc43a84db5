// One rank's local attention, bf16 in / bf16 out, head_dim 128, on gfx950
// matrix cores: softmax(Q K^T / sqrt(D)) V per head ("Comparing Ulysses and
// Megatron Sequence Parallelism", attention skeleton in the Introduction),
// grouped key/value heads, optional causal triangle ("Sequence Parallelism II:
// DeepSpeed Ulysses and All-to-All Attention", section 8).
//
// Flash-style fused kernel.  A workgroup is 8 wavefronts and owns 256 query
// rows of one head (32 rows per wavefront; 128 rows with the key split below
// when 256-row blocks would leave CUs idle, as for short sequences); it
// streams the head's keys and values in tiles of 64 rows through LDS (two stages: tile n+1 is requested
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
// Row sums.  The normaliser is the sum of the same bf16 weights that
// multiply V: each lane adds its 32 packed weights of a tile with 16
// v_dot2c_f32_bf16 (two weights times one per instruction, fp32 sum), and the
// lanes l and l^32 that share a query row combine their halves once at the
// end.  (Summing on the matrix core with 16x16x32 products against a 0/1
// operand cost 6 % of the product time and 60 more registers; the vector
// unit has room for 16 more instructions per tile.)
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
// and their keys/values stay in its L2.  When the grid is large enough, a
// causal workgroup takes two query blocks, nqb-1-i and then i (the longest
// with the shortest): all workgroups then stream the same number of tiles,
// which measured 2-5 % faster than longest-first single blocks at S >= 32k.
// The second block walks its keys from the diagonal down: workgroup i starts
// it 4i tiles before workgroup i+1 does and 4 tiles nearer key 0, so the
// second blocks of an XCD read the same tile at the same time, as the first
// blocks do going up, and share it in L2 (HBM reads 1.03e9 -> 2.2e8 bytes per
// launch at s32k).
//
// Chunk calls (one visit of a circulating key/value block, section 8 of the
// same page): the same kernel with Sq query rows against Skv keys and the
// causal diagonal shifted by delta = query position - key position of the
// first rows, so a block sees every key (a block from the past), a shifted
// triangle, or nothing (a block from the future: o = 0, lse = -inf, no tile
// is read).  A compile-time flag keeps the full-sequence instantiation free
// of the extra terms.
//
// Algorithmic work: 4*D flops per visible (query, key) pair.
#include "attn_fwd.h"

namespace uly {
namespace {

// Schedule model for the key split's two block heights.  Each CU holds one
// 8-wavefront workgroup at a time; workgroups start in grid order, which is
// longest first (pairs, or blocks from the bottom of the triangle).  The span
// is the busiest CU's total in (query row, key) pairs, keys rounded up to
// whole tiles, from a list schedule of the grid.
double schedule_span(int64_t rows, int64_t Sq, int64_t Skv, int64_t delta, int64_t heads,
                     bool causal, int cus) {
    const int64_t nqb = (Sq + rows - 1) / rows;
    const bool paired = causal && (nqb + 1) / 2 * heads >= cus;
    const int64_t nwg = paired ? (nqb + 1) / 2 : nqb;
    auto block = [&](int64_t qb) {
        const int64_t kend =
            causal ? std::min(Skv, std::max<int64_t>(0, (qb + 1) * rows + delta)) : Skv;
        return double(rows) * double((kend + kBN - 1) / kBN * kBN);
    };
    auto work = [&](int64_t pi) {
        double w = block(causal ? nqb - 1 - pi : pi);
        if (paired && nqb - 1 - pi != pi) w += block(pi);
        return w;
    };
    if (nwg * heads <= cus) return work(0);  // one round: the first is the longest
    std::priority_queue<double, std::vector<double>, std::greater<double>> load;
    for (int i = 0; i < cus; ++i) load.push(0.0);
    double span = 0.0;
    for (int64_t pi = 0; pi < nwg; ++pi) {
        const double w = work(pi);
        for (int64_t h = 0; h < heads; ++h) {
            const double t = load.top() + w;
            load.pop();
            load.push(t);
            span = std::max(span, t);
        }
    }
    return span;
}

// Pairs per unit time of the chain split's 64-row blocks against 128-row
// blocks, both with the key split: at 4 heads, S = 8192, non-causal, the two
// spans are equal and the times 166.5 and 129.8 us.
constexpr double kChainSplitRate = 0.78;

// Workgroup size.  8 wavefronts (two per SIMD, so one's softmax overlaps the
// other's products) when their blocks cover every CU at least once; causal
// blocks then run as long-with-short pairs, which balance the triangle.  Where
// the pairs would not cover the CUs, unpaired 8-wavefront blocks are kept as
// long as the longest-first schedule still balances: the mean work per CU
// reaches 0.6 of the longest block (measured at 4 heads: S = 24576, where it
// is 0.76, 925 vs 886 TFLOP/s for paired 4-wavefront blocks; S = 16384, 0.51,
// 684 vs 800 for paired 4-wavefront blocks).  Otherwise the key split (KS =
// 2): 8 wavefronts on 128-row blocks, twice the blocks, paired if that covers
// the CUs; against 4-wavefront blocks it measured +10-22 % (S = 2048-16384),
// against 256-row blocks where those balance -7-10 % (S >= 20480).  Within
// the key split, 64-row blocks with the chain split where the schedule model
// above says their shorter span pays for their lower rate.
hipError_t launch_any(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                      int64_t Sq, int64_t Skv, int64_t delta, int64_t Hq, int64_t Hkv, bool causal,
                      bool chunk, bool acc, int64_t sp, hipStream_t st) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    // a chunk whose every key precedes every query row needs no mask
    if (chunk && causal && delta >= Skv - 1) causal = false;
    const int64_t nqb8 = (Sq + 255) / 256, heads = B * Hq;
    bool use8 = nqb8 * heads >= cus;
    if (causal && use8 && (nqb8 + 1) / 2 * heads < cus) {
        // block i holds i+1 units of work; mean per CU against the longest
        const double total = double(heads) * double(nqb8) * double(nqb8 + 1) / 2;
        use8 = total / cus >= 0.6 * double(nqb8);
    }
    if (use8) return launch_nw<8, 1>(q, k, v, o, lse, B, Sq, Skv, delta, Hq, Hkv, causal, chunk, acc, sp, cus, st);
    const double span128 = schedule_span(128, Sq, Skv, delta, heads, causal, cus);
    const double span64 = schedule_span(64, Sq, Skv, delta, heads, causal, cus);
    if (span64 < kChainSplitRate * span128)
        return launch_chain_split(q, k, v, o, lse, B, Sq, Skv, delta, Hq, Hkv, causal, chunk, acc, sp, cus, st);
    return launch_nw<8, 2>(q, k, v, o, lse, B, Sq, Skv, delta, Hq, Hkv, causal, chunk, acc, sp, cus, st);
}


// Plan of the split forward: 64-row chain-split blocks, block qb holding T(qb)
// key tiles (qb + 1 causal, every tile otherwise), cut into ceil(T / c) units
// of consecutive tiles.  c is chosen with the same one-workgroup-per-CU list
// schedule as schedule_span, in tiles, each workgroup charged kSplitUnitCost
// tiles beyond its own and a split plan kSplitMergeCost more for the merge
// launch; no split unless that beats the unsplit blocks' span by kSplitGain.
// Units are listed longest first.  The costs are measured on MI355X
// (timestamps per workgroup, S = 128 ... 4096): a 64-key tile takes 0.52 us;
// a workgroup's first tile copy and Q load 3.4-3.9 us, the combine of its four
// partial states 2.0 us and its stores 0.6 us, about 12 tiles; the merge
// kernel 7-10 us and the gap before it about 5.7 us, about 25 tiles.  The
// model runs 0.05-0.1 optimistic against measured times (S = 2500 ... 16384,
// 1-2 heads), hence the margin of kSplitGain.
constexpr double kSplitUnitCost = 12.0;
constexpr double kSplitMergeCost = 25.0;
constexpr double kSplitGain = 0.84;
struct SplitPlan {
    int nqb = 0, htot = 0, cus = 0, causal = 0;  // the sizes it is for
    int ctiles = 0;      // at most ctiles tiles per unit
    int umax = 1;        // units of the longest block
    int units = 0;       // table entries (units per head)
    bool split = false;  // some block has more than one unit
    SplitTable table{};
};

int split_block_tiles(int qb, int nqb, bool causal) { return causal ? qb + 1 : nqb; }

// units of one head for ctiles, longest first; false if they overflow the table
bool split_units(int nqb, bool causal, int ctiles, std::vector<uint32_t> &out, std::vector<int> &len) {
    if (nqb > kSplitMaxUnits) return false;  // every block is at least one unit
    struct U { int tiles, qb, u, n; };
    std::vector<U> us;
    for (int qb = 0; qb < nqb; ++qb) {
        const int t = split_block_tiles(qb, nqb, causal), n = (t + ctiles - 1) / ctiles;
        if (n > 255) return false;
        if (int(us.size()) + n > kSplitMaxUnits) return false;
        for (int u = 0; u < n; ++u) us.push_back({(u + 1) * t / n - u * t / n, qb, u, n});
    }
    std::stable_sort(us.begin(), us.end(), [](const U &a, const U &b) {
        return a.tiles != b.tiles ? a.tiles > b.tiles : a.qb > b.qb;
    });
    out.clear();
    len.clear();
    for (const U &x : us) {
        out.push_back(uint32_t(x.qb) << 16 | uint32_t(x.u) << 8 | uint32_t(x.n));
        len.push_back(x.tiles);
    }
    return true;
}

double split_span(const std::vector<int> &len, int htot, int cus) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> load;
    for (int i = 0; i < cus; ++i) load.push(0.0);
    double span = 0.0;
    for (int t : len)
        for (int h = 0; h < htot; ++h) {
            const double e = load.top() + t + kSplitUnitCost;
            load.pop();
            load.push(e);
            span = std::max(span, e);
        }
    return span;
}

SplitPlan make_split_plan(int nqb, int htot, bool causal, int cus) {
    SplitPlan p;
    p.nqb = nqb;
    p.htot = htot;
    p.cus = cus;
    p.causal = causal;
    p.ctiles = nqb;  // no split
    std::vector<uint32_t> tab;
    std::vector<int> len;
    // many blocks per CU already balance a longest-first schedule (and keep the
    // model's own cost down): no split
    if (nqb == 0 || int64_t(nqb) * htot > 8 * int64_t(cus)) return p;
    if (!split_units(nqb, causal, nqb, tab, len)) return p;
    const double base = split_span(len, htot, cus);
    const double total = double(htot) * (causal ? 0.5 * nqb * (nqb + 1.0) : double(nqb) * nqb);
    const double target = total / cus;
    double best = base * kSplitGain;
    int best_c = 0;
    std::vector<uint32_t> btab;
    for (int f = 5; f <= 15; ++f) {
        const int ct = std::max(1, std::min(nqb - 1, int(std::ceil(target * f / 10.0))));
        if (ct >= nqb || ct == best_c) continue;
        if (!split_units(nqb, causal, ct, tab, len)) continue;
        const double sp = split_span(len, htot, cus) + kSplitMergeCost;
        if (sp < best) {
            best = sp;
            best_c = ct;
            btab = tab;
        }
    }
    if (!best_c) return p;
    p.ctiles = best_c;
    p.split = true;
    p.units = int(btab.size());
    p.umax = (nqb + best_c - 1) / best_c;
    for (int i = 0; i < p.units; ++i) p.table.unit[i] = btab[i];
    return p;
}

// plans by sizes, computed once (a list schedule per candidate is too slow
// for every call of a short sequence)
SplitPlan split_plan(int64_t S, int64_t htot, bool causal) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int nqb = int((S + kSplitRows - 1) / kSplitRows);
    static std::mutex mu;
    static SplitPlan cache[8];
    static int next = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (const SplitPlan &p : cache)
        if (p.nqb == nqb && p.htot == htot && p.cus == cus && p.causal == int(causal) && p.nqb)
            return p;
    SplitPlan p = make_split_plan(nqb, int(htot), causal, cus);
    cache[next] = p;
    next = (next + 1) % 8;
    return p;
}
}  // namespace

hipError_t launch_attention_bf16_d128(const void *q, const void *k, const void *v, void *o,
                                      float *lse, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                      int64_t sp, bool causal, hipStream_t st) {
    // with one batch entry the pieces are the plain sequence order
    return launch_any(q, k, v, o, lse, B, S, S, 0, Hq, Hkv, causal, false, false, B > 1 ? sp : 0, st);
}

hipError_t launch_attention_chunk_bf16_d128(const void *q, const void *k, const void *v, void *o,
                                            float *lse, int64_t B, int64_t Sq, int64_t Skv,
                                            int64_t delta, int64_t Hq, int64_t Hkv, bool causal,
                                            bool accumulate, hipStream_t st) {
    return launch_any(q, k, v, o, lse, B, Sq, Skv, delta, Hq, Hkv, causal, true, accumulate, 0, st);
}

uint64_t attention_bf16_d128_split_workspace(int64_t B, int64_t S, int64_t Hq, bool causal) {
    const SplitPlan p = split_plan(S, B * Hq, causal);
    return p.split ? uint64_t(B * Hq) * uint64_t(p.nqb) * uint64_t(p.umax) * kSplitSlot * 4u : 0;
}

hipError_t launch_attention_bf16_d128_split(const void *q, const void *k, const void *v, void *o,
                                            float *lse, int64_t B, int64_t S, int64_t Hq,
                                            int64_t Hkv, bool causal, void *workspace,
                                            hipStream_t st) {
    const SplitPlan p = split_plan(S, B * Hq, causal);
    if (!p.split)  // nothing to cut: the plain call
        return launch_any(q, k, v, o, lse, B, S, S, 0, Hq, Hkv, causal, false, false, 0, st);
    SplitTable t = p.table;
    t.ws = static_cast<float *>(workspace);
    t.umax = p.umax;
    const int htot = int(B * Hq), s = int(S), hq = int(Hq), hkv = int(Hkv);
    const dim3 grid(uint32_t(int64_t(p.units) * htot));
    hipError_t err = launch_split_units(grid, st, q, k, v, o, lse, s, hq, hkv, p.nqb, htot, causal, t);
    if (err != hipSuccess) return err;
    // blocks of more than one unit: causal, those past ctiles tiles; otherwise all
    const int first = causal ? p.ctiles : 0;
    return launch_split_merge(static_cast<const float *>(workspace), o, lse, s, hq, p.nqb, p.umax,
                              p.ctiles, first, htot, causal, st);
}

}  // namespace uly
