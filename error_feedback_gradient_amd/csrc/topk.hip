// Top-k sparsification with error feedback (flat and layer-wise), gfx950.
//
// What is computed ("Gradient sparsification" page, step-by-step algorithm
// steps 2-4, error-compensation and top-k sections): x = g + e; keep the k
// entries of largest |x| (ties: lower index first); send them with their
// indices in ascending order; e = x where dropped, +0 where kept.
//
// How (per tensor, "segment"; the flat call is one segment):
//   1. sample     a strided sample of x = g + e is histogrammed on the top 12
//                 bits of its magnitude key, and at 1/1024 octave around the
//                 tensor's threshold of the previous call on the workspace.
//                 Two bin edges are read off it (by one wave per tensor; in a
//                 call with few regions, by the stream's blocks themselves),
//                 in the fine bins where they hold the rank: T_lo, with (by a
//                 wide statistical margin) at least k elements of the tensor
//                 above it, and T_hi, with (very likely) fewer than k above
//                 it.  The fine bins keep the window tight where error
//                 feedback crowds the residual just below T.
//   2. stream     ONE pass over the tensor, one wave per 4096-element region
//                 (eight waves per region in a call with few regions): read g
//                 and e (128-bit non-temporal loads, all of a wave's in flight
//                 per lane and array), write e (128-bit stores), and append
//                 every element with key >= T_lo to the region's candidate
//                 slot, in index order, with wave ballots.
//                 Candidates with key >= T_hi are almost surely kept, so the
//                 stream already writes e = 0 for them.  Each block adds its
//                 regions' candidate counts to their group totals with one
//                 atomic per group.  This is the only full pass: 12 B/element.
//   3. compact    per group of 256 regions: the tensor's group totals decide
//                 its path (exact fallback when its candidates exceed its slot
//                 capacity or fewer than k were found); candidate slots -> one
//                 dense index-ordered list, plus the first radix histogram.
//                 A region whose slot overflowed (its first `cap` candidates
//                 are in the slot, the rest are untouched in e) is read again
//                 past its last stored index by one wave of the same block,
//                 which appends the rest at their places in the dense list.
//                 Clustered magnitudes thus cost one extra read of the crowded
//                 regions instead of the exact pass over the whole tensor.
//   4. radix      exact k-th largest key T over the candidates: digits of 11,
//                 10 and 10 bits, each histogram (LDS-privatised) built by one
//                 kernel and its digit found by the blocks of the next one.
//   5. emit       entries with key > T, plus the first r entries with key == T
//                 in index order, are written in index order: the last radix
//                 pass leaves the suffix sums of each block's histogram of its
//                 contiguous range of the list, and every write block finds T
//                 itself and starts after the totals of the blocks before it
//                 (two words of each one's suffix sums).
//                 Their residual becomes +0 unless the stream already cleared
//                 it; a dropped candidate that the stream cleared gets x back.
// The exact fallback runs steps 4-5 over the whole tensor (x sits in e) in
// two reads of x (three when T's first digit lies outside the sample's
// window): its compaction blocks histogram x for the first digit (and, for
// the first digits the window spans, the second one) and put x back wherever
// the stream cleared it; then the last radix pass, which also keeps each
// block's suffix sums and appends, in index order, every key whose top 21
// bits are T's or above to the block's segment of the (otherwise unused)
// dense list.  The write places from those segments; it reads x once more
// only for a block whose segment overflowed, or when statistics, which need
// every entry's fate, are asked for.  The write kernel leaves T in the
// workspace as the next call's hint.  Only integer atomics are used, so results do not
// depend on timing, and no path (nor the hint) changes them.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <vector>

#include "common.hpp"

namespace efg {
namespace topk {

constexpr int kBlock = 256;                        // threads of the select / emit kernels
constexpr int kWavesPerBlock = kBlock / kWave;
// Streaming-pass shape, measured on MI355X: 4096-element regions per wave,
// all 16 x 128-bit loads of a region issued per lane and array before the
// first use (176 VGPRs, no spills), 512-thread blocks.
#ifndef EFG_STREAM_BLOCK
#define EFG_STREAM_BLOCK 512
#endif
#ifndef EFG_STREAM_REGION
#define EFG_STREAM_REGION 4096
#endif
#ifndef EFG_STREAM_UNROLL
#define EFG_STREAM_UNROLL 16
#endif
constexpr int kStreamBlock = EFG_STREAM_BLOCK;     // threads of the streaming kernel
constexpr int kStreamWaves = kStreamBlock / kWave;
constexpr int64_t kFewRegions = 4096;             // below: split stream blocks, one copy of each histogram
#ifndef EFG_SPLIT
#define EFG_SPLIT 8
#endif
constexpr int kSplit = EFG_SPLIT;                  // waves per region in the split streaming pass
constexpr int kRegion = EFG_STREAM_REGION;         // elements per wave in the streaming pass
constexpr int kUnroll = EFG_STREAM_UNROLL;         // 128-bit loads in flight per lane and array
constexpr int kGroup = 256;                        // regions per group (candidate totals, compaction)
constexpr int kSampleChunk = 256;                  // contiguous elements per sample chunk
constexpr int kSampleChunksMax = 4096;
#ifndef EFG_SAMPLE_DIV
#define EFG_SAMPLE_DIV 16
#endif
#ifndef EFG_SAMPLE_MIN
#define EFG_SAMPLE_MIN 256
#endif
constexpr int kSampleChunksMin = EFG_SAMPLE_MIN;  // fewest sample chunks of a sampled tensor
constexpr int kSampleDiv = EFG_SAMPLE_DIV;         // sample one chunk in kSampleDiv (up to the maximum)
constexpr int kSampleBlock = 256;                  // threads of the sample kernel
constexpr int kSampleChunksPerWave = 4;
constexpr int kSampleBlockChunks = kSampleChunksPerWave * (kSampleBlock / kWave);
constexpr int kSampleBlocksTarget = 1024;            // enough sample blocks to fill the chip
constexpr int kSampleRoundsMax = 8;
constexpr int kSampleBins = 4096;
// After its fine bins every sample histogram keeps 64 coarse bins of 64 fine
// ones each, so that one wave can find a rank in it with two reads.
constexpr int kSampleCoarse = 64;
constexpr int kSampleWords = kSampleBins + kSampleCoarse;
constexpr int kSampleShift = 19;                   // 31-bit key >> 19 = 12 bits
// Each copy of a sample histogram also keeps a window of fine bins around the
// tensor's threshold of the previous call on the workspace (its hint):
// kFineBins bins of 2^kFineShift key units (1/1024 octave) over the hint
// +-1/4 octave, their sums in groups of 64, and the count of samples above
// the window.  The sample ranks for T_lo and T_hi lie within about a tenth
// of an octave of T, and T moves little from one step to the next; when it
// moves farther, the 12-bit bins decide as they would without a hint.
// Where the residual has crowded values just below the threshold (the steady
// state of error feedback under a gradient with a drift), a 12-bit bin below
// T can hold many times k elements; the fine window puts T_lo within 1/1024
// octave of the sample rank it stands for, so the candidates stay few.
constexpr int kFineShift = 13;
constexpr int kFineBins = 512;
constexpr int kFineGroups = kFineBins / 64;
constexpr uint32_t kFineSpan = static_cast<uint32_t>(kFineBins) << kFineShift;
constexpr int kFineWords = kFineBins + 32;  // bins, group sums, count above, padding
static_assert(kFineGroups + 1 <= 32, "group sums and the count above fit the padding");
constexpr int kSampleStride = kSampleWords + kFineWords;  // words of one histogram copy
static_assert(kSampleStride % 4 == 0, "histogram copies stay 16-byte aligned");
#ifndef EFG_CHUNK
#define EFG_CHUNK 2048
#endif
constexpr int kChunk = EFG_CHUNK;                  // entries per block-unit in select and emit
static_assert(kChunk % kBlock == 0, "k_write: each wave takes kChunk / kBlock rows of 64 entries");
constexpr int kRadixBins = 2048;
constexpr int kSpec = 2;  // first digits the exact fallback guesses T's among (second-digit histograms)
// Every radix histogram keeps, after its fine bins, coarse bins of 32 fine
// ones each (64 for the 11-bit first digit, 32 for the 10-bit ones): the
// kernel that needs a tensor's digit finds it from the coarse bins and one
// slice of 32 fine bins, instead of a digit launch reading every bin.
constexpr int kCoarse = 64;
constexpr int kHistWords = kRadixBins + kCoarse;
// The last radix histogram of each select block is also kept whole, with the
// block's count of keys above the digits fixed before it.
constexpr int kBlockHistWords = 1024 + 64;  // 1024 bins, the count above the prefix, padding
// A fallback tensor's elements are taken in units of kRawChunk (kRawSub
// chunks of kChunk), so that its per-unit monitoring partials stay few
// (79,346 units at 1.3e9 elements).
constexpr int kRawSub = 8;
constexpr int kRawChunk = kRawSub * kChunk;
constexpr int kSelectBlocks = 2048;                // select / emit blocks shared out among the tensors
// 2048 blocks of 256 threads are 8 waves per SIMD on 256 CUs: the histogram
// and write kernels are held to the registers that let the whole grid run
// at once (a second round for the blocks that do not fit would double them)
constexpr int kSelectWaves = 8;
constexpr int kHistCopies = 8;                     // copies of a histogram when a call has few tensors (1 or this)
constexpr int64_t kCompactBlocksMax = 2048;        // compaction blocks the GPU holds at once (8 per CU)
constexpr int kMaxGrid = 2048;
constexpr uint32_t kNoKey = 0xffffffffu;           // above every 31-bit key

enum : int32_t { MODE_NORMAL = 0, MODE_NONE = 1, MODE_ALL = 2 };

// upper_index (largest i in [0, n) with a[i] <= v, a non-decreasing, a[0] <= v)
// for a v that every lane of the wave holds, all 64 lanes active:
// each round splits what is left into 64 sub-ranges and probes the first
// element of every sub-range but the first, one per lane, so a table of up to
// 4096 entries takes two dependent loads instead of about twelve.
template <typename T>
__device__ __forceinline__ int upper_index_wave(const T* a, int n, T v) {
    int lo = 0, hi = n;  // the answer lies in [lo, hi)
    while (hi - lo > 1) {
        const int step = (hi - lo + kWave - 1) / kWave;
        const int p = lo + (static_cast<int>(lane()) + 1) * step;
        const bool le = p < hi && a[p] <= v;
        // a is non-decreasing, so the lanes with le set are the lowest ones
        lo += static_cast<int>(popc64(__ballot(le))) * step;
        hi = min(lo + step, hi);
    }
    return lo;
}

struct alignas(16) SegPlan {
    int64_t off;        // first element in the packed buffer
    int64_t n;          // elements
    int64_t k;          // kept
    int64_t out_off;    // first output slot
    int64_t cand_base;  // first candidate slot entry
    int32_t region_begin, nregions, group_begin, ngroups;
    int32_t cap;        // candidate slots per region
    int32_t mode;
    int32_t sample_chunks, sample_rank;
    int32_t sample_rank_hi, exhaustive, direct, raw_units;  // raw units: kRawChunk elements each
    int32_t compact_split;  // blocks per group in the compaction (a power of two, 1 to 32)
    int32_t cunit_base;     // first entry of the tensor's candidate units in the per-unit count arrays
    int32_t runit_base;     // first entry of its raw units
    int32_t pad[3];
};
static_assert(sizeof(SegPlan) == 112, "SegPlan layout");

// Per-call state of a tensor.  Each field is written by one kernel (the
// tensor's first block in it) and read by later kernels only.
struct alignas(16) SegState {
    uint32_t tlo;       // keys >= tlo become candidates (sample select)
    uint32_t thi;       // stored candidates with key >= thi get e = 0 in the stream
    uint32_t fallback;  // the exact full-pass selection (compaction)
    uint32_t ncand;     // candidates found (compaction)
    uint32_t p0, w0;    // top 11 key bits of T and the rank left below them (first select pass)
    uint32_t p1, w1;    // top 21 bits and the rank left (second select pass)
    uint32_t T, r;      // the k-th largest key and the ties kept (write pass, the first block)
    // exact fallback: the first digits [spec_lo, spec_lo + spec_n) that the
    // sample's window [tlo, thi) spans, whose second-digit histograms the
    // compaction builds with the first one; hit = 1 + the one that held T's
    // (its histogram stands in for the first select pass), else 0
    uint32_t spec_lo, spec_n, hit;
    uint32_t pad[3];
};
static_assert(sizeof(SegState) == 64, "SegState layout");

// ------------------------------------------------------------------ host plan
// A vector with inline room for N elements: a call over one tensor builds its
// plan without touching the host heap (the allocation-free entry point relies
// on it); longer plans spill to a std::vector.
template <typename T, size_t N>
class SmallVec {
public:
    size_t size() const { return n_; }
    T* data() { return n_ <= N ? inl_ : heap_.data(); }
    const T* data() const { return n_ <= N ? inl_ : heap_.data(); }
    T& operator[](size_t i) { return data()[i]; }
    const T& operator[](size_t i) const { return data()[i]; }
    T* begin() { return data(); }
    T* end() { return data() + n_; }
    void assign(size_t n, const T& v) {
        n_ = n;
        if (n > N) heap_.assign(n, v);
        else for (size_t i = 0; i < n; ++i) inl_[i] = v;
    }

private:
    size_t n_ = 0;
    T inl_[N];
    std::vector<T> heap_;
};

struct Plan {
    int32_t nseg = 0;
    int64_t R = 0;      // regions (waves of the streaming pass)
    int64_t G = 0;      // region groups
    int64_t SB = 0;     // sample blocks
    int32_t sample_rounds = 1;  // groups of kSampleBlockChunks chunks per sample block
    int32_t hcopies = 1;        // copies of each radix histogram (blocks add to copy blockIdx % hcopies)
    int64_t QR = 0;     // raw units (fallback units) of every tensor
    int64_t QC = 0;     // bound on candidate units (kChunk entries each)
    int64_t HB = 0;     // select / emit blocks (static share of each tensor: hb)
    int64_t Ctot = 0;   // candidate slot entries
    int64_t CB = 0;     // compaction blocks
    bool any_normal = false;
    SmallVec<SegPlan, 1> seg;
    SmallVec<int32_t, 2> rb, gbb, sbb, cbb, hb;  // prefix tables, nseg+1 each
};

struct Layout {
    size_t status, plan, rb, gbb, sbb, cbb, hb, static_end, hint;
    size_t state, shist, rhist, grp_cnt, zero_end;
    size_t region_cnt, cpair, dval, didx, bh, spart, gpart, cpart, rpart;
    size_t total;
};

// The part of the layout that depends on the number of tensors alone: the
// tables, the hints and the per-tensor state (L.status .. L.state).
static size_t layout_prefix(size_t ns, Layout& L) {
    size_t at = 0;
    auto take = [&](size_t bytes) { size_t o = at; at = round_up(at + bytes, 256); return o; };
    // word 0: indices the call found out of their tensor's range in its own
    // workspace entries (written as part of the tables, so it starts at 0)
    L.status = take(256);
    L.plan = take(ns * sizeof(SegPlan));
    L.rb = at; at += (ns + 1) * 4;
    L.gbb = at; at += (ns + 1) * 4;
    L.sbb = at; at += (ns + 1) * 4;
    L.cbb = at; at += (ns + 1) * 4;
    L.hb = at; at += (ns + 1) * 4;
    at = round_up(at, 256);
    L.static_end = at;
    // each tensor's exact threshold of the last call, kept from call to call
    // (neither the tables' copy nor the clearing touches it)
    L.hint = take(ns * 4);
    L.state = take(ns * sizeof(SegState));
    return at;
}

static Layout make_layout(const Plan& p) {
    Layout L{};
    size_t at = layout_prefix(static_cast<size_t>(p.nseg), L);
    auto take = [&](size_t bytes) { size_t o = at; at = round_up(at + bytes, 256); return o; };
    const size_t ns = static_cast<size_t>(p.nseg);
    L.shist = take(ns * static_cast<size_t>(p.hcopies) * kSampleStride * 4);
    L.rhist = take((3 + kSpec) * ns * static_cast<size_t>(p.hcopies) * kHistWords * 4);
    L.grp_cnt = take(static_cast<size_t>(p.G) * 4);
    L.zero_end = at;
    L.region_cnt = take(static_cast<size_t>(p.R) * 4);
    L.cpair = take(static_cast<size_t>(p.Ctot) * 8);
    L.dval = take(static_cast<size_t>(p.Ctot) * 4);
    L.didx = take(static_cast<size_t>(p.Ctot) * 4);
    // per select block: the suffix sums of its last radix histogram
    L.bh = take(static_cast<size_t>(p.HB) * kBlockHistWords * 4);
    // monitoring partials (sent, dropped energy): per region, per candidate unit, per raw unit
    L.spart = take(static_cast<size_t>(p.R) * 16);
    L.gpart = take(static_cast<size_t>(p.G) * 16);
    L.cpart = take(static_cast<size_t>(p.QC) * 16);
    L.rpart = take(static_cast<size_t>(p.QR) * 16);
    L.total = at;
    return L;
}

// Builds the per-tensor plan; validates the tables.
static int make_plan(int32_t nseg, const int64_t* off, const int64_t* ks, Plan& p) {
    if (nseg < 0) return fail(EF_EINVAL, "nseg must be >= 0 (got %d)", nseg);
    if (nseg > 0 && (!off || !ks)) return fail(EF_EINVAL, "segment tables must not be NULL");
    if (nseg > 0 && off[0] < 0) return fail(EF_EINVAL, "seg_off[0] must be >= 0");
    for (int32_t s = 0; s < nseg; ++s)
        if (off[s + 1] < off[s]) return fail(EF_EINVAL, "seg_off must be non-decreasing (segment %d)", s);
    if (nseg > 0 && off[nseg] > kMaxElems) return fail(EF_EINVAL, "packed buffer exceeds 2^31-1 elements");
    p = Plan{};
    p.nseg = nseg;
    p.seg.assign(nseg, SegPlan{});
    p.rb.assign(nseg + 1, 0);
    p.gbb.assign(nseg + 1, 0);
    p.sbb.assign(nseg + 1, 0);
    p.cbb.assign(nseg + 1, 0);
    p.hb.assign(nseg + 1, 0);
    int64_t out = 0;
    for (int32_t s = 0; s < nseg; ++s) {
        const int64_t n = off[s + 1] - off[s];
        const int64_t k = ks[s];
        if (k < 0 || k > n) return fail(EF_EINVAL, "segment %d: k=%lld outside [0, n=%lld]", s, (long long)k, (long long)n);
        SegPlan& P = p.seg[s];
        memset(&P, 0, sizeof P);
        P.off = off[s];
        P.n = n;
        P.k = k;
        P.out_off = out;
        out += k;
        P.mode = (k == 0) ? MODE_NONE : (k == n ? MODE_ALL : MODE_NORMAL);
        P.nregions = static_cast<int32_t>(cdiv(n, kRegion));
        P.ngroups = static_cast<int32_t>(cdiv(P.nregions, kGroup));
        if (P.mode == MODE_NORMAL) {
            // Sample: every element of small tensors, else 1/16 of the 256-element
            // chunks (at least 256 and at most 4096 chunks), evenly spaced.  On the
            // layer-wise BERT-base layout 1/16 reads 6 % of the data instead of
            // 12.5 % and is 3 % faster per step than 1/8; 1/32 gained nothing more.
            const int64_t chunks = cdiv(n, kSampleChunk);
            int64_t S = std::min<int64_t>(kSampleChunksMax, chunks / kSampleDiv);
            S = std::min<int64_t>(chunks, std::max<int64_t>(kSampleChunksMin, S));
            const bool exhaustive = (S == chunks);
            const int64_t S_el = exhaustive ? n : S * kSampleChunk;
            int64_t m, m_hi;
            if (exhaustive) {
                // exact histogram: the bin holding the k-th largest key bounds T from below,
                // the bin above it bounds it from above
                m = k;
                m_hi = k;
            } else {
                // mu = expected sample count above the k-th largest key; rank m is
                // above that by 8 standard deviations plus 64, rank m_hi below it
                const double mu = static_cast<double>(k) * static_cast<double>(S_el) / static_cast<double>(n);
                m = static_cast<int64_t>(ceil(mu + 8.0 * sqrt(mu))) + 64;
                m = std::min<int64_t>(S_el, m);
                m_hi = static_cast<int64_t>(floor(mu - 4.0 * sqrt(mu))) - 16;
                if (m_hi < 1) m_hi = 0;
            }
            const double rho = static_cast<double>(m) / static_cast<double>(S_el);
            const int64_t region_len = std::min<int64_t>(n, kRegion);
            if (rho * 3.0 >= 0.5) {
                // dense selection: candidates would not save anything; take the
                // exact full-pass path directly
                P.direct = 1;
                P.cap = 0;
                P.compact_split = 1;
            } else {
                int64_t cap = static_cast<int64_t>(ceil(kRegion * rho * 3.0)) + 32;
                cap = static_cast<int64_t>(round_up(static_cast<size_t>(cap), 4));
                P.cap = static_cast<int32_t>(std::min<int64_t>(cap, region_len));
                P.sample_chunks = static_cast<int32_t>(S);
                P.sample_rank = static_cast<int32_t>(m);
                P.sample_rank_hi = static_cast<int32_t>(m_hi);
                P.exhaustive = exhaustive ? 1 : 0;
                // at most about 512 expected candidates per compaction block (up to
                // 32 blocks per group of 256 regions, 8 regions each): the
                // block's time is a chain of dependent steps, and where the large
                // values crowd into a few groups, short blocks keep those groups
                // from holding up the rest (a flat 108.9M-element call over the
                // BERT-base tensors: compaction 51 us with 2048, 19 us with 512)
                const double per_group = std::min<double>(P.nregions, kGroup) * std::min<double>(region_len, kRegion * rho);
                P.compact_split = 1;
                while (P.compact_split < 32 && per_group > 512.0 * P.compact_split) P.compact_split *= 2;
            }
            P.raw_units = static_cast<int32_t>(cdiv(n, kRawChunk));
            p.any_normal = true;
        }
        P.cand_base = p.Ctot;
        P.cunit_base = static_cast<int32_t>(p.QC);
        P.runit_base = static_cast<int32_t>(p.QR);
        p.Ctot += static_cast<int64_t>(P.nregions) * P.cap;
        p.QC += cdiv(static_cast<int64_t>(P.nregions) * P.cap, kChunk);
        P.region_begin = static_cast<int32_t>(p.R);
        P.group_begin = static_cast<int32_t>(p.G);
        p.rb[s] = static_cast<int32_t>(p.R);
        p.gbb[s] = static_cast<int32_t>(p.G);
        p.R += P.nregions;
        p.G += P.ngroups;
        p.SB += P.sample_chunks;  // total sample chunks for now; blocks below
        p.QR += P.raw_units;
        p.cbb[s] = static_cast<int32_t>(p.CB);
        if (P.mode == MODE_NORMAL) p.CB += static_cast<int64_t>(P.ngroups) * P.compact_split;
    }
    // Sample blocks: many small tensors would otherwise give thousands of blocks,
    // each clearing and flushing a whole 4096-bin histogram; beyond about
    // kSampleBlocksTarget blocks every block takes several chunk groups.
    // A tensor's sampling, compaction and histogram blocks run on every XCD;
    // their atomics on one histogram meet beyond the L2s and are applied in
    // turn.  With few tensors (few histograms, many blocks each) every sample
    // and radix histogram gets eight copies, one per XCD (blocks are handed to
    // the XCDs in turn, so block b adds to copy b % 8); with many tensors, or
    // a small call, the blocks per histogram are few anyway, and one copy
    // spares the clearing and the reading of the others.
    p.hcopies = (nseg <= 8 && p.R >= kFewRegions) ? kHistCopies : 1;
    p.sample_rounds = static_cast<int32_t>(std::min<int64_t>(
        kSampleRoundsMax, std::max<int64_t>(1, cdiv(p.SB, static_cast<int64_t>(kSampleBlockChunks) * kSampleBlocksTarget))));
    p.SB = 0;
    for (int32_t s = 0; s < nseg; ++s) {
        p.sbb[s] = static_cast<int32_t>(p.SB);
        p.SB += cdiv(p.seg[s].sample_chunks, static_cast<int64_t>(kSampleBlockChunks) * p.sample_rounds);
    }
    // Compaction blocks: splitting a group pays while the grid fits on the
    // GPU at once; beyond kCompactBlocksMax blocks a second round would start,
    // so the splits are halved until the grid fits or every split is 1.
    while (p.CB > kCompactBlocksMax) {
        bool any = false;
        for (auto& P : p.seg)
            if (P.compact_split > 1) {
                P.compact_split /= 2;
                any = true;
            }
        if (!any) break;
        p.CB = 0;
        for (int32_t s = 0; s < nseg; ++s) {
            p.cbb[s] = static_cast<int32_t>(p.CB);
            if (p.seg[s].mode == MODE_NORMAL) p.CB += static_cast<int64_t>(p.seg[s].ngroups) * p.seg[s].compact_split;
        }
    }
    p.rb[nseg] = static_cast<int32_t>(p.R);
    p.gbb[nseg] = static_cast<int32_t>(p.G);
    p.sbb[nseg] = static_cast<int32_t>(p.SB);
    p.cbb[nseg] = static_cast<int32_t>(p.CB);
    p.QC += 1;
    // Select / emit blocks: each tensor that selects gets a fixed share of
    // about kSelectBlocks blocks, in proportion to its size (at least one, at
    // most one per raw unit), so that a block finds its tensor in a static
    // table and strides over the tensor's units, whichever path it takes.
    int64_t raw_total = 0;
    for (int32_t s = 0; s < nseg; ++s)
        if (p.seg[s].mode == MODE_NORMAL) raw_total += p.seg[s].raw_units;
    p.HB = 0;
    for (int32_t s = 0; s < nseg; ++s) {
        p.hb[s] = static_cast<int32_t>(p.HB);
        const SegPlan& P = p.seg[s];
        if (P.mode != MODE_NORMAL) continue;
        const int64_t share = raw_total > 0 ? kSelectBlocks * static_cast<int64_t>(P.raw_units) / raw_total : 0;
        p.HB += std::max<int64_t>(1, std::min<int64_t>(P.raw_units, share));
    }
    p.hb[nseg] = static_cast<int32_t>(p.HB);
    return EF_OK;
}

// ------------------------------------------------------------------ kernels
// Clears the per-call state and writes the plan tables into the workspace:
// a small plan from the kernel arguments (chunk c), a cached one from pinned
// host memory (tsrc, tvec 16-byte words; every block copies a slice).
__global__ __launch_bounds__(kBlock) void k_init(uint4* zero, int64_t nvec, uint32_t* nonfinite, uint32_t* dst,
                                                 WordChunk c, const uint4* __restrict__ tsrc, int64_t tvec) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < nvec; i += stride)
        zero[i] = make_uint4(0, 0, 0, 0);
    uint4* tdst = reinterpret_cast<uint4*>(dst);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < tvec; i += stride)
        tdst[i] = tsrc[i];
    if (blockIdx.x == 0) {
        for (uint32_t i = threadIdx.x; i < c.n; i += kBlock) dst[i] = c.w[i];
        if (nonfinite && threadIdx.x == 0) *nonfinite = 0;
    }
}

// The window of fine sample bins of a tensor whose previous exact threshold
// was `hint`: [base, base + kFineSpan), centred on the hint (rounded down to
// a fine bin edge).  Any 32-bit value is a valid hint: a workspace holding
// something else only leaves the window where no rank falls.
__device__ __forceinline__ uint32_t fine_base(uint32_t hint) {
    const uint32_t c = (hint & 0x7fffffffu) & ~((1u << kFineShift) - 1u);
    return c >= kFineSpan / 2 ? c - kFineSpan / 2 : 0u;
}

// The sample histograms (top 12 key bits of x = g + e, and with FINE the fine
// window at fbase) of one block's `rounds` consecutive groups of
// kSampleBlockChunks chunks of a tensor (block bl of the tensor), in the LDS
// histograms h and hf, which it clears first; *above_lds gets the block's
// count of samples above the fine window.  Every thread of the block calls
// it; the histograms are complete on return.
__device__ __forceinline__ void sample_block(const float* __restrict__ g, const float* __restrict__ e,
                                             const SegPlan& P, int bl, int32_t rounds, bool fine, uint32_t fbase,
                                             uint32_t* h, uint32_t* hf, uint32_t* above_lds) {
    const int64_t off = P.off, n = P.n;
    const int S = P.sample_chunks;
    const bool exhaustive = P.exhaustive != 0;
    for (int i = threadIdx.x; i < kSampleBins; i += kSampleBlock) h[i] = 0;
    if (fine)
        for (int i = threadIdx.x; i < kFineBins; i += kSampleBlock) hf[i] = 0;
    if (threadIdx.x == 0) *above_lds = 0;
    __syncthreads();
    const int w = threadIdx.x / kWave;
    const int l = lane();
    uint32_t above = 0;
    for (int rd = 0; rd < rounds; ++rd) {
        const int c0 = (bl * rounds + rd) * kSampleBlockChunks + w * kSampleChunksPerWave;
        if (c0 >= S) break;  // wave-uniform: the rest of this block's chunks lie past the sample
        float xs[kSampleChunksPerWave][4];
        bool ok[kSampleChunksPerWave][4];
#pragma unroll
        for (int u = 0; u < kSampleChunksPerWave; ++u) {
            const int c = c0 + u;
            int64_t start = 0;
            if (exhaustive) start = static_cast<int64_t>(c) * kSampleChunk;
            else if (S > 1) start = static_cast<int64_t>(c) * (n - kSampleChunk) / (S - 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // every load is issued before any is used: a position past the
                // sample or the tensor reads the tensor's last element (n >= 1)
                const int64_t loc = start + j * kWave + l;
                ok[u][j] = (c < S) && (loc < n);
                const int64_t at = off + min(loc, n - 1);
                const float x = g[at] + e[at];
                xs[u][j] = ok[u][j] ? x : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < kSampleChunksPerWave; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (ok[u][j]) {
                    const uint32_t key = key_of(xs[u][j]);
                    atomicAdd(&h[key >> kSampleShift], 1u);
                    if (fine) {
                        const uint32_t d = key - fbase;  // wraps for keys below the window
                        if (d < kFineSpan) atomicAdd(&hf[d >> kFineShift], 1u);
                        else above += key >= fbase ? 1u : 0u;
                    }
                }
    }
    if (fine) {
        above = wave_sum(above);
        if (l == 0 && above) atomicAdd(above_lds, above);
    }
    __syncthreads();
}

// Coarse bin c (64 fine bins) of an LDS sample histogram, read with a
// rotation so that the lanes hit different banks.
__device__ __forceinline__ uint32_t sample_coarse(const uint32_t* h, int c) {
    uint32_t t = 0;
    for (int i = 0; i < 64; ++i) t += h[c * 64 + ((i + c) & 63)];
    return t;
}

// 1. sample histograms, each block adding its own to copy b % hcopies of its
//    tensor's (12-bit bins and their coarse sums; with `fine`, the fine window
//    around the tensor's hint, its group sums and the count above it)
__global__ __launch_bounds__(kSampleBlock) void k_sample(const float* __restrict__ g, const float* __restrict__ e,
                                                   const SegPlan* __restrict__ plan, int32_t nseg,
                                                   const int32_t* __restrict__ sbb, int32_t rounds,
                                                   uint32_t* __restrict__ shist, int32_t hcopies,
                                                   const uint32_t* __restrict__ hint, int32_t fine) {
    __shared__ uint32_t h[kSampleBins];
    __shared__ uint32_t hf[kFineBins];
    __shared__ uint32_t above;
    const int b = blockIdx.x;
    const int s = upper_index_wave(sbb, nseg, b);
    const uint32_t fbase = fine ? fine_base(hint[s]) : 0u;
    sample_block(g, e, plan[s], b - sbb[s], rounds, fine != 0, fbase, h, hf, &above);
    uint32_t* gh = shist + (static_cast<size_t>(s) * hcopies + blockIdx.x % hcopies) * kSampleStride;
    for (int c = threadIdx.x; c < kSampleCoarse; c += kSampleBlock) {
        const uint32_t t = sample_coarse(h, c);
        if (t) atomicAdd(&gh[kSampleBins + c], t);
    }
    for (int i = threadIdx.x; i < kSampleBins; i += kSampleBlock)
        if (h[i]) atomicAdd(&gh[i], h[i]);
    if (!fine) return;
    uint32_t* gf = gh + kSampleWords;
    for (int c = threadIdx.x; c < kFineGroups; c += kSampleBlock) {
        const uint32_t t = sample_coarse(hf, c);
        if (t) atomicAdd(&gf[kFineBins + c], t);
    }
    for (int i = threadIdx.x; i < kFineBins; i += kSampleBlock)
        if (hf[i]) atomicAdd(&gf[i], hf[i]);
    if (threadIdx.x == 0 && above) atomicAdd(&gf[kFineBins + kFineGroups], above);
}

// T_lo, T_hi and the guessed first digits of tensor s from its sample
// histograms (the hcopies <= C copies summed), found by one wave; every lane
// calls it and gets the results.  T_lo is the lower edge of the bin holding
// the sample's rank P.sample_rank (0 when the sample holds fewer), T_hi the
// upper edge of the bin holding rank P.sample_rank_hi (none when that rank is
// 0 or the sample holds fewer), counting from the top, each rank taken in the
// fine window at fbase when the window holds it and in the 12-bit bins
// otherwise.  Both ranks are searched together in two rounds of loads: the
// group sums of the 12-bit bins and of the fine window (with the count above
// the window), then the 64 bins of the group each rank falls in.
template <int C>
__device__ __forceinline__ void wave_sample_edges(const uint32_t* shist, int32_t hcopies, const SegPlan& P, int s,
                                                  uint32_t fbase, uint32_t* tlo, uint32_t* thi, uint32_t* spec_lo,
                                                  uint32_t* spec_n) {
    const int l = static_cast<int>(lane());
    const uint32_t* h0 = shist + static_cast<size_t>(s) * hcopies * kSampleStride;
    const uint32_t rank[2] = {static_cast<uint32_t>(P.sample_rank), static_cast<uint32_t>(P.sample_rank_hi)};
    // round 1 (lane l: 12-bit group 63 - l, fine group 31 - l, the top first)
    uint32_t cw[C], gw[C], aw[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const uint32_t* hc = h0 + static_cast<size_t>(c < hcopies ? c : 0) * kSampleStride;
        cw[c] = hc[kSampleBins + 63 - l];
        gw[c] = hc[kSampleWords + kFineBins + (l < kFineGroups ? kFineGroups - 1 - l : 0)];
        aw[c] = hc[kSampleWords + kFineBins + kFineGroups];
    }
    uint32_t cv = 0, gv = 0, ab = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (c >= hcopies) break;
        cv += cw[c];
        gv += l < kFineGroups ? gw[c] : 0u;
        ab += aw[c];
    }
    const uint32_t ccum = wave_incl_scan(cv);  // samples in the top l + 1 groups of 12-bit bins
    const uint32_t gcum = wave_incl_scan(gv);  // samples in the top l + 1 fine groups
    const uint32_t ctot = __shfl(ccum, kWave - 1, kWave), wtot = __shfl(gcum, kWave - 1, kWave);
    bool found[2], fine[2];
    uint32_t grp[2], abv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t want = rank[i];
        fine[i] = want > ab && want - ab <= wtot;
        found[i] = want > 0 && ctot >= want;
        const uint64_t hit = fine[i] ? __ballot(l < kFineGroups && ab + gcum >= want) : __ballot(ccum >= want);
        const int L = hit ? static_cast<int>(__ffsll(static_cast<long long>(hit))) - 1 : 0;
        grp[i] = fine[i] ? static_cast<uint32_t>(kFineGroups - 1 - L) : static_cast<uint32_t>(63 - L);
        abv[i] = fine[i] ? ab + __shfl(gcum, L, kWave) - __shfl(gv, L, kWave)
                         : __shfl(ccum, L, kWave) - __shfl(cv, L, kWave);
    }
    // round 2 (lane l: bin 64 grp + 63 - l of each rank's group)
    uint32_t bw[2][C];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const uint32_t* hc = h0 + static_cast<size_t>(c < hcopies ? c : 0) * kSampleStride;
            bw[i][c] = hc[(fine[i] ? kSampleWords : 0) + 64 * grp[i] + 63 - l];
        }
    uint32_t edge[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (c >= hcopies) break;
            v += bw[i][c];
        }
        const uint32_t cum = wave_incl_scan(v);
        const uint64_t hit = __ballot(abv[i] + cum >= rank[i]);
        const int L = hit ? static_cast<int>(__ffsll(static_cast<long long>(hit))) - 1 : 63;
        const uint32_t bin = 64 * grp[i] + 63 - static_cast<uint32_t>(L) + (i == 1 ? 1u : 0u);  // T_hi: upper edge
        edge[i] = fine[i] ? fbase + (bin << kFineShift) : bin << kSampleShift;
    }
    *tlo = found[0] ? edge[0] : 0u;
    *thi = found[1] ? edge[1] : kNoKey;
    const uint32_t lo = *tlo >> 20, hi = *thi == kNoKey ? kRadixBins - 1 : (*thi - 1) >> 20;
    *spec_lo = lo;
    *spec_n = hi - lo + 1 <= static_cast<uint32_t>(kSpec) ? hi - lo + 1 : 0u;
}

// 1b. T_lo and T_hi of each tensor (one wave per tensor), for calls whose
//     stream blocks do not find them themselves
__global__ __launch_bounds__(kWave) void k_sample_select(const SegPlan* __restrict__ plan,
                                                         const uint32_t* __restrict__ shist, int32_t hcopies,
                                                         const uint32_t* __restrict__ hint,
                                                         SegState* __restrict__ st) {
    const int s = blockIdx.x;
    const SegPlan& P = plan[s];
    if (P.mode != MODE_NORMAL || P.direct) return;
    uint32_t lo, hi, sl, sn;
    wave_sample_edges<kHistCopies>(shist, hcopies, P, s, fine_base(hint[s]), &lo, &hi, &sl, &sn);
    if (lane() == 0) {
        st[s].tlo = lo;
        st[s].thi = hi;
        st[s].spec_lo = sl;
        st[s].spec_n = sn;
    }
}

typedef float f4 __attribute__((ext_vector_type(4)));

// Appends the hits of one group of 64 lanes x NV consecutive elements to the
// wave's candidate slot, preserving index order: lane l owns elements
// [gidx0, gidx0 + NV) and lanes are in index order.  stored[j] tells whether
// element j went into the slot (false once the slot is full).
template <int NV>
__device__ __forceinline__ void append_hits(const float (&x)[NV], const bool (&hit)[NV], int64_t gidx0,
                                            uint32_t& cnt, uint32_t cap, uint2* __restrict__ cp,
                                            bool (&stored)[NV]) {
    uint64_t bal[NV];
    uint64_t any = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        bal[j] = __ballot(hit[j]);
        any |= bal[j];
        stored[j] = false;
    }
    if (!any) return;
    uint32_t pos = cnt;
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        pos += count_below(bal[j]);
        tot += popc64(bal[j]);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        if (hit[j]) {
            if (pos < cap) {
                cp[pos] = make_uint2(__float_as_uint(x[j]), static_cast<uint32_t>(gidx0 + j));
                stored[j] = true;
            }
            ++pos;
        }
    }
    cnt += tot;
}

// e value written by the stream for one element
template <int MODE>
__device__ __forceinline__ float stream_e(float x, uint32_t key, bool stored, uint32_t thi) {
    if (MODE == MODE_ALL) return 0.0f;
    if (MODE == MODE_NORMAL && stored && key >= thi) return 0.0f;
    return x;
}

// Square of a finite value in float64 (exact), 0 for Inf / NaN.
__device__ __forceinline__ double sq_finite(float x, uint32_t key) {
    const double d = static_cast<double>(x);
    return key < 0x7f800000u ? d * d : 0.0;
}

template <int MODE, bool STATS>
__device__ __forceinline__ void stream_region(const float* __restrict__ g, float* __restrict__ e, int64_t gbeg,
                                              int64_t gend, uint32_t tlo, uint32_t thi, uint32_t cap,
                                              uint2* __restrict__ cp, float* __restrict__ vals,
                                              int32_t* __restrict__ idx,
                                              int64_t out_base, uint32_t& cnt, uint32_t& nf, double& acc) {
    const int l = lane();
    // body [a, bnd) is 16-byte aligned (g and e are 16-byte aligned)
    int64_t a = (gbeg + 3) & ~static_cast<int64_t>(3);
    int64_t bnd = gend & ~static_cast<int64_t>(3);
    if (a > bnd) a = bnd = gend;  // region shorter than one aligned quad
    auto scalar_part = [&](int64_t from, int64_t to) {
        // at most 3 elements, one per lane; lane l <-> index from + l
        const int64_t i = from + l;
        const bool ok = i < to;
        float xv[1] = {0.0f};
        bool hit[1] = {false};
        uint32_t key = 0;
        if (ok) {
            xv[0] = g[i] + e[i];
            key = key_of(xv[0]);
            nf += key >= 0x7f800000u;
            hit[0] = (MODE == MODE_NORMAL) && key >= tlo;
            if (STATS && !hit[0]) acc += sq_finite(xv[0], key);
        }
        bool stored[1] = {false};
        if (MODE == MODE_NORMAL) append_hits<1>(xv, hit, from + l, cnt, cap, cp, stored);
        if (ok) {
            e[i] = stream_e<MODE>(xv[0], key, stored[0], thi);
            if (MODE == MODE_ALL) {
                vals[out_base + (i - gbeg)] = xv[0];
                idx[out_base + (i - gbeg)] = static_cast<int32_t>(i);
            }
        }
    };
    if (gbeg < a) scalar_part(gbeg, a);
    const f4* __restrict__ g4 = reinterpret_cast<const f4*>(g + a);
    f4* __restrict__ e4 = reinterpret_cast<f4*>(e + a);
    const int64_t nv = (bnd - a) >> 2;
    // one iteration: kUnroll float4 of g and of e per lane, all loads issued
    // before the first use; GUARD only for the last, partial iteration
    auto iteration = [&](int64_t base, auto guard) {
        constexpr bool GUARD = decltype(guard)::value;
        f4 gv[kUnroll], ev[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = base + u * kWave + l;
            if (!GUARD || j < nv) {
                gv[u] = __builtin_nontemporal_load(g4 + j);
                ev[u] = __builtin_nontemporal_load(e4 + j);
            } else {
                gv[u] = f4{0.f, 0.f, 0.f, 0.f};
                ev[u] = f4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = base + u * kWave + l;
            const bool ok = !GUARD || j < nv;
            const f4 x = gv[u] + ev[u];
            float xs[4] = {x.x, x.y, x.z, x.w};
            uint32_t key[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) key[t] = key_of(xs[t]);
            // common case in one compare: no candidate and no Inf/NaN among the four
            const uint32_t kmax = max(max(key[0], key[1]), max(key[2], key[3]));
            const uint32_t lim = MODE == MODE_NORMAL ? min(tlo, 0x7f800000u) : 0x7f800000u;
            f4 eo = MODE == MODE_ALL ? f4{0.f, 0.f, 0.f, 0.f} : x;
            const bool rare = ok && kmax >= lim;
            if (STATS && ok && !rare)
                acc += (sq_finite(xs[0], key[0]) + sq_finite(xs[1], key[1])) +
                       (sq_finite(xs[2], key[2]) + sq_finite(xs[3], key[3]));
            if (__ballot(rare)) {
                bool hit[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    nf += (ok && key[t] >= 0x7f800000u) ? 1u : 0u;
                    hit[t] = (MODE == MODE_NORMAL) && ok && key[t] >= tlo;
                    if (STATS && rare && !hit[t]) acc += sq_finite(xs[t], key[t]);
                }
                if (MODE == MODE_NORMAL) {
                    bool stored[4];
                    append_hits<4>(xs, hit, a + 4 * j, cnt, cap, cp, stored);
                    eo = f4{stream_e<MODE>(xs[0], key[0], stored[0], thi),
                            stream_e<MODE>(xs[1], key[1], stored[1], thi),
                            stream_e<MODE>(xs[2], key[2], stored[2], thi),
                            stream_e<MODE>(xs[3], key[3], stored[3], thi)};
                }
            }
            if (ok) {
                __builtin_nontemporal_store(eo, e4 + j);
                if (MODE == MODE_ALL) {
                    const int64_t i0 = a + 4 * j;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        vals[out_base + (i0 + t - gbeg)] = xs[t];
                        idx[out_base + (i0 + t - gbeg)] = static_cast<int32_t>(i0 + t);
                    }
                }
            }
        }
    };
    constexpr int64_t kStep = kWave * kUnroll;
    const int64_t nfull = nv / kStep * kStep;
    for (int64_t base = 0; base < nfull; base += kStep) iteration(base, std::false_type{});
    if (nfull < nv) iteration(nfull, std::true_type{});
    if (bnd < gend) scalar_part(bnd, gend);
}

// 2. the streaming pass; one wave per region of kRegion elements.  With STATS
// each region also records the float64 energy of the elements it already knows
// the fate of (all of them unless they are candidates): spart[w] = {sent, dropped}.
template <bool STATS, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void k_stream(const float* __restrict__ g, float* __restrict__ e,
                                                         const SegPlan* __restrict__ plan, int32_t nseg,
                                                         const int32_t* __restrict__ rb, int64_t R,
                                                         SegState* __restrict__ st,
                                                         uint32_t* __restrict__ region_cnt,
                                                         uint32_t* __restrict__ grp_cnt, uint2* __restrict__ cpair,
                                                         float* __restrict__ vals,
                                                         int32_t* __restrict__ idx, uint32_t* __restrict__ nonfinite,
                                                         double2* __restrict__ spart) {
    __shared__ uint32_t lcnt[WAVES];
    __shared__ int32_t lgrp[WAVES];
    const int64_t w = static_cast<int64_t>(blockIdx.x) * WAVES + threadIdx.x / kWave;
    uint32_t cnt = 0;
    int32_t grp = -1;
    if (w < R) {
        const int s = upper_index_wave(rb, nseg, static_cast<int32_t>(w));
        const SegPlan& P = plan[s];
        const int64_t rl = w - rb[s];
        const int64_t lbeg = rl * kRegion;
        const int64_t lend = min(lbeg + static_cast<int64_t>(kRegion), P.n);
        const int64_t gbeg = P.off + lbeg, gend = P.off + lend;
        const int mode = P.mode;
        uint32_t nf = 0;
        double acc = 0.0;
        const uint32_t cap = static_cast<uint32_t>(P.cap);
        uint2* cp = cpair + P.cand_base + rl * P.cap;
        if (mode == MODE_NORMAL) {
            // a direct (dense) selection collects nothing
            const uint32_t tlo = P.direct ? kNoKey : st[s].tlo;
            const uint32_t thi = P.direct ? kNoKey : st[s].thi;
            stream_region<MODE_NORMAL, STATS>(g, e, gbeg, gend, tlo, thi, cap, cp, vals, idx, 0, cnt, nf, acc);
        } else if (mode == MODE_ALL) {
            stream_region<MODE_ALL, STATS>(g, e, gbeg, gend, 0, 0, 0, cp, vals, idx, P.out_off + lbeg, cnt, nf, acc);
        } else {
            stream_region<MODE_NONE, STATS>(g, e, gbeg, gend, 0, 0, 0, cp, vals, idx, 0, cnt, nf, acc);
        }
        if (STATS) {
            acc = wave_sum(acc);
            if (lane() == 0) spart[w] = mode == MODE_ALL ? make_double2(acc, 0.0) : make_double2(0.0, acc);
        }
        nf = wave_sum(nf);
        if (lane() == 0) {
            // the true count: the slot holds the first min(cnt, cap) candidates
            region_cnt[w] = cnt;
            if (nf && nonfinite) atomicAdd(nonfinite, nf);
        }
        grp = P.group_begin + static_cast<int32_t>(rl / kGroup);
    }
    // Group totals: global atomics per block instead of per region.  The 256 regions of a group run on blocks of every XCD, so
    // their atomics meet at one address outside the L2s and are applied one
    // after another; per region, that queue outlasted the stream by ~50 us.
    if (lane() == 0) {
        lcnt[threadIdx.x / kWave] = cnt;
        lgrp[threadIdx.x / kWave] = cnt ? grp : -1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t g0 = -1;
        uint32_t sum = 0;
        for (int i = 0; i < WAVES; ++i) {
            if (lgrp[i] < 0) continue;
            if (lgrp[i] != g0) {
                if (sum) atomicAdd(&grp_cnt[g0], sum);
                g0 = lgrp[i];
                sum = 0;
            }
            sum += lcnt[i];
        }
        if (sum) atomicAdd(&grp_cnt[g0], sum);
    }
}

// One wave's part [sb, se) of a region that starts at gbeg, in the split
// streaming pass: the head and tail (at most three elements each, one per
// lane) and the 16-byte aligned body, NV float4 of g and of e per lane, all
// loaded before any is used.  Phase 1 counts the wave's candidates into
// wcnt[wave]; after the block's barrier, phase 2 appends them to the
// region's slot after the candidates of the block's earlier waves, in index
// order (head, body rows, tail), and writes e.  *total comes back with the
// region's candidate count.  Every thread of the block calls it.
template <int MODE, bool STATS, int NV, class Edges>
__device__ __forceinline__ void stream_part(const float* __restrict__ g, float* __restrict__ e, int64_t gbeg,
                                            int64_t sb, int64_t se, Edges&& edges, uint32_t cap,
                                            uint2* __restrict__ cp, float* __restrict__ vals,
                                            int32_t* __restrict__ idx, int64_t out_base, uint32_t* wcnt,
                                            uint32_t& total, uint32_t& nf, double& acc) {
    const int q = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int l = lane();
    int64_t a = (sb + 3) & ~static_cast<int64_t>(3);
    int64_t b = se & ~static_cast<int64_t>(3);
    if (a > b) a = b = se;  // shorter than one aligned quad: all head
    const int64_t nv = (b - a) >> 2;
    const int64_t ih = sb + l, it = b + l;
    const bool okh = ih < a, okt = it < se;
    const f4* __restrict__ g4 = reinterpret_cast<const f4*>(g + a);
    f4* __restrict__ e4 = reinterpret_cast<f4*>(e + a);
    f4 gv[NV], ev[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int64_t j = u * kWave + l;
        if (j < nv) {
            gv[u] = __builtin_nontemporal_load(g4 + j);
            ev[u] = __builtin_nontemporal_load(e4 + j);
        } else {
            gv[u] = f4{0.f, 0.f, 0.f, 0.f};
            ev[u] = f4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const float xh = okh ? g[ih] + e[ih] : 0.0f;
    const float xt = okt ? g[it] + e[it] : 0.0f;
    f4 xb[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) xb[u] = gv[u] + ev[u];
    // the edges, with the loads in flight (edges() may read the sample
    // histogram and synchronise the block)
    uint32_t tlo = kNoKey, thi = kNoKey;
    edges(tlo, thi);
    // phase 1: the wave's candidates, non-finite values and known energy
    uint32_t mine = 0;
    auto note = [&](float x, bool ok) {
        if (!ok) return;
        const uint32_t key = key_of(x);
        nf += key >= 0x7f800000u ? 1u : 0u;
        const bool hit = MODE == MODE_NORMAL && key >= tlo;
        mine += hit ? 1u : 0u;
        if (STATS && !hit) acc += sq_finite(x, key);
    };
    note(xh, okh);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const bool ok = u * kWave + l < nv;
        note(xb[u].x, ok);
        note(xb[u].y, ok);
        note(xb[u].z, ok);
        note(xb[u].w, ok);
    }
    note(xt, okt);
    mine = wave_sum(mine);
    if (l == 0) wcnt[q] = mine;
    __syncthreads();
    uint32_t cnt = 0;
    total = 0;
    for (int i = 0; i < nw; ++i) {
        cnt += i < q ? wcnt[i] : 0u;
        total += wcnt[i];
    }
    // phase 2: append after the earlier waves' candidates, write e
    auto one = [&](float x, bool ok, int64_t i) {
        const uint32_t key = key_of(x);
        float xa[1] = {x};
        bool ha[1] = {MODE == MODE_NORMAL && ok && key >= tlo};
        bool sa[1] = {false};
        if (MODE == MODE_NORMAL) append_hits<1>(xa, ha, i, cnt, cap, cp, sa);
        if (ok) {
            e[i] = stream_e<MODE>(x, key, sa[0], thi);
            if (MODE == MODE_ALL) {
                vals[out_base + (i - gbeg)] = x;
                idx[out_base + (i - gbeg)] = static_cast<int32_t>(i);
            }
        }
    };
    one(xh, okh, ih);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int64_t j = u * kWave + l;
        const bool ok = j < nv;
        float xs[4] = {xb[u].x, xb[u].y, xb[u].z, xb[u].w};
        uint32_t key[4];
        bool hit[4], stored[4] = {false, false, false, false};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            key[t] = key_of(xs[t]);
            hit[t] = MODE == MODE_NORMAL && ok && key[t] >= tlo;
        }
        if (MODE == MODE_NORMAL) append_hits<4>(xs, hit, a + 4 * j, cnt, cap, cp, stored);
        if (ok) {
            __builtin_nontemporal_store(f4{stream_e<MODE>(xs[0], key[0], stored[0], thi),
                                           stream_e<MODE>(xs[1], key[1], stored[1], thi),
                                           stream_e<MODE>(xs[2], key[2], stored[2], thi),
                                           stream_e<MODE>(xs[3], key[3], stored[3], thi)},
                                        e4 + j);
            if (MODE == MODE_ALL) {
                const int64_t i0 = a + 4 * j;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    vals[out_base + (i0 + t - gbeg)] = xs[t];
                    idx[out_base + (i0 + t - gbeg)] = static_cast<int32_t>(i0 + t);
                }
            }
        }
    }
    one(xt, okt, it);
}

// 2'. The streaming pass of a call with few regions (fewer than
// kFewRegions): one block of SPLIT waves per region, wave q taking the
// region's elements [q L, (q + 1) L), L = kRegion / SPLIT, so that a small
// call still puts several waves on every CU.  The candidates land in the
// region's slot in index order, as one wave over the region would put them
// (stream_part); the block adds the region's count to its group total.
template <bool STATS, int SPLIT>
__global__ __launch_bounds__(SPLIT * kWave) void k_stream_split(const float* __restrict__ g, float* __restrict__ e,
                                                               const SegPlan* __restrict__ plan, int32_t nseg,
                                                               const int32_t* __restrict__ rb,
                                                               SegState* __restrict__ st,
                                                               uint32_t* __restrict__ region_cnt,
                                                               uint32_t* __restrict__ grp_cnt,
                                                               uint2* __restrict__ cpair, float* __restrict__ vals,
                                                               int32_t* __restrict__ idx,
                                                               uint32_t* __restrict__ nonfinite,
                                                               double2* __restrict__ spart,
                                                               const uint32_t* __restrict__ shist,
                                                               int32_t hcopies,
                                                               const uint32_t* __restrict__ hint) {
    constexpr int L = kRegion / SPLIT;
    constexpr int NV = L / (4 * kWave);
    static_assert(L % (4 * kWave) == 0, "a wave's part is whole rows of 64 float4");
    __shared__ uint32_t wcnt[SPLIT];
    __shared__ double wacc[SPLIT];
    __shared__ uint32_t s_edge[2];
    const int64_t w = blockIdx.x;  // the region (one block each)
    const int q = threadIdx.x / kWave;
    const int s = upper_index_wave(rb, nseg, static_cast<int32_t>(w));
    const SegPlan& P = plan[s];
    const int64_t rl = w - rb[s];
    const int64_t lbeg = rl * kRegion;
    const int64_t lend = min(lbeg + static_cast<int64_t>(kRegion), P.n);
    const int64_t gbeg = P.off + lbeg, gend = P.off + lend;
    const int64_t sb = min(gbeg + static_cast<int64_t>(q) * L, gend), se = min(sb + L, gend);
    const uint32_t cap = static_cast<uint32_t>(P.cap);
    uint2* cp = cpair + P.cand_base + rl * P.cap;
    uint32_t total = 0, nf = 0;
    double acc = 0.0;
    auto none = [](uint32_t&, uint32_t&) {};
    if (P.mode == MODE_NORMAL) {
        // T_lo and T_hi straight from the sample histogram (no select launch):
        // the first wave reads them off while the block's loads are in
        // flight; the tensor's first block records them for later kernels.
        // A direct (dense) selection collects nothing.
        auto edges = [&](uint32_t& tlo, uint32_t& thi) {
            if (P.direct) return;
            if (q == 0) {
                uint32_t lo, hi, sl, sn;
                wave_sample_edges<1>(shist, hcopies, P, s, fine_base(hint[s]), &lo, &hi, &sl, &sn);
                if (lane() == 0) {
                    s_edge[0] = lo;
                    s_edge[1] = hi;
                    if (rl == 0) {
                        st[s].tlo = lo;
                        st[s].thi = hi;
                        st[s].spec_lo = sl;
                        st[s].spec_n = sn;
                    }
                }
            }
            __syncthreads();
            tlo = s_edge[0];
            thi = s_edge[1];
        };
        stream_part<MODE_NORMAL, STATS, NV>(g, e, gbeg, sb, se, edges, cap, cp, vals, idx, 0, wcnt, total, nf, acc);
    } else if (P.mode == MODE_ALL) {
        stream_part<MODE_ALL, STATS, NV>(g, e, gbeg, sb, se, none, 0, cp, vals, idx, P.out_off + lbeg, wcnt, total,
                                         nf, acc);
    } else {
        stream_part<MODE_NONE, STATS, NV>(g, e, gbeg, sb, se, none, 0, cp, vals, idx, 0, wcnt, total, nf, acc);
    }
    nf = wave_sum(nf);
    if (lane() == 0 && nf && nonfinite) atomicAdd(nonfinite, nf);
    if (STATS) {
        acc = wave_sum(acc);
        if (lane() == 0) wacc[q] = acc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        region_cnt[w] = total;  // the true count: the slot holds the first min(total, cap)
        if (total) atomicAdd(&grp_cnt[P.group_begin + static_cast<int32_t>(rl / kGroup)], total);
        if (STATS) {
            double t = 0.0;
            for (int i = 0; i < SPLIT; ++i) t += wacc[i];
            spart[w] = P.mode == MODE_ALL ? make_double2(t, 0.0) : make_double2(0.0, t);
        }
    }
}

// Radix histogram of pass p (0..2) of tensor s, copy c: kRadixBins fine bins
// then kCoarse coarse ones.  Each pass has its own histograms, cleared by
// k_init, so no kernel has to clear one after use.
__device__ __forceinline__ uint32_t* radix_hist(uint32_t* rhist, int pass, int s, int c, int32_t nseg,
                                                int32_t hcopies) {
    return rhist + ((static_cast<size_t>(pass) * nseg + s) * hcopies + c) * kHistWords;
}

// Sum of the 32 fine bins of coarse bin c of an LDS histogram, read with a
// rotation so that the lanes of a wave hit different banks.
__device__ __forceinline__ uint32_t coarse_sum(const uint32_t* h, int c) {
    uint32_t t = 0;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) t += h[c * 32 + ((i + c) & 31)];
    return t;
}

// Adds a block's LDS histogram h (nb fine bins) to the global one gh: the
// fine bins that are not zero, then the coarse sums.  Every thread of the
// block calls it; h is not changed.
__device__ __forceinline__ void flush_hist(const uint32_t* h, int nb, uint32_t* gh) {
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += kBlock)
        if (h[i]) atomicAdd(&gh[i], h[i]);
    for (int c = threadIdx.x; c < nb / 32; c += kBlock) {
        const uint32_t t = coarse_sum(h, c);
        if (t) atomicAdd(&gh[kRadixBins + c], t);
    }
}

// The same for one wave's own LDS histogram (the wave's lanes only).
__device__ __forceinline__ void flush_hist_wave(const uint32_t* h, uint32_t* gh) {
    for (int i = lane(); i < kRadixBins; i += kWave)
        if (h[i]) atomicAdd(&gh[i], h[i]);
    const uint32_t t = coarse_sum(h, lane());
    if (t) atomicAdd(&gh[kRadixBins + lane()], t);
}

// The bin d of a tensor's histogram (nb = 2048 or 1024 fine bins, summed over
// its hcopies copies) that holds the want-th largest key: fewer than `want`
// keys lie above d and at least `want` from d up; *above = keys above d.
// Called by a whole wave, every lane gets the result: one round of loads for
// the coarse bins, one for the 32 fine bins of the coarse bin found (all of a
// lane's copies loaded together).  Needs want >= 1 and at least want keys.
__device__ __forceinline__ void wave_find_digit(const uint32_t* gh0, int32_t hcopies, int nb, uint32_t want,
                                                uint32_t* d, uint32_t* above) {
    const int l = static_cast<int>(lane());
    const int nc = nb / 32;
    uint32_t w[kHistCopies];
    // lane l: coarse bin nc - 1 - l (the top one first)
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c)
        w[c] = gh0[(c < hcopies ? c : 0) * kHistWords + kRadixBins + (l < nc ? nc - 1 - l : 0)];
    uint32_t cv = 0;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) cv += (c < hcopies && l < nc) ? w[c] : 0u;
    const uint32_t cum = wave_incl_scan(cv);  // keys in the top l + 1 coarse bins
    const uint64_t hit = __ballot(l < nc && cum >= want);
    const int L = hit ? static_cast<int>(__ffsll(static_cast<long long>(hit))) - 1 : nc - 1;
    const int cb = nc - 1 - L;
    const uint32_t above_c = __shfl(cum, L, kWave) - __shfl(cv, L, kWave);
    // lane l < 32: fine bin 32 cb + 31 - l
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c)
        w[c] = gh0[(c < hcopies ? c : 0) * kHistWords + 32 * cb + (l < 32 ? 31 - l : 0)];
    uint32_t fv = 0;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) fv += (c < hcopies && l < 32) ? w[c] : 0u;
    const uint32_t cum2 = wave_incl_scan(fv);
    const uint64_t hit2 = __ballot(l < 32 && above_c + cum2 >= want);
    const int L2 = hit2 ? static_cast<int>(__ffsll(static_cast<long long>(hit2))) - 1 : 31;
    *d = static_cast<uint32_t>(32 * cb + 31 - L2);
    *above = above_c + __shfl(cum2, L2, kWave) - __shfl(fv, L2, kWave);
}

// Calls f(key, ok) for the keys of x[lo, hi), a range that the block reads
// as a whole: 128-bit non-temporal loads (R per thread in flight, all issued
// before any is used) over the 16-byte aligned body, one element per thread
// for the head and tail.  ok is false for the padding a thread's last loads
// read past the body; f must do nothing then.  Order is not index order.
template <int R, class F>
__device__ __forceinline__ void for_keys(const float* __restrict__ x, int64_t lo, int64_t hi, F&& f) {
    const int t = threadIdx.x;
    const int64_t a = min(hi, (lo + 3) & ~static_cast<int64_t>(3));
    const int64_t b = max(a, hi & ~static_cast<int64_t>(3));
    if (t < a - lo) f(key_of(x[lo + t]), true);
    if (t < hi - b) f(key_of(x[b + t]), true);
    const f4* __restrict__ x4 = reinterpret_cast<const f4*>(x + a);
    const int64_t nv = (b - a) >> 2;
    for (int64_t v0 = 0; v0 < nv; v0 += static_cast<int64_t>(kBlock) * R) {
        f4 w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) w[r] = __builtin_nontemporal_load(x4 + min(v0 + r * kBlock + t, nv - 1));
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool ok = v0 + r * kBlock + t < nv;
            f(key_of(w[r].x), ok);
            f(key_of(w[r].y), ok);
            f(key_of(w[r].z), ok);
            f(key_of(w[r].w), ok);
        }
    }
}
#ifndef EFG_RAW_LOADS
#define EFG_RAW_LOADS 6
#endif
constexpr int kRawLoads = EFG_RAW_LOADS;  // 128-bit loads per thread in flight in the passes over x

// 3. compaction, one block per group of kGroup regions (compact_split blocks
//    per group for tensors with many expected candidates, each taking a slice
//    of the group's regions).  Every block first sums its tensor's group
//    counts: the candidates before its group give its dense offset, their
//    total decides the path (the tensor's first block records both).
//    Candidate path: the group's slots -> the dense index-ordered list, plus
//    the first radix histogram (top 11 key bits).  An overflowed region then
//    gets one wave of the block, which reads e again past the region's last
//    stored index (eight 64-element rows in flight per lane) and appends the
//    rest of its candidates in index order at the dense places the copy left
//    free; like the stream for stored ones, it clears e where the key is >=
//    thi, so that every entry of the dense list obeys the rule k_write relies
//    on.  Exact fallback: the block's elements are read for the first radix
//    histogram of the full pass, and then x is put back where the stream
//    cleared it (those reads saw +0: the histogram moves each such element
//    from bin 0 to its own bin).
constexpr int kCompactItems = 8;
constexpr int kRecollectRows = 8;
__global__ __launch_bounds__(kBlock) void k_compact(const SegPlan* __restrict__ plan, int32_t nseg,
                                                    const int32_t* __restrict__ cbb, const int32_t* __restrict__ gbb,
                                                    const int32_t* __restrict__ rb, SegState* __restrict__ st,
                                                    const uint32_t* __restrict__ grp_cnt,
                                                    const uint32_t* __restrict__ region_cnt,
                                                    const uint2* __restrict__ cpair, float* __restrict__ dval,
                                                    int32_t* __restrict__ didx, uint32_t* __restrict__ rhist,
                                                    int32_t hcopies, float* __restrict__ e,
                                                    uint32_t* __restrict__ stray, uint32_t force_fallback) {
    __shared__ uint32_t loff[kGroup];
    __shared__ uint32_t h[kRadixBins];
    __shared__ uint32_t hs[kSpec][1024];  // exact fallback: second-digit histograms of the guessed first digits
    __shared__ uint32_t lds[kWavesPerBlock + 1];
    __shared__ uint32_t red[2][kWavesPerBlock];
    const int b = blockIdx.x;
    const int s = upper_index_wave(cbb, nseg, b);
    const SegPlan& P = plan[s];
    const int split = P.compact_split;
    const int lb = b - cbb[s];
    const int gl = lb / split, part = lb % split;
    const int t = threadIdx.x;
    // the tensor's candidates before this group, and in all
    uint32_t before = 0, total = 0;
    for (int g = t; g < P.ngroups; g += kBlock) {
        const uint32_t c = grp_cnt[gbb[s] + g];
        total += c;
        before += g < gl ? c : 0u;
    }
    before = wave_sum(before);
    total = wave_sum(total);
    if (lane() == 0) {
        red[0][t / kWave] = before;
        red[1][t / kWave] = total;
    }
    for (int i = t; i < kRadixBins; i += kBlock) h[i] = 0;
    __syncthreads();
    before = 0;
    total = 0;
    for (int i = 0; i < kWavesPerBlock; ++i) {
        before += red[0][i];
        total += red[1][i];
    }
    const int64_t capacity = static_cast<int64_t>(P.nregions) * P.cap;
    const bool fb = force_fallback || P.direct || static_cast<int64_t>(total) > capacity ||
                    static_cast<int64_t>(total) < P.k;
    if (t == 0 && lb == 0) {
        st[s].fallback = fb ? 1u : 0u;
        st[s].ncand = total;
    }
    const int64_t r0 = rb[s] + static_cast<int64_t>(gl) * kGroup;  // first region (global)
    const int nr = min(kGroup, P.nregions - gl * kGroup);
    const int slice = kGroup / split;
    const int rs = part * slice;  // this block's regions [rs, re)
    const int re = min(nr, rs + slice);
    if (rs >= re) return;
    const int64_t cap = P.cap;
    const uint32_t spec_lo = st[s].spec_lo, spec_n = st[s].spec_n;
    if (fb) {
        // the first radix histogram of x over the block's elements [a, z),
        // and the second-digit ones of the guessed first digits; e reads +0
        // where the stream cleared a stored candidate
        for (int i = t; i < kSpec * 1024; i += kBlock) hs[i / 1024][i % 1024] = 0;
        __syncthreads();
        const int64_t a = P.off + (static_cast<int64_t>(gl) * kGroup + rs) * kRegion;
        const int64_t z = P.off + min((static_cast<int64_t>(gl) * kGroup + re) * kRegion, P.n);
        for_keys<kRawLoads>(e, a, z, [&](uint32_t key, bool ok) {
            if (!ok) return;
            atomicAdd(&h[key >> 20], 1u);
            const uint32_t j = (key >> 20) - spec_lo;
            if (j < spec_n) atomicAdd(&hs[j][(key >> 10) & 1023u], 1u);
        });
        __syncthreads();  // every read of e is done before x is put back
        const uint32_t thi = st[s].thi;
        const int64_t lo = P.off, hi = P.off + P.n;
        for (int r = rs + t / kWave; r < re; r += kWavesPerBlock) {
            const uint32_t cnt = min(region_cnt[r0 + r], static_cast<uint32_t>(cap));
            const int64_t slot = P.cand_base + (r0 + r - rb[s]) * cap;
            for (uint32_t j = lane(); j < cnt; j += kWave) {
                const uint2 pr = cpair[slot + j];
                const float v = __uint_as_float(pr.x);
                const uint32_t key = key_of(v);
                // indices were written by the stream of this call; the range check
                // keeps a workspace overwritten meanwhile from becoming a stray
                // write, and counts it
                if (key >= thi) {
                    if (pr.y >= lo && pr.y < hi) {
                        e[pr.y] = v;
                        atomicSub(&h[0], 1u);
                        atomicAdd(&h[key >> 20], 1u);
                        if (spec_lo == 0 && spec_n > 0) atomicSub(&hs[0][0], 1u);
                        const uint32_t j = (key >> 20) - spec_lo;
                        if (j < spec_n) atomicAdd(&hs[j][(key >> 10) & 1023u], 1u);
                    } else {
                        atomicAdd(stray, 1u);
                    }
                }
            }
        }
    } else {
        const uint32_t c = t < nr ? region_cnt[r0 + t] : 0u;
        uint32_t tot;
        const uint32_t ex = block_excl_scan<kBlock>(c, lds, &tot);
        loff[t] = ex;
        __syncthreads();
        const uint32_t q0 = loff[rs], q1 = re < nr ? loff[re] : tot;
        const int64_t dbase = P.cand_base + before;
        const int64_t slot0 = P.cand_base + (r0 - rb[s]) * cap;
        // kCompactItems entries per thread in flight: an entry past the block's
        // range or past its region's slot (written below) reads the group's
        // first slot instead and is not used
        for (uint32_t qb = q0; qb < q1; qb += kBlock * kCompactItems) {
            uint2 pr[kCompactItems];
            bool ok[kCompactItems];
#pragma unroll
            for (int u = 0; u < kCompactItems; ++u) {
                const uint32_t q = qb + u * kBlock + t;
                int64_t src = slot0;
                ok[u] = q < q1;
                if (ok[u]) {
                    const int r = rs + upper_index(loff + rs, re - rs, q);
                    ok[u] = q - loff[r] < cap;
                    if (ok[u]) src = slot0 + r * cap + (q - loff[r]);
                }
                pr[u] = cpair[src];
            }
#pragma unroll
            for (int u = 0; u < kCompactItems; ++u) {
                if (!ok[u]) continue;
                const uint32_t q = qb + u * kBlock + t;
                const float v = __uint_as_float(pr[u].x);
                dval[dbase + q] = v;
                didx[dbase + q] = static_cast<int32_t>(pr[u].y);
                atomicAdd(&h[key_of(v) >> 20], 1u);
            }
        }
        // overflowed regions, one wave each (none in the common case)
        const uint32_t tlo = st[s].tlo, thi = st[s].thi;
        const int l = lane();
        for (int r = rs + t / kWave; r < re; r += kWavesPerBlock) {
            const uint32_t cnt = region_cnt[r0 + r];
            if (cnt <= cap) continue;
            const int64_t rl = static_cast<int64_t>(gl) * kGroup + r;  // region within the tensor
            const int64_t gend = P.off + min(rl * kRegion + kRegion, P.n);
            const int64_t last = cpair[slot0 + r * cap + cap - 1].y;  // index of the last stored candidate
            const int64_t base = dbase + loff[r];
            uint32_t pos = static_cast<uint32_t>(cap);  // next entry of this region
            for (int64_t i0 = last + 1; i0 < gend && pos < cnt; i0 += kWave * kRecollectRows) {
                float x[kRecollectRows];
#pragma unroll
                for (int u = 0; u < kRecollectRows; ++u) {
                    const int64_t i = i0 + u * kWave + l;
                    x[u] = i < gend ? e[i] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < kRecollectRows; ++u) {
                    const int64_t i = i0 + u * kWave + l;
                    const uint32_t key = key_of(x[u]);
                    const bool hit = i < gend && key >= tlo;
                    const uint64_t bal = __ballot(hit);
                    const uint32_t p = pos + count_below(bal);
                    if (hit && p < cnt) {
                        dval[base + p] = x[u];
                        didx[base + p] = static_cast<int32_t>(i);
                        atomicAdd(&h[key >> 20], 1u);
                        if (key >= thi) e[i] = 0.0f;
                    }
                    pos += popc64(bal);
                }
            }
        }
    }
    flush_hist(h, kRadixBins, radix_hist(rhist, 0, s, b % hcopies, nseg, hcopies));
    if (fb)
        for (uint32_t j = 0; j < spec_n; ++j)
            flush_hist(hs[j], 1024, radix_hist(rhist, 3 + static_cast<int>(j), s, b % hcopies, nseg, hcopies));
}

// Radix digit of `key` in pass p (11, 10, 10 bits from the top) and whether the
// key matches the digits already fixed.
__device__ __forceinline__ bool radix_digit(int pass, uint32_t key, uint32_t prefix, uint32_t* d) {
    if (pass == 0) {
        *d = key >> 20;
        return true;
    }
    if (pass == 1) {
        *d = (key >> 10) & 1023u;
        return (key >> 20) == prefix;
    }
    *d = key & 1023u;
    return (key >> 10) == prefix;
}

// The select / emit blocks: each tensor that selects owns blocks
// [hb[s], hb[s+1]) (static) and shares out the tensor's work units among
// them, which depend on the path the compaction chose: the dense candidate
// list in units of kChunk entries, or x itself (in e) in units of kRawChunk
// elements, each taken as kRawSub chunks of kChunk.  The histogram blocks
// stride over the units; the count and write blocks take contiguous ranges
// [u0, u1) (block lb: units lb * U / nb .. (lb + 1) * U / nb, rounded up, so
// the first block's range is never empty), which makes a block's place in
// the output the counts of the blocks before it.  Per-unit statistics sit
// at the tensor's static bases (cunit_base, runit_base).
struct SelBlock {
    int s;
    int lb, nb;      // this block among the tensor's blocks
    bool raw;        // exact fallback: units of x
    uint32_t units;
    uint32_t u0, u1;  // this block's contiguous range of units
};

__device__ __forceinline__ SelBlock sel_block(const SegPlan* plan, int32_t nseg, const int32_t* hb,
                                              const SegState* st) {
    SelBlock sb;
    sb.s = upper_index_wave(hb, nseg, static_cast<int32_t>(blockIdx.x));
    sb.lb = static_cast<int>(blockIdx.x) - hb[sb.s];
    sb.nb = hb[sb.s + 1] - hb[sb.s];
    sb.raw = st[sb.s].fallback != 0;
    sb.units = sb.raw ? static_cast<uint32_t>(plan[sb.s].raw_units)
                      : (st[sb.s].ncand + kChunk - 1) / kChunk;
    const uint64_t U = sb.units, nb = static_cast<uint64_t>(sb.nb);
    sb.u0 = static_cast<uint32_t>((U * static_cast<uint64_t>(sb.lb) + nb - 1) / nb);
    sb.u1 = static_cast<uint32_t>((U * static_cast<uint64_t>(sb.lb + 1) + nb - 1) / nb);
    return sb;
}

// One kChunk piece of a unit: chunk j (0 .. kRawSub - 1) of raw unit u, or
// candidate unit u (j = 0).
struct Chunk {
    const float* v;      // values
    const int32_t* id;   // indices (candidate units)
    int64_t idx_base;    // first index (raw chunks)
    uint32_t cnt;        // entries (0: nothing left in this raw unit)
};

__device__ __forceinline__ Chunk chunk_of(const SegPlan& P, const SegState& S, bool raw, uint32_t u, int j,
                                          const float* dval, const int32_t* didx, const float* e) {
    Chunk c;
    if (!raw) {
        const int64_t base = P.cand_base + static_cast<int64_t>(u) * kChunk;
        c.v = dval + base;
        c.id = didx + base;
        c.idx_base = 0;
        c.cnt = min(static_cast<uint32_t>(kChunk), S.ncand - u * kChunk);
    } else {
        const int64_t lbeg = static_cast<int64_t>(u) * kRawChunk + static_cast<int64_t>(j) * kChunk;
        c.idx_base = P.off + lbeg;
        c.v = e + c.idx_base;
        c.id = nullptr;
        c.cnt = lbeg < P.n ? static_cast<uint32_t>(min(static_cast<int64_t>(kChunk), P.n - lbeg)) : 0u;
    }
    return c;
}

// A chunk's entries as the select and emit kernels read them: wave w of the
// block takes entries [w R 64, (w + 1) R 64), R = kChunk / kBlock rows of 64,
// lane l entry w R 64 + 64 i + l in row i, so every row is one coalesced load.
// All R loads are issued before any is used: an entry past the chunk's end
// (cnt >= 1) reads the chunk's last entry instead and is marked absent.
constexpr int kRows = kChunk / kBlock;
__device__ __forceinline__ uint32_t load_rows(const Chunk& c, float (&v)[kRows]) {
    const uint32_t j0 = static_cast<uint32_t>(threadIdx.x / kWave) * (kRows * kWave) + lane();
#pragma unroll
    for (int i = 0; i < kRows; ++i) v[i] = c.v[min(j0 + i * kWave, c.cnt - 1)];
    return j0;
}

// The digits fixed before pass `pass` (1, 2 or 3 = the count) of tensor s, as
// each select block finds them from the previous pass's histogram:
// pass 1: p0, w0 from the first histogram; pass 2: p1, w1 from the second and
// (p0, w0); pass 3: T, r from the third and (p1, w1).  The tensor's first
// block records them for the later kernels.
__device__ __forceinline__ void digits_before(int pass, int s, int lb, const SegPlan* plan, int32_t nseg,
                                              SegState* st, const uint32_t* rhist, int32_t hcopies,
                                              uint32_t* prefix, uint32_t* want, uint32_t* hint = nullptr) {
    uint32_t d, above;
    // the previous pass's histogram: after a hit, the guessed first digit's
    // second-digit histogram stands in for the first select pass's
    const int slot = (pass == 2 && st[s].hit) ? 2 + static_cast<int>(st[s].hit) : pass - 1;
    const uint32_t* gh = radix_hist(const_cast<uint32_t*>(rhist), slot, s, 0, nseg, hcopies);
    if (pass == 1) {
        const uint32_t k = static_cast<uint32_t>(plan[s].k);
        wave_find_digit(gh, hcopies, 2048, k, &d, &above);
        *prefix = d;
        *want = k - above;
        if (lb == 0 && threadIdx.x == 0) {
            st[s].p0 = *prefix;
            st[s].w0 = *want;
        }
    } else if (pass == 2) {
        const uint32_t p0 = st[s].p0, w0 = st[s].w0;
        wave_find_digit(gh, hcopies, 1024, w0, &d, &above);
        *prefix = (p0 << 10) | d;
        *want = w0 - above;
        if (lb == 0 && threadIdx.x == 0) {
            st[s].p1 = *prefix;
            st[s].w1 = *want;
        }
    } else {
        const uint32_t p1 = st[s].p1, w1 = st[s].w1;
        wave_find_digit(gh, hcopies, 1024, w1, &d, &above);
        *prefix = (p1 << 10) | d;  // T
        *want = w1 - above;        // r
        if (lb == 0 && threadIdx.x == 0) {
            st[s].T = *prefix;
            st[s].r = *want;
            if (hint) hint[s] = *prefix;  // the next call's fine sample window
        }
    }
}


// The exact fallback's ordered passes over x (in e) take a block's range of
// raw units in chunks of kWChunk elements: wave w takes rows w kWRows ..
// (w + 1) kWRows - 1 of 256 elements, lane l elements 4l .. 4l + 3 of a row
// (one 128-bit load when the tensor starts 16-byte aligned, else four scalar
// loads), so entries are ordered (chunk, wave, row, lane, element).
constexpr int kWRows = 2;                     // rows of 256 elements per wave and chunk
constexpr int kWChunk = kBlock * 4 * kWRows;  // 4096 elements
static_assert(kRawChunk % kWChunk == 0, "raw units are whole write chunks");

// The segment of the tensor's dense list that exact-fallback select block lb
// (of nb) collects its possible survivors into: the dense list, sized for the
// candidate slots, is otherwise unused on that path.  0 entries for a tensor
// with no candidate slots (a dense selection).
__device__ __forceinline__ uint32_t seg_cap(const SegPlan& P, int nb) {
    return static_cast<uint32_t>(min(static_cast<int64_t>(P.nregions) * P.cap / nb, static_cast<int64_t>(0x7fffffff)));
}

// Exact fallback, last select pass over x: in the same ordered read, the
// histogram of the last digit of the keys whose top 21 bits equal the pass's
// prefix p1 (LDS h), the count of keys above it (*above, per thread), and the
// keys that can be kept (top 21 bits >= p1) appended in index order to the
// block's segment sv / si (the first segcap of them).  Returns how many such
// keys the range holds (also past segcap).  Every thread of the block calls
// it; wcnt needs 2 * kWavesPerBlock words.
__device__ uint32_t collect_raw(const SegPlan& P, const SelBlock& sb, uint32_t p1, const float* __restrict__ e,
                                float* __restrict__ sv, int32_t* __restrict__ si, uint32_t segcap, uint32_t* h,
                                uint32_t* above, uint32_t* wcnt) {
    const int wv = threadIdx.x / kWave;
    const int l = lane();
    const bool al = (P.off & 3) == 0;
    const int64_t lo = P.off + static_cast<int64_t>(sb.u0) * kRawChunk;
    const int64_t end = min(P.off + static_cast<int64_t>(sb.u1) * kRawChunk, P.off + P.n);
    const int wo = wv * (kWRows * 256) + 4 * l;  // lane's first offset in the chunk, row 0
    auto load_chunk = [&](int64_t c0, float (&x)[kWRows][4]) {
        const int rem = static_cast<int>(min(end - c0, static_cast<int64_t>(kWChunk)));
        const float* ec = e + c0;
#pragma unroll
        for (int i = 0; i < kWRows; ++i) {
            const int o = wo + i * 256;
            if (al && o + 3 < rem) {
                const f4 q = __builtin_nontemporal_load(reinterpret_cast<const f4*>(ec + o));
                x[i][0] = q.x;
                x[i][1] = q.y;
                x[i][2] = q.z;
                x[i][3] = q.w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) x[i][c] = o + c < rem ? ec[o + c] : 0.0f;
            }
        }
    };
    uint32_t before = 0;  // collected in the earlier chunks (block-uniform)
    uint32_t ab = 0;
    float xn[kWRows][4];
    if (lo < end) load_chunk(lo, xn);
    int par = 0;  // wcnt half of this chunk: a wave may write the next chunk's half while another reads this one
    for (int64_t c0 = lo; c0 < end; c0 += kWChunk, par ^= 1) {
        const int rem = static_cast<int>(min(end - c0, static_cast<int64_t>(kWChunk)));
        float x[kWRows][4];
#pragma unroll
        for (int i = 0; i < kWRows; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) x[i][c] = xn[i][c];
        if (c0 + kWChunk < end) load_chunk(c0 + kWChunk, xn);
        uint64_t bal[kWRows][4];
        uint32_t n = 0;
#pragma unroll
        for (int i = 0; i < kWRows; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool ok = wo + i * 256 + c < rem;
                const uint32_t key = key_of(x[i][c]);
                const uint32_t top = key >> 10;
                if (ok && top == p1) atomicAdd(&h[key & 1023u], 1u);
                ab += (ok && top > p1) ? 1u : 0u;
                bal[i][c] = __ballot(ok && top >= p1);
                n += popc64(bal[i][c]);
            }
        uint32_t* wc = wcnt + par * kWavesPerBlock;
        if (l == 0) wc[wv] = n;
        __syncthreads();
        uint32_t base = before;
        for (int i = 0; i < kWavesPerBlock; ++i) {
            if (i < wv) base += wc[i];
            before += wc[i];
        }
#pragma unroll
        for (int i = 0; i < kWRows; ++i) {
            const uint64_t any = bal[i][0] | bal[i][1] | bal[i][2] | bal[i][3];
            if (!any) continue;  // wave-uniform
            uint32_t pos = base;
#pragma unroll
            for (int c = 0; c < 4; ++c) pos += count_below(bal[i][c]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if ((bal[i][c] >> l) & 1u) {
                    if (pos < segcap) {
                        sv[pos] = x[i][c];
                        si[pos] = static_cast<int32_t>(c0 + wo + i * 256 + c);
                    }
                    ++pos;
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) base += popc64(bal[i][c]);
        }
    }
    *above = ab;
    return before;
}

// 5. radix histograms of passes 1 and 2 (pass 0 came with the compaction),
//    each block over its contiguous range of units (of x itself: one
//    element range).  Pass 2 also leaves, per block, the suffix sums of its
//    own histogram (bh, kBlockHistWords words each: word i counts the
//    block's keys whose top 21 bits are above the pass's prefix or equal to
//    it with a last digit >= i; word 1024 those above the prefix), so that
//    the write kernel finds any block's counts above T and at T with two
//    loads instead of reading its entries again.
// (eight waves per SIMD: all 2048 select blocks of a call run at once)
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(8))) void k_hist(int pass, const SegPlan* __restrict__ plan, int32_t nseg,
                                                 const int32_t* __restrict__ hb, SegState* __restrict__ st,
                                                 const float* __restrict__ dval, const float* __restrict__ e,
                                                 uint32_t* __restrict__ rhist, int32_t hcopies,
                                                 uint32_t* __restrict__ bh, int32_t collect,
                                                 float* __restrict__ seg_v, int32_t* __restrict__ seg_i) {
    __shared__ uint32_t h[1024];
    __shared__ uint32_t s_above[kWavesPerBlock];
    __shared__ uint32_t s_scan[kWavesPerBlock + 1];
    __shared__ uint32_t s_wcnt[2 * kWavesPerBlock];
    const SelBlock sb = sel_block(plan, nseg, hb, st);
    if (sb.u0 >= sb.u1) return;  // never the tensor's first block, which records the digits
    uint32_t prefix, want;
    digits_before(pass, sb.s, sb.lb, plan, nseg, st, rhist, hcopies, &prefix, &want);
    if (pass == 1 && sb.raw && prefix - st[sb.s].spec_lo < st[sb.s].spec_n) {
        // exact fallback, first digit guessed right: the compaction built this pass's histogram
        if (sb.lb == 0 && threadIdx.x == 0) st[sb.s].hit = 1u + (prefix - st[sb.s].spec_lo);
        return;
    }
    for (int i = threadIdx.x; i < 1024; i += kBlock) h[i] = 0;
    __syncthreads();
    const SegPlan& P = plan[sb.s];
    const SegState& S = st[sb.s];
    uint32_t above = 0;  // pass 2: keys whose top 21 bits are above the prefix
    auto add = [&](uint32_t key, bool ok) {
        uint32_t d;
        if (ok && radix_digit(pass, key, prefix, &d)) atomicAdd(&h[d], 1u);
        if (pass == 2) above += (ok && (key >> 10) > prefix) ? 1u : 0u;
    };
    const uint32_t segcap = seg_cap(P, sb.nb);
    if (sb.raw && pass == 2 && collect && segcap > 0) {
        // exact fallback: the possible survivors of the block's range go to its
        // segment of the dense list, so the write need not read x again
        const int64_t seg = P.cand_base + static_cast<int64_t>(sb.lb) * segcap;
        (void)collect_raw(P, sb, prefix, e, seg_v + seg, seg_i + seg, segcap, h, &above, s_wcnt);
    } else if (sb.raw) {
        const int64_t lo = P.off + static_cast<int64_t>(sb.u0) * kRawChunk;
        const int64_t hi = P.off + min(static_cast<int64_t>(sb.u1) * kRawChunk, P.n);
        for_keys<kRawLoads>(e, lo, hi, add);
    } else {
        for (uint32_t u = sb.u0; u < sb.u1; ++u) {
            const Chunk c = chunk_of(P, S, false, u, 0, dval, nullptr, e);
            float v[kRows];
            const uint32_t j0 = load_rows(c, v);
#pragma unroll
            for (int i = 0; i < kRows; ++i) add(key_of(v[i]), j0 + i * kWave < c.cnt);
        }
    }
    flush_hist(h, 1024, radix_hist(rhist, pass, sb.s, blockIdx.x % hcopies, nseg, hcopies));
    if (pass == 2) {
        above = wave_sum(above);
        if (lane() == 0) s_above[threadIdx.x / kWave] = above;
        __syncthreads();
        uint32_t ab = 0;
        for (int i = 0; i < kWavesPerBlock; ++i) ab += s_above[i];
        // thread t owns bins 4t .. 4t + 3; the bins above them sum to the
        // block total less the threads up to t
        static_assert(1024 == 4 * kBlock, "pass-2 suffix sums: four bins per thread");
        const int t4 = 4 * static_cast<int>(threadIdx.x);
        const uint32_t b0 = h[t4], b1 = h[t4 + 1], b2 = h[t4 + 2], b3 = h[t4 + 3];
        const uint32_t mine4 = b0 + b1 + b2 + b3;
        uint32_t tot;
        const uint32_t before = block_excl_scan<kBlock>(mine4, s_scan, &tot);
        uint32_t* mine = bh + static_cast<size_t>(blockIdx.x) * kBlockHistWords;
        const uint32_t s3 = ab + (tot - before - mine4) + b3;
        mine[t4 + 3] = s3;
        mine[t4 + 2] = s3 + b2;
        mine[t4 + 1] = s3 + b2 + b1;
        mine[t4] = s3 + b2 + b1 + b0;
        if (threadIdx.x == 0) mine[1024] = ab;
    }
}

// The exact fallback's write over x (in e) for one block's range of raw
// units, in chunks of kWChunk elements: wave w takes rows w kWRows ..
// (w + 1) kWRows - 1 of 256 elements, lane l elements 4l .. 4l + 3 of a row
// (one 128-bit load when the tensor starts 16-byte aligned, else four
// scalar loads).  Entries are thus ordered (wave, row, lane, element): an
// entry's place counts the block's entries before the chunk, the chunk's
// earlier waves (LDS exchange), the wave's earlier rows, the row's lower
// lanes (one ballot per element position) and the lane's earlier elements.
// A first sweep counts with ballots and marks the rows that hold any key >=
// T; only those are placed (every row, when the statistics need each
// entry's fate).  Kept entries get e = +0; nothing else changes (thi plays
// no part: the compaction put x back everywhere).

template <bool STATS>
__device__ __forceinline__ void write_raw(const SegPlan& P, const SelBlock& sb, uint32_t T, uint32_t r,
                                          uint32_t gtu, uint32_t equ, uint32_t* wgt, uint32_t* weq,
                                          double2* lsum, float* __restrict__ e, float* __restrict__ vals,
                                          int32_t* __restrict__ idx, double2* __restrict__ part) {
    const int wv = threadIdx.x / kWave;
    const int l = lane();
    const bool al = (P.off & 3) == 0;
    const int64_t lo = P.off + static_cast<int64_t>(sb.u0) * kRawChunk;
    const int64_t end = min(P.off + static_cast<int64_t>(sb.u1) * kRawChunk, P.off + P.n);
    const int wo = wv * (kWRows * 256) + 4 * l;  // lane's first offset in the chunk, row 0
    double sent = 0.0, drop = 0.0;
    // the lane's entries of the chunk at c0 (+0 past the range)
    auto load_chunk = [&](int64_t c0, float (&x)[kWRows][4]) {
        const int rem = static_cast<int>(min(end - c0, static_cast<int64_t>(kWChunk)));
        const float* ec = e + c0;
#pragma unroll
        for (int i = 0; i < kWRows; ++i) {
            const int o = wo + i * 256;
            if (al && o + 3 < rem) {
                const f4 q = __builtin_nontemporal_load(reinterpret_cast<const f4*>(ec + o));
                x[i][0] = q.x;
                x[i][1] = q.y;
                x[i][2] = q.z;
                x[i][3] = q.w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) x[i][c] = o + c < rem ? ec[o + c] : 0.0f;
            }
        }
    };
    // each chunk's loads are issued before the chunk before it is swept and
    // placed, so they are in flight across its two barriers
    float xn[kWRows][4];
    if (lo < end) load_chunk(lo, xn);
    for (int64_t c0 = lo; c0 < end; c0 += kWChunk) {
        const int rem = static_cast<int>(min(end - c0, static_cast<int64_t>(kWChunk)));  // entries in the chunk
        float* ec = e + c0;
        float x[kWRows][4];
#pragma unroll
        for (int i = 0; i < kWRows; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) x[i][c] = xn[i][c];
        if (c0 + kWChunk < end) load_chunk(c0 + kWChunk, xn);
        // sweep 1: the wave's counts, and its rows holding a key >= T
        uint32_t ngt = 0, neq = 0;
        uint32_t rows = 0;  // bit i: row i holds a key >= T (wave-uniform)
#pragma unroll
        for (int i = 0; i < kWRows; ++i) {
            uint64_t any = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool ok = wo + i * 256 + c < rem;
                const uint32_t key = key_of(x[i][c]);
                const uint64_t bg = __ballot(ok && key > T), be = __ballot(ok && key == T);
                ngt += popc64(bg);
                neq += popc64(be);
                any |= bg | be;
            }
            rows |= any ? (1u << i) : 0u;
        }
        if (l == 0) {
            wgt[wv] = ngt;
            weq[wv] = neq;
        }
        __syncthreads();
        uint32_t gtb = gtu, eqb = equ;
        for (int i = 0; i < kWavesPerBlock; ++i) {
            if (i < wv) {
                gtb += wgt[i];
                eqb += weq[i];
            }
            gtu += wgt[i];
            equ += weq[i];
        }
        __syncthreads();  // wgt / weq are rewritten by the next chunk
        // sweep 2: places
#pragma unroll
        for (int i = 0; i < kWRows; ++i) {
            if (!STATS && !(rows & (1u << i))) continue;
            const int o = wo + i * 256;
            uint32_t gb = gtb, eb = eqb;  // the row's entries before this lane's first
            uint32_t tg = 0, te = 0;      // the row's totals
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool ok = o + c < rem;
                const uint32_t key = key_of(x[i][c]);
                const uint64_t bg = __ballot(ok && key > T), be = __ballot(ok && key == T);
                gb += count_below(bg);
                eb += count_below(be);
                tg += popc64(bg);
                te += popc64(be);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool ok = o + c < rem;
                const uint32_t key = key_of(x[i][c]);
                const bool gt = ok && key > T, eq = ok && key == T;
                int64_t pos = -1;
                if (gt) pos = static_cast<int64_t>(gb) + min(r, eb);
                else if (eq && eb < r) pos = static_cast<int64_t>(gb) + eb;
                gb += gt ? 1u : 0u;
                eb += eq ? 1u : 0u;
                if (STATS && ok) {
                    if (pos >= 0) sent += sq_finite(x[i][c], key);
                    else drop += sq_finite(x[i][c], key);
                }
                if (pos >= 0 && pos < P.k) {
                    vals[P.out_off + pos] = x[i][c];
                    idx[P.out_off + pos] = static_cast<int32_t>(c0 + o + c);
                    ec[o + c] = 0.0f;
                }
            }
            gtb += tg;
            eqb += te;
        }
        // a unit ends with this chunk: its partial, a fixed-order block sum
        if (STATS && ((c0 + kWChunk - lo) % kRawChunk == 0 || c0 + kWChunk >= end)) {
            sent = wave_sum(sent);
            drop = wave_sum(drop);
            if (l == 0) lsum[wv] = make_double2(sent, drop);
            __syncthreads();
            if (threadIdx.x == 0) {
                double2 t = make_double2(0.0, 0.0);
                for (int i = 0; i < kWavesPerBlock; ++i) {
                    t.x += lsum[i].x;
                    t.y += lsum[i].y;
                }
                part[sb.u0 + static_cast<uint32_t>((c0 - lo) / kRawChunk)] = t;
            }
            __syncthreads();
            sent = 0.0;
            drop = 0.0;
        }
    }
}

// 6. the kept entries at their index-ordered places, each chunk read in rows
//    as load_rows lays them out, so loads and (mostly kept-together) stores
//    coalesce.  Every block first finds T and r from the last histogram (the
//    tensor's first block records them, and T as the next call's hint).  An
//    entry's place is (entries with key > T before it) + min(r, entries with
//    key == T before it): the totals of the tensor's earlier blocks (two words
//    of each one's pass-2 suffix sums), those of the block's earlier chunks,
//    of its earlier waves, of the wave's earlier rows, and of the row's lower
//    lanes (ballots).  Kept entries get e = +0 unless the stream cleared them
//    (key >= thi); dropped ones the stream cleared get x back.
template <bool STATS>
__global__ __launch_bounds__(kBlock) void k_write(const SegPlan* __restrict__ plan, int32_t nseg,
                                                  const int32_t* __restrict__ hb, SegState* __restrict__ st,
                                                  const uint32_t* __restrict__ rhist, int32_t hcopies,
                                                  const uint32_t* __restrict__ bh, uint32_t* __restrict__ hint,
                                                  const float* __restrict__ dval, const int32_t* __restrict__ didx,
                                                  float* __restrict__ e, float* __restrict__ vals,
                                                  int32_t* __restrict__ idx, double2* __restrict__ cpart,
                                                  double2* __restrict__ rpart, uint32_t* __restrict__ stray) {
    __shared__ uint32_t wgt[kWavesPerBlock], weq[kWavesPerBlock];
    __shared__ double2 lsum[kWavesPerBlock];
    const SelBlock sb = sel_block(plan, nseg, hb, st);
    if (sb.u0 >= sb.u1) return;  // never the tensor's first block, which records T and r
    const int wv = threadIdx.x / kWave;
    const int l = lane();
    uint32_t T, r;
    digits_before(3, sb.s, sb.lb, plan, nseg, st, rhist, hcopies, &T, &r, hint);
    const uint32_t d = T & 1023u;
    // counts before the block's range: the tensor's earlier blocks' keys
    // above T (suffix word d + 1) and at T (word d less word d + 1); a block
    // with no units ran no pass 2 and counts nothing
    uint32_t gtu = 0, equ = 0;
    const uint64_t U = sb.units, nbk = static_cast<uint64_t>(sb.nb);
    for (int b = hb[sb.s] + static_cast<int>(threadIdx.x); b < static_cast<int>(blockIdx.x); b += kBlock) {
        const uint64_t lb = static_cast<uint64_t>(b - hb[sb.s]);
        if ((U * lb + nbk - 1) / nbk >= (U * (lb + 1) + nbk - 1) / nbk) continue;
        const uint32_t* m = bh + static_cast<size_t>(b) * kBlockHistWords;
        const uint32_t gt = m[d + 1], ge = m[d];
        gtu += gt;
        equ += ge - gt;
    }
    gtu = wave_sum(gtu);
    equ = wave_sum(equ);
    if (l == 0) {
        wgt[wv] = gtu;
        weq[wv] = equ;
    }
    __syncthreads();
    gtu = 0;
    equ = 0;
    for (int i = 0; i < kWavesPerBlock; ++i) {
        gtu += wgt[i];
        equ += weq[i];
    }
    __syncthreads();  // wgt / weq are rewritten by the first chunk
    const SegPlan& P = plan[sb.s];
    const SegState& S = st[sb.s];
    const uint32_t thi = sb.raw ? kNoKey : S.thi;
    const int64_t out_off = P.out_off, kseg = P.k;
    const int64_t seg_lo = P.off, seg_hi = P.off + P.n;
    double2* part = sb.raw ? (rpart ? rpart + P.runit_base : nullptr) : (cpart ? cpart + P.cunit_base : nullptr);
    // places one chunk of dense entries (values with their indices)
    auto place_chunk = [&](const Chunk& c, double& sent, double& drop) {
        float v[kRows];
        const uint32_t j0 = load_rows(c, v);
        int32_t ids[kRows];  // the entries' indices, loaded with the values
#pragma unroll
        for (int i = 0; i < kRows; ++i) ids[i] = c.id[min(j0 + i * kWave, c.cnt - 1)];
        // per row: the entries above T, equal to T, and with a key >= thi (a
        // dropped one of those gets x back); wave-uniform, kept for the
        // placing loop, which skips rows where all three are empty
        uint64_t bgs[kRows], bes[kRows], bhs[kRows];
        uint32_t ngt = 0, neq = 0;  // this wave's counts (wave-uniform)
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const bool ok = j0 + i * kWave < c.cnt;
            const uint32_t key = key_of(v[i]);
            bgs[i] = __ballot(ok && key > T);
            bes[i] = __ballot(ok && key == T);
            bhs[i] = __ballot(ok && key >= thi);
            ngt += popc64(bgs[i]);
            neq += popc64(bes[i]);
        }
        if (l == 0) {
            wgt[wv] = ngt;
            weq[wv] = neq;
        }
        __syncthreads();
        uint32_t gtb = gtu, eqb = equ;
        for (int i = 0; i < kWavesPerBlock; ++i) {
            if (i < wv) {
                gtb += wgt[i];
                eqb += weq[i];
            }
            gtu += wgt[i];
            equ += weq[i];
        }
        __syncthreads();  // wgt / weq are rewritten by the next chunk
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const uint32_t jj = j0 + i * kWave;
            const bool ok = jj < c.cnt;
            const uint32_t key = key_of(v[i]);
            const uint64_t bg = bgs[i], be = bes[i];
            if (!STATS && (bg | be | bhs[i]) == 0) continue;  // nothing to place or restore in this row
            const bool gt = ok && key > T, eq = ok && key == T;
            const uint32_t g_before = gtb + count_below(bg), e_before = eqb + count_below(be);
            gtb += popc64(bg);
            eqb += popc64(be);
            if (!ok) continue;
            int64_t pos = -1;
            if (gt) pos = static_cast<int64_t>(g_before) + min(r, e_before);
            else if (eq && e_before < r) pos = static_cast<int64_t>(g_before) + e_before;
            if (STATS) {
                if (pos >= 0) sent += sq_finite(v[i], key);
                else drop += sq_finite(v[i], key);
            }
            const int64_t id = static_cast<int64_t>(ids[i]);
            if (id < seg_lo || id >= seg_hi) {  // only if the workspace was overwritten meanwhile
                atomicAdd(stray, 1u);
                continue;
            }
            if (pos >= 0 && pos < kseg) {
                vals[out_off + pos] = v[i];
                idx[out_off + pos] = static_cast<int32_t>(id);
                if (key < thi) e[id] = 0.0f;
            } else if (pos < 0 && key >= thi) {
                e[id] = v[i];
            }
        }
    };
    if (sb.raw) {
        // exact fallback: from the block's segment of the dense list when the
        // last select pass collected every possible survivor of its range
        // there (their count is word 0 of its suffix sums: the keys whose top
        // 21 bits are T's or above), else by a pass over x
        const uint32_t segcap = seg_cap(P, sb.nb);
        const uint32_t ncol = bh[static_cast<size_t>(blockIdx.x) * kBlockHistWords];
        if (!STATS && segcap > 0 && ncol <= segcap) {
            const int64_t seg = P.cand_base + static_cast<int64_t>(sb.lb) * segcap;
            double sent = 0.0, drop = 0.0;
            for (uint32_t q = 0; q < ncol; q += kChunk) {
                Chunk c;
                c.v = dval + seg + q;
                c.id = didx + seg + q;
                c.idx_base = 0;
                c.cnt = min(static_cast<uint32_t>(kChunk), ncol - q);
                place_chunk(c, sent, drop);
            }
            return;
        }
        write_raw<STATS>(P, sb, T, r, gtu, equ, wgt, weq, lsum, e, vals, idx, part);
        return;
    }
    for (uint32_t u = sb.u0; u < sb.u1; ++u) {  // gtu, equ: counts before the next chunk
        double sent = 0.0, drop = 0.0;
        place_chunk(chunk_of(P, S, false, u, 0, dval, didx, e), sent, drop);
        if (STATS) {
            // fixed-order block sum of the unit's sent and dropped energy
            sent = wave_sum(sent);
            drop = wave_sum(drop);
            if (l == 0) lsum[wv] = make_double2(sent, drop);
            __syncthreads();
            if (threadIdx.x == 0) {
                double2 t = make_double2(0.0, 0.0);
                for (int i = 0; i < kWavesPerBlock; ++i) {
                    t.x += lsum[i].x;
                    t.y += lsum[i].y;
                }
                part[u] = t;
            }
            __syncthreads();
        }
    }
}

// 7. per-tensor monitoring statistics {sent energy, residual energy} from the
// stream's and the emit's partials, summed in a fixed order.
__device__ __forceinline__ double2 block_sum2(double2 v, double2* lsum) {
    v.x = wave_sum(v.x);
    v.y = wave_sum(v.y);
    if (lane() == 0) lsum[threadIdx.x / kWave] = v;
    __syncthreads();
    double2 t = make_double2(0.0, 0.0);
    for (int i = 0; i < kWavesPerBlock; ++i) {
        t.x += lsum[i].x;
        t.y += lsum[i].y;
    }
    __syncthreads();
    return t;
}

// 7a. one block per group of kGroup regions: the group's stream partials
__global__ __launch_bounds__(kGroup) void k_stats_groups(const SegPlan* __restrict__ plan, int32_t nseg,
                                                         const int32_t* __restrict__ gbb,
                                                         const int32_t* __restrict__ rb,
                                                         const double2* __restrict__ spart,
                                                         double2* __restrict__ gpart) {
    __shared__ double2 lsum[kWavesPerBlock];
    const int gi = blockIdx.x;
    const int s = upper_index_wave(gbb, nseg, gi);
    const int gl = gi - gbb[s];
    const int64_t r = rb[s] + static_cast<int64_t>(gl) * kGroup + threadIdx.x;
    const bool ok = static_cast<int>(threadIdx.x) < plan[s].nregions - gl * kGroup;
    const double2 t = block_sum2(ok ? spart[r] : make_double2(0.0, 0.0), lsum);
    if (threadIdx.x == 0) gpart[gi] = t;
}

// 7b. per tensor
__global__ __launch_bounds__(kBlock) void k_stats(const SegPlan* __restrict__ plan, const SegState* __restrict__ st,
                                                  const int32_t* __restrict__ gbb,
                                                  const double2* __restrict__ gpart, const double2* __restrict__ cpart,
                                                  const double2* __restrict__ rpart, double* __restrict__ stats) {
    __shared__ double2 lsum[kWavesPerBlock];
    const int s = blockIdx.x;
    const int mode = plan[s].mode;
    const bool fb = mode == MODE_NORMAL && st[s].fallback;
    double2 a = make_double2(0.0, 0.0);
    if (!fb) {
        // the stream's groups (every element of a k = 0 or k = n tensor, the
        // non-candidates of a candidate-path tensor)
        for (int64_t gi = gbb[s] + threadIdx.x; gi < gbb[s + 1]; gi += kBlock) {
            a.x += gpart[gi].x;
            a.y += gpart[gi].y;
        }
    }
    if (mode == MODE_NORMAL) {
        const double2* p = fb ? rpart + plan[s].runit_base : cpart + plan[s].cunit_base;
        const int64_t nu = fb ? plan[s].raw_units : (st[s].ncand + kChunk - 1) / kChunk;
        for (int64_t q = threadIdx.x; q < nu; q += kBlock) {
            a.x += p[q].x;
            a.y += p[q].y;
        }
    }
    const double2 t = block_sum2(a, lsum);
    if (threadIdx.x == 0) {
        stats[2 * s] = t.x;
        stats[2 * s + 1] = t.y;
    }
}

__global__ void k_stats_zero(double* __restrict__ stats, int32_t n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) stats[i] = 0.0;
}

// ------------------------------------------------------------------ host driver
// The plan and prefix tables as the kernels read them at the start of the
// workspace (L.static_end bytes).
static void fill_words(const Plan& P, const Layout& L, uint32_t* words) {
    uint8_t* h = reinterpret_cast<uint8_t*>(words);
    memset(h, 0, L.static_end);
    memcpy(h + L.plan, P.seg.data(), P.seg.size() * sizeof(SegPlan));
    memcpy(h + L.rb, P.rb.data(), P.rb.size() * 4);
    memcpy(h + L.gbb, P.gbb.data(), P.gbb.size() * 4);
    memcpy(h + L.sbb, P.sbb.data(), P.sbb.size() * 4);
    memcpy(h + L.cbb, P.cbb.data(), P.cbb.size() * 4);
    memcpy(h + L.hb, P.hb.data(), P.hb.size() * 4);
}

static int check_ws(const Layout& L, const void* ws, size_t ws_bytes) {
    if (!ws) return fail(EF_EWS, "workspace is NULL (%zu bytes needed)", L.total);
    if (ws_bytes < L.total) return fail(EF_EWS, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
    if (!aligned256(ws)) return fail(EF_EINVAL, "workspace must be 256-byte aligned");
    return EF_OK;
}

// A plan's tables on the host (words) and, when they sit in pinned host
// memory, the address the device reads them at (words_dev).
struct Tables {
    const uint32_t* words;
    const uint4* words_dev;
};

static int run(const float* g, float* e, const Plan& P, const Layout& L, Tables tb, float* vals, int32_t* idx,
               void* ws, size_t ws_bytes, uint32_t* nonfinite, double* stats, uint32_t flags, hipStream_t s,
               bool* read_pinned = nullptr) {
    if (read_pinned) *read_pinned = false;
    WordChunk none;
    none.n = 0;
    if (P.R == 0) {
        // nothing to stream: only the counter and the statistics need clearing
        if (nonfinite)
            EF_TRY(launch("topk_init", k_init, dim3(1), dim3(kBlock), s, static_cast<uint4*>(nullptr),
                          static_cast<int64_t>(0), nonfinite, static_cast<uint32_t*>(nullptr), none,
                          static_cast<const uint4*>(nullptr), static_cast<int64_t>(0)));
        if (stats && P.nseg > 0)
            EF_TRY(launch("topk_stats", k_stats_zero, dim3(1), dim3(kBlock), s, stats, 2 * P.nseg));
        return EF_OK;
    }
    EF_TRY(check_ws(L, ws, ws_bytes));
    uint8_t* W = static_cast<uint8_t*>(ws);
    auto at = [&](size_t o) { return W + o; };

    // The plan tables reach the workspace in k_init: a small plan (up to 11
    // tensors) in its kernel arguments, a larger one read by its blocks from
    // the plan cache's pinned host copy.  Under HIP graph capture a larger
    // plan goes in kernel-argument chunks of kWordChunk words instead, which
    // the graph keeps by value: a replay must not depend on a host buffer the
    // cache may reuse later.
    const size_t nwords = L.static_end / 4;
    WordChunk first;
    first.n = 0;
    const uint4* tsrc = nullptr;
    int64_t tvec = 0;
    if (nwords <= kWordChunk) {
        first.n = static_cast<uint32_t>(nwords);
        memcpy(first.w, tb.words, first.n * 4);
    } else {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess) return fail(EF_EHIP, "stream capture query failed");
        if (cs == hipStreamCaptureStatusActive || !tb.words_dev) {
            EF_TRY(upload_words(W, tb.words, nwords, s));
        } else {
            tsrc = tb.words_dev;
            tvec = static_cast<int64_t>(L.static_end / 16);
            if (read_pinned) *read_pinned = true;
        }
    }
    const int64_t nzero = static_cast<int64_t>((L.zero_end - L.state) / 16);
    const unsigned zgrid = static_cast<unsigned>(
        std::min<int64_t>(kMaxGrid, std::max<int64_t>({1, cdiv(nzero, kBlock), cdiv(tvec, kBlock)})));
    EF_TRY(launch("topk_init", k_init, dim3(zgrid), dim3(kBlock), s, reinterpret_cast<uint4*>(at(L.state)), nzero,
                  nonfinite, reinterpret_cast<uint32_t*>(W), first, tsrc, tvec));

    const SegPlan* plan = reinterpret_cast<const SegPlan*>(at(L.plan));
    const int32_t* rb = reinterpret_cast<const int32_t*>(at(L.rb));
    const int32_t* gbb = reinterpret_cast<const int32_t*>(at(L.gbb));
    const int32_t* sbb = reinterpret_cast<const int32_t*>(at(L.sbb));
    const int32_t* hb = reinterpret_cast<const int32_t*>(at(L.hb));
    uint32_t* stray = reinterpret_cast<uint32_t*>(at(L.status));
    SegState* st = reinterpret_cast<SegState*>(at(L.state));
    uint32_t* shist = reinterpret_cast<uint32_t*>(at(L.shist));
    uint32_t* hint = reinterpret_cast<uint32_t*>(at(L.hint));
    uint32_t* rhist = reinterpret_cast<uint32_t*>(at(L.rhist));
    uint32_t* grp_cnt = reinterpret_cast<uint32_t*>(at(L.grp_cnt));
    uint32_t* region_cnt = reinterpret_cast<uint32_t*>(at(L.region_cnt));
    uint2* cpair = reinterpret_cast<uint2*>(at(L.cpair));
    float* dval = reinterpret_cast<float*>(at(L.dval));
    int32_t* didx = reinterpret_cast<int32_t*>(at(L.didx));
    uint32_t* bh = reinterpret_cast<uint32_t*>(at(L.bh));
    double2* spart = reinterpret_cast<double2*>(at(L.spart));
    double2* cpart = stats ? reinterpret_cast<double2*>(at(L.cpart)) : nullptr;
    double2* rpart = stats ? reinterpret_cast<double2*>(at(L.rpart)) : nullptr;
    const int32_t nseg = P.nseg;
    double2* gpart = reinterpret_cast<double2*>(at(L.gpart));
    auto finish_stats = [&]() -> int {
        if (!stats) return EF_OK;
        EF_TRY(launch("topk_stats_groups", k_stats_groups, dim3(static_cast<unsigned>(P.G)), dim3(kGroup), s, plan,
                      nseg, gbb, rb, static_cast<const double2*>(spart), gpart));
        return launch("topk_stats", k_stats, dim3(static_cast<unsigned>(nseg)), dim3(kBlock), s, plan,
                      static_cast<const SegState*>(st), gbb, static_cast<const double2*>(gpart),
                      static_cast<const double2*>(reinterpret_cast<double2*>(at(L.cpart))),
                      static_cast<const double2*>(reinterpret_cast<double2*>(at(L.rpart))), stats);
    };

    // A call with few regions streams each with a block of kSplit waves, so
    // that a small call still puts several waves on every CU (the flat N = 1e6
    // call has 245 regions); those blocks read T_lo and T_hi off the sample
    // histogram themselves.
    const bool few = P.R < kFewRegions;
    // (such calls keep one copy of each histogram, which is all the split
    // stream's edge search reads)
    if (few && P.hcopies != 1) return fail(EF_EINVAL, "internal: split stream with %d histogram copies", P.hcopies);
    if (P.any_normal && P.SB > 0) {
        // the fine window is left out when the statistics are asked for: their
        // fixed-order sums run over a split of the elements that depends on
        // T_lo, which then depends on the call's inputs alone
        EF_TRY(launch("topk_sample_hist", k_sample, dim3(static_cast<unsigned>(P.SB)), dim3(kSampleBlock), s, g,
                      static_cast<const float*>(e), plan, nseg, sbb, P.sample_rounds, shist, P.hcopies,
                      static_cast<const uint32_t*>(hint), static_cast<int32_t>(stats ? 0 : 1)));
        if (!few)
            EF_TRY(launch("topk_sample_select", k_sample_select, dim3(static_cast<unsigned>(nseg)), dim3(kWave), s,
                          plan, static_cast<const uint32_t*>(shist), P.hcopies, static_cast<const uint32_t*>(hint),
                          st));
    }
    auto stream = [&](auto stats_on) -> int {
        constexpr bool ST = decltype(stats_on)::value;
        if (few)
            return launch("topk_stream", k_stream_split<ST, kSplit>, dim3(static_cast<unsigned>(P.R)),
                          dim3(kSplit * kWave), s, g, e, plan, nseg, rb, st, region_cnt, grp_cnt, cpair, vals, idx,
                          nonfinite, spart, static_cast<const uint32_t*>(shist), P.hcopies,
                          static_cast<const uint32_t*>(hint));
        return launch("topk_stream", k_stream<ST, kStreamWaves>, dim3(static_cast<unsigned>(cdiv(P.R, kStreamWaves))),
                      dim3(kStreamWaves * kWave), s, g, e, plan, nseg, rb, P.R, st, region_cnt, grp_cnt, cpair, vals,
                      idx, nonfinite, spart);
    };
    if (stats)
        EF_TRY(stream(std::true_type{}));
    else
        EF_TRY(stream(std::false_type{}));
    if (!P.any_normal) return finish_stats();

    EF_TRY(launch("topk_compact", k_compact, dim3(static_cast<unsigned>(P.CB)), dim3(kBlock), s, plan, nseg,
                  static_cast<const int32_t*>(reinterpret_cast<int32_t*>(at(L.cbb))), gbb, rb, st,
                  static_cast<const uint32_t*>(grp_cnt), static_cast<const uint32_t*>(region_cnt),
                  static_cast<const uint2*>(cpair), dval, didx, rhist, P.hcopies, e, stray,
                  static_cast<uint32_t>((flags & EF_FLAG_FORCE_FALLBACK) ? 1u : 0u)));
    const dim3 hgrid(static_cast<unsigned>(P.HB));
    for (int pass = 1; pass < 3; ++pass)
        EF_TRY(launch("topk_hist", k_hist, hgrid, dim3(kBlock), s, pass, plan, nseg, hb, st,
                      static_cast<const float*>(dval), static_cast<const float*>(e), rhist, P.hcopies, bh,
                      static_cast<int32_t>(stats ? 0 : 1), dval, didx));
    EF_TRY(launch("topk_write", stats ? k_write<true> : k_write<false>, hgrid, dim3(kBlock), s, plan, nseg, hb,
                  st, static_cast<const uint32_t*>(rhist), P.hcopies, static_cast<const uint32_t*>(bh), hint,
                  static_cast<const float*>(dval), static_cast<const int32_t*>(didx), e, vals, idx, cpart, rpart,
                  stray));
    return finish_stats();
}

static int check_common(const float* g, const float* e, int64_t total, int64_t ksum, const float* vals,
                        const int32_t* idx, uint32_t flags) {
    if (flags & ~EF_FLAG_FORCE_FALLBACK) return fail(EF_EINVAL, "unknown flags 0x%x", flags);
    if (total > 0 && (!g || !e)) return fail(EF_EINVAL, "g and e must not be NULL");
    if (total > 0 && (!aligned16(g) || !aligned16(e))) return fail(EF_EINVAL, "g and e must be 16-byte aligned");
    if (ksum > 0 && (!vals || !idx)) return fail(EF_EINVAL, "vals and idx must not be NULL when k > 0");
    return EF_OK;
}

// ------------------------------------------------------------------ plan cache
// A layer-wise call usually repeats the same tables step after step.  Its
// plan is built and checked once and kept, with its tables in pinned host
// memory that k_init reads straight into the workspace: a repeated call
// neither rebuilds the plan nor launches a separate copy, and the contents of
// the workspace on entry still do not matter.  A full cache reuses its least
// recently used entry, waiting first (the only host wait of a call) until
// the last call that read that entry's pinned tables has passed its k_init.
constexpr int kPlanCacheSize = 16;
struct CachedPlan {
    int32_t nseg = -1;  // -1: empty
    uint64_t hash = 0;
    std::vector<int64_t> off, ks;
    Plan plan;
    Layout L{};
    uint32_t* host = nullptr;  // pinned, L.static_end bytes used
    const uint4* dev = nullptr;  // the same memory as the device addresses it
    size_t cap = 0;
    hipEvent_t read_done = nullptr;  // recorded after the last k_init that read `host`
    bool filled = false;             // host holds this entry's tables
    bool pending = false;
    uint64_t stamp = 0;
};

namespace {
std::mutex g_cache_mu;
CachedPlan g_cache[kPlanCacheSize];
uint64_t g_cache_clock = 0;
}  // namespace

static uint64_t table_hash(int32_t nseg, const int64_t* off, const int64_t* ks) {
    uint64_t h = 1469598103934665603ull ^ static_cast<uint64_t>(static_cast<uint32_t>(nseg));
    auto mix = [&](int64_t v) {
        h ^= static_cast<uint64_t>(v);
        h *= 1099511628211ull;
    };
    for (int32_t i = 0; i <= nseg; ++i) mix(off[i]);
    for (int32_t i = 0; i < nseg; ++i) mix(ks[i]);
    return h;
}

// The cache entry for these tables, built on a miss (which also checks them).
// Called with g_cache_mu held; the entry stays valid while it is held.
static int cached_plan(int32_t nseg, const int64_t* off, const int64_t* ks, CachedPlan** out) {
    if (nseg < 0) return fail(EF_EINVAL, "nseg must be >= 0 (got %d)", nseg);
    if (nseg > 0 && (!off || !ks)) return fail(EF_EINVAL, "segment tables must not be NULL");
    const int64_t zero_off[1] = {0};
    if (nseg == 0 && !off) off = zero_off;
    const uint64_t h = table_hash(nseg, off, ks);
    CachedPlan* victim = nullptr;  // the first empty entry, else the least recently used one
    for (CachedPlan& c : g_cache) {
        if (c.nseg == nseg && c.hash == h && std::equal(c.off.begin(), c.off.end(), off) &&
            std::equal(c.ks.begin(), c.ks.end(), ks)) {
            c.stamp = ++g_cache_clock;
            *out = &c;
            return EF_OK;
        }
        if (c.nseg < 0) {
            if (!victim || victim->nseg >= 0) victim = &c;
        } else if (!victim || (victim->nseg >= 0 && c.stamp < victim->stamp)) {
            victim = &c;
        }
    }
    Plan p;
    EF_TRY(make_plan(nseg, off, ks, p));
    CachedPlan& c = *victim;
    if (c.pending) {
        // its pinned tables may still be read by a queued k_init
        if (hipEventSynchronize(c.read_done) != hipSuccess)
            return fail(EF_EHIP, "plan cache: wait for an evicted entry failed");
        c.pending = false;
    }
    c.nseg = -1;
    c.filled = false;
    c.L = make_layout(p);
    c.plan = std::move(p);
    c.off.assign(off, off + nseg + 1);
    c.ks.assign(ks, ks + nseg);
    c.hash = h;
    c.nseg = nseg;
    c.stamp = ++g_cache_clock;
    *out = &c;
    return EF_OK;
}

// The entry's tables in pinned host memory, written on its first use by a
// call (the size query needs no device and never gets here).
static int pinned_tables(CachedPlan& c) {
    if (c.filled) return EF_OK;
    const size_t bytes = c.L.static_end;
    if (c.cap < bytes) {
        if (c.host) (void)hipHostFree(c.host);
        c.host = nullptr;
        c.dev = nullptr;
        c.cap = 0;
        void* hp = nullptr;
        if (hipHostMalloc(&hp, bytes, hipHostMallocPortable | hipHostMallocMapped) != hipSuccess)
            return fail(EF_EHIP, "plan cache: pinned allocation of %zu bytes failed", bytes);
        void* dp = nullptr;
        if (hipHostGetDevicePointer(&dp, hp, 0) != hipSuccess) {
            (void)hipHostFree(hp);
            return fail(EF_EHIP, "plan cache: no device address for the pinned tables");
        }
        c.host = static_cast<uint32_t*>(hp);
        c.dev = static_cast<const uint4*>(dp);
        c.cap = bytes;
    }
    if (!c.read_done && hipEventCreateWithFlags(&c.read_done, hipEventDisableTiming) != hipSuccess)
        return fail(EF_EHIP, "plan cache: event creation failed");
    fill_words(c.plan, c.L, c.host);
    c.filled = true;
    return EF_OK;
}

// ------------------------------------------------------------------ allocation-free entry point
// The scratch of ef_topk_compress_noalloc: one array per GPU the library runs
// on, kept until the process ends and shared by every such call on that GPU.
// In host code `scratch` names a host-side stand-in, not device memory: only
// the device address looked up below (once per device, with that device
// current) is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[EF_TOPK_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];
}  // namespace

// Device address of this library's scratch array on the device that runs
// stream s (the current device for the NULL stream).
static int scratch_address(hipStream_t s, void** out) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return fail(EF_EHIP, "ef_topk_compress_noalloc: no current device");
    int dev = cur;
    if (s && hipStreamGetDevice(s, &dev) != hipSuccess)
        return fail(EF_EHIP, "ef_topk_compress_noalloc: cannot tell the stream's device");
    if (dev < 0 || dev >= kMaxDevices) return fail(EF_EINVAL, "ef_topk_compress_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess)
            return fail(EF_EHIP, "ef_topk_compress_noalloc: cannot select device %d", dev);
        void* ptr = nullptr;
        const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (err != hipSuccess || !ptr)
            return fail(EF_EHIP, "ef_topk_compress_noalloc: scratch address lookup failed: %s",
                        hipGetErrorString(err));
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return EF_OK;
}

}  // namespace topk
}  // namespace efg

using namespace efg;

extern "C" {

size_t ef_topk_workspace_bytes(int64_t n, int64_t k) {
    if (n < 0 || k < 0 || k > n || n > kMaxElems) return 0;
    int64_t off[2] = {0, n}, ks[1] = {k};
    topk::Plan p;
    if (topk::make_plan(1, off, ks, p) != EF_OK) return 0;
    return topk::make_layout(p).total;
}

// One flat tensor: a plan of one segment, built on the stack, whose tables
// always fit k_init's kernel arguments.
static int topk_flat(const float* g, float* e, int64_t n, int64_t k, float* vals, int32_t* idx, void* ws,
                     size_t ws_bytes, bool static_scratch, uint32_t* nonfinite, double* stats, uint32_t flags,
                     hipStream_t s) {
    if (n < 0 || n > kMaxElems) return fail(EF_EINVAL, "n=%lld outside [0, 2^31-1]", (long long)n);
    if (k < 0 || k > n) return fail(EF_EINVAL, "k=%lld outside [0, n=%lld]", (long long)k, (long long)n);
    EF_TRY(topk::check_common(g, e, n, k, vals, idx, flags));
    int64_t off[2] = {0, n}, ks[1] = {k};
    topk::Plan p;
    EF_TRY(topk::make_plan(1, off, ks, p));
    const topk::Layout L = topk::make_layout(p);
    if (static_scratch) {
        if (L.total > EF_TOPK_NOALLOC_SCRATCH_BYTES)
            return fail(EF_EWS, "ef_topk_compress_noalloc: n=%lld, k=%lld needs %zu bytes of scratch; the static "
                        "scratch holds %zu (use ef_topk_compress with a workspace)",
                        (long long)n, (long long)k, L.total, static_cast<size_t>(EF_TOPK_NOALLOC_SCRATCH_BYTES));
        ws_bytes = EF_TOPK_NOALLOC_SCRATCH_BYTES;
        ws = nullptr;
        if (p.R > 0) EF_TRY(topk::scratch_address(s, &ws));
    }
    uint32_t words[kWordChunk];
    static_assert(sizeof(words) >= 512, "a one-segment plan's tables fit the kernel arguments");
    topk::fill_words(p, L, words);
    return topk::run(g, e, p, L, topk::Tables{words, nullptr}, vals, idx, ws, ws_bytes, nonfinite, stats, flags, s);
}

int ef_topk_compress(const float* g, float* e, int64_t n, int64_t k, float* vals, int32_t* idx, void* ws,
                     size_t ws_bytes, uint32_t* nonfinite, double* stats, uint32_t flags, void* stream) {
    return topk_flat(g, e, n, k, vals, idx, ws, ws_bytes, false, nonfinite, stats, flags,
                     static_cast<hipStream_t>(stream));
}

int ef_topk_compress_noalloc(const float* g, float* e, int64_t n, int64_t k, float* vals, int32_t* idx,
                             uint32_t* nonfinite, double* stats, uint32_t flags, void* stream) {
    return topk_flat(g, e, n, k, vals, idx, nullptr, 0, true, nonfinite, stats, flags,
                     static_cast<hipStream_t>(stream));
}

__global__ void k_copy_status(const uint32_t* __restrict__ status, uint32_t* __restrict__ out) { *out = *status; }

__global__ void k_copy_paths(const topk::SegState* __restrict__ st, int32_t nseg, uint32_t* __restrict__ out) {
    for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < nseg; s += gridDim.x * blockDim.x) {
        out[2 * s] = st[s].fallback;
        out[2 * s + 1] = st[s].ncand;
    }
}

int ef_topk_workspace_status(const void* ws, uint32_t* stray, void* stream) {
    if (!stray) return fail(EF_EINVAL, "ef_topk_workspace_status: stray must not be NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* w = const_cast<void*>(ws);
    if (!w) EF_TRY(topk::scratch_address(s, &w));
    if (!aligned256(w)) return fail(EF_EINVAL, "ef_topk_workspace_status: workspace must be 256-byte aligned");
    return launch("topk_status", k_copy_status, dim3(1), dim3(1), s, static_cast<const uint32_t*>(w), stray);
}

int ef_topk_workspace_paths(const void* ws, size_t ws_bytes, int32_t nseg, uint32_t* out, void* stream) {
    if (nseg < 0) return fail(EF_EINVAL, "ef_topk_workspace_paths: nseg must be >= 0 (got %d)", nseg);
    if (nseg == 0) return EF_OK;
    if (!out) return fail(EF_EINVAL, "ef_topk_workspace_paths: out must not be NULL");
    topk::Layout L{};
    const size_t need = topk::layout_prefix(static_cast<size_t>(nseg), L);
    if (!ws) ws_bytes = EF_TOPK_NOALLOC_SCRATCH_BYTES;
    if (ws_bytes < need)
        return fail(EF_EWS, "ef_topk_workspace_paths: %d tensors need a workspace of at least %zu bytes (got %zu)",
                    nseg, need, ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* w = const_cast<void*>(ws);
    if (!w) EF_TRY(topk::scratch_address(s, &w));
    if (!aligned256(w)) return fail(EF_EINVAL, "ef_topk_workspace_paths: workspace must be 256-byte aligned");
    const topk::SegState* st = reinterpret_cast<const topk::SegState*>(static_cast<const uint8_t*>(w) + L.state);
    return launch("topk_paths", k_copy_paths, dim3(static_cast<unsigned>(std::min<int64_t>(1024, cdiv(nseg, 256)))),
                  dim3(256), s, st, nseg, out);
}

size_t ef_topk_segmented_workspace_bytes(int32_t nseg, const int64_t* seg_off, const int64_t* seg_k) {
    std::lock_guard<std::mutex> lk(topk::g_cache_mu);
    topk::CachedPlan* c = nullptr;
    if (topk::cached_plan(nseg, seg_off, seg_k, &c) != EF_OK) return 0;
    return c->L.total;
}

int ef_topk_compress_segmented(const float* g, float* e, int32_t nseg, const int64_t* seg_off,
                               const int64_t* seg_k, float* vals, int32_t* idx, void* ws, size_t ws_bytes,
                               uint32_t* nonfinite, double* stats, uint32_t flags, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lk(topk::g_cache_mu);
    topk::CachedPlan* c = nullptr;
    EF_TRY(topk::cached_plan(nseg, seg_off, seg_k, &c));
    int64_t ksum = 0;
    for (int32_t i = 0; i < nseg; ++i) ksum += seg_k[i];
    EF_TRY(topk::check_common(g, e, nseg > 0 ? seg_off[nseg] : 0, ksum, vals, idx, flags));
    if (c->plan.R > 0) {
        EF_TRY(topk::check_ws(c->L, ws, ws_bytes));
        EF_TRY(topk::pinned_tables(*c));
    }
    bool read_pinned = false;
    const int rc = topk::run(g, e, c->plan, c->L, topk::Tables{c->host, c->dev}, vals, idx, ws, ws_bytes, nonfinite,
                             stats, flags, s, &read_pinned);
    if (read_pinned) {
        // this call's k_init reads the entry's pinned tables when it runs
        if (hipEventRecord(c->read_done, s) != hipSuccess) return fail(EF_EHIP, "plan cache: event record failed");
        c->pending = true;
    }
    return rc;
}

}  // extern "C"
