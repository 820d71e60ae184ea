// Receiver side: sparse packets summed into a dense buffer, then the SGD update.
//
// "Gradient sparsification" page, basic-principle section (values of all
// workers that share an index are added) and step-by-step algorithm steps 6-7
// (aggregate, then w = w - lr * G).
//
// Decode without float atomics and in packet order: G is cut into tiles of
// 4096 positions, each summed in LDS by one block, so the sum at each index is
// ((G + v_p0) + v_p1) + ... in packet order, bit for bit.
//
// k_decode_tiles (up to 64 packets): a block owns a run of consecutive tiles
// (as many blocks as the GPU holds at once).  A packet's position is searched
// once per block and then carried from tile to tile, so a tile costs one
// round of loads, issued a tile ahead: every packet's next 16 entries and,
// fused with the SGD update, the tile's w.  Entries are applied in rounds
// that an LDS atomic min orders by packet (see the kernel).  Fused, G is
// written whole and w only where w - fl(lr * G) differs from w in its bits
// (where the packets land), with plain stores: on the 16-packet 25.6M
// workload, whose w and G (205 MB) fit the 256 MB last-level cache,
// non-temporal stores took 72 us a step against 54, and writing every quad of
// w 54 against 43.
// k_decode (more packets): one block per tile, each searching every packet
// for its entries (the design the multi-tile kernel replaced: 81 us fused).
#include <algorithm>

#include "common.hpp"

namespace efg {
namespace decode {

constexpr int kBlock = 256;
#ifndef EFG_DECODE_TILE
#define EFG_DECODE_TILE 4096
#endif
constexpr int kTile = EFG_DECODE_TILE;               // positions of G per block
#ifndef EFG_DECODE_STAGE
#define EFG_DECODE_STAGE 512
#endif
constexpr int kStage = EFG_DECODE_STAGE;             // staged entries per packet group (more: the global path)
constexpr int kSearchLanes = 16;                     // lanes that search one packet together
constexpr int kPkGroup = kBlock / kSearchLanes;      // packets searched at once per block

typedef float f4 __attribute__((ext_vector_type(4)));

#ifndef EFG_DECODE_NT_LOAD
#define EFG_DECODE_NT_LOAD 0
#endif
#ifndef EFG_DECODE_NT_STORE
#define EFG_DECODE_NT_STORE 0
#endif
__device__ __forceinline__ f4 ld4(const f4* p) {
    if (EFG_DECODE_NT_LOAD) return __builtin_nontemporal_load(p);
    return *p;
}
__device__ __forceinline__ void st4(f4 v, f4* p) {
    if (EFG_DECODE_NT_STORE) __builtin_nontemporal_store(v, p);
    else *p = v;
}
// w - fl(lr * G) stored only where its bits differ from w's: where G is +0 the
// difference is w itself (a signalling NaN comes back quiet and is stored), so
// a sparse G writes back only the quads its entries touch.  The result in
// memory is the same as storing every quad.
__device__ __forceinline__ void st4_changed(f4 wn, f4 wo, f4* p) {
    const bool same = __float_as_uint(wn.x) == __float_as_uint(wo.x) && __float_as_uint(wn.y) == __float_as_uint(wo.y) &&
                      __float_as_uint(wn.z) == __float_as_uint(wo.z) && __float_as_uint(wn.w) == __float_as_uint(wo.w);
    if (!same) st4(wn, p);
}

__global__ void k_zero_u32(uint32_t* p) { *p = 0; }

// entries that break the packet contract: index outside [0, n), or not above
// the previous entry of the same packet
__global__ __launch_bounds__(kBlock) void k_validate(int64_t n, const int32_t* __restrict__ idx,
                                                     const int64_t* __restrict__ pk_off,
                                                     uint32_t* __restrict__ invalid) {
    const int p = blockIdx.x;
    const int64_t b = pk_off[p], en = pk_off[p + 1];
    uint32_t bad = 0;
    for (int64_t j = b + threadIdx.x; j < en; j += kBlock) {
        const int32_t i = idx[j];
        bad += (i < 0 || i >= n || (j > b && idx[j - 1] >= i)) ? 1u : 0u;
    }
    bad = wave_sum(bad);
    if (lane() == 0 && bad) atomicAdd(invalid, bad);
}

// lower_bound(a[0..len), v) for two values at once, computed by the 16 lanes
// of one aligned lane group (gl = lane within the group).  A first round
// probes 16 positions 16 apart around the guess len * v / n (where the bound
// lies when the indices are spread evenly over [0, n)); each later round
// probes the last element of 16 equal sub-ranges of what is left.  Every
// round keeps the range between the last probe below v and the first one that
// is not, so a search takes two dependent loads when the guess is within 128
// entries and about log16(len) more when it is not; the two searches share
// their rounds.  Every lane of the wave must call it (it ballots); inactive
// groups pass len = 0.  For an unsorted list each result is still some
// position in [0, len].
struct Search {
    int64_t L, R, v;
};

__device__ __forceinline__ void search_round(const int32_t* a, Search& s, int gl, int shift, bool first,
                                             int64_t guess, int64_t len) {
    int64_t pos = 0;
    bool act = false;
    if (first) {
        act = len > 0;
        pos = min(max(guess + static_cast<int64_t>(gl - 8) * kSearchLanes, static_cast<int64_t>(0)), len - 1);
    } else if (s.R - s.L > kSearchLanes) {
        act = true;
        const int64_t step = (s.R - s.L + kSearchLanes - 1) / kSearchLanes;
        pos = min(s.L + static_cast<int64_t>(gl + 1) * step - 1, s.R - 1);
    }
    const bool below = act && static_cast<int64_t>(a[pos]) < s.v;
    const uint32_t m = static_cast<uint32_t>(__ballot(below) >> shift) & 0xffffu;
    if (!act) return;
    // probe positions are non-decreasing in the lane index: the range left
    // lies after the last probe below v (c of them) and up to the next one
    // (the group's lanes are all active here: act is the same for all 16)
    const int c = __popc(m);
    const int g0 = static_cast<int>(lane()) & ~(kSearchLanes - 1);
    const int64_t pl = __shfl(pos, g0 + max(c - 1, 0), kWave);
    const int64_t pr = __shfl(pos, g0 + min(c, kSearchLanes - 1), kWave);
    const int64_t nl = c > 0 ? pl + 1 : s.L;
    const int64_t nr = c < kSearchLanes ? pr : s.R;
    s.L = min(nl, s.R);
    s.R = max(nr, s.L);
}

__device__ __forceinline__ void group_lower_bound2(const int32_t* a, int64_t len, int64_t n, int64_t v0,
                                                   int64_t v1, int gl, int64_t* r0, int64_t* r1) {
    const int shift = threadIdx.x & 48;  // this group's 16 bits of the wave's ballot
    Search s0{0, len, v0}, s1{0, len, v1};
    const int64_t g0 = n > 0 ? len * v0 / n : 0, g1 = n > 0 ? len * v1 / n : 0;
    search_round(a, s0, gl, shift, true, g0, len);
    search_round(a, s1, gl, shift, true, g1, len);
    while (__any(s0.R - s0.L > kSearchLanes || s1.R - s1.L > kSearchLanes)) {
        search_round(a, s0, gl, shift, false, 0, len);
        search_round(a, s1, gl, shift, false, 0, len);
    }
    // at most 16 entries left: one probe each
    const int64_t p0 = s0.L + gl, p1 = s1.L + gl;
    const bool b0 = p0 < s0.R && static_cast<int64_t>(a[p0]) < v0;
    const bool b1 = p1 < s1.R && static_cast<int64_t>(a[p1]) < v1;
    *r0 = s0.L + __popc(static_cast<uint32_t>(__ballot(b0) >> shift) & 0xffffu);
    *r1 = s1.L + __popc(static_cast<uint32_t>(__ballot(b1) >> shift) & 0xffffu);
}

// FUSED: the receiver's whole step on a G that starts at zero.  Every
// position of the tile starts at +0 in LDS (no G load), the packets are added
// as above, and the tile is written out whole: G (if given) = the sum, and
// w = w - fl(lr * G), the same two roundings as sgd_apply.  One pass over w and
// G instead of a zero fill, the scatter-add and the update.
template <bool FUSED>
__global__ __launch_bounds__(kBlock) void k_decode(float* __restrict__ G, int64_t n, int32_t npk,
                                                   const float* __restrict__ vals, const int32_t* __restrict__ idx,
                                                   const int64_t* __restrict__ pk_off, float* __restrict__ w,
                                                   float lr) {
    __shared__ float acc[kTile];
    __shared__ uint32_t touched[kTile / 32];
    __shared__ uint16_t st_loc[kStage];
    __shared__ float st_val[kStage];
    __shared__ int64_t p_lo[kPkGroup];
    __shared__ uint32_t p_cnt[kPkGroup], p_sof[kPkGroup + 1];
    __shared__ uint32_t lds[kBlock / kWave + 1];

    const int64_t lo = static_cast<int64_t>(blockIdx.x) * kTile;
    const int64_t hi = min(lo + kTile, n);
    if (FUSED) {
        for (int i = threadIdx.x; i < kTile; i += kBlock) acc[i] = 0.0f;
    } else {
        for (int i = threadIdx.x; i < kTile / 32; i += kBlock) touched[i] = 0;
    }
    __syncthreads();

    // first touch of a position loads G; later touches add in LDS
    auto touch = [&](uint32_t loc) {
        if (FUSED) return;
        const uint32_t bit = 1u << (loc & 31);
        const uint32_t old = atomicOr(&touched[loc >> 5], bit);
        if (!(old & bit)) acc[loc] = G[lo + loc];
    };
    // is entry j of packet [pb, pe) a valid member of this tile?  returns its local slot or -1
    auto local_of = [&](int64_t j, int64_t pb) -> int32_t {
        const int64_t i = idx[j];
        if (i < lo || i >= hi) return -1;
        if (j > pb && static_cast<int64_t>(idx[j - 1]) >= i) return -1;
        return static_cast<int32_t>(i - lo);
    };

    for (int32_t pg = 0; pg < npk; pg += kPkGroup) {
        const int32_t np = min(kPkGroup, npk - pg);
        {
            // lane group grp searches packet pg + grp for the entries inside [lo, hi)
            const int grp = threadIdx.x / kSearchLanes, gl = threadIdx.x % kSearchLanes;
            int64_t pb = 0, len = 0;
            if (grp < np) {
                pb = pk_off[pg + grp];
                const int64_t pe = pk_off[pg + grp + 1];
                len = pe > pb ? pe - pb : 0;
            }
            int64_t a, b;
            group_lower_bound2(idx + pb, len, n, lo, hi, gl, &a, &b);
            if (grp < np && gl == 0) {
                p_lo[grp] = pb + a;
                p_cnt[grp] = static_cast<uint32_t>(b > a ? b - a : 0);
            }
        }
        __syncthreads();
        const uint32_t cnt = static_cast<int32_t>(threadIdx.x) < np ? p_cnt[threadIdx.x] : 0u;
        uint32_t total;
        const uint32_t ex = block_excl_scan<kBlock>(cnt, lds, &total);
        if (static_cast<int32_t>(threadIdx.x) < np) p_sof[threadIdx.x] = ex;
        if (threadIdx.x == 0) p_sof[np] = total;
        __syncthreads();

        if (total <= kStage) {
            // stage every entry of the group, in packet order
            for (uint32_t q = threadIdx.x; q < total; q += kBlock) {
                const int p = upper_index(p_sof, np, q);
                const int64_t j = p_lo[p] + (q - p_sof[p]);
                const int32_t loc = local_of(j, pk_off[pg + p]);
                st_loc[q] = loc < 0 ? 0xffffu : static_cast<uint16_t>(loc);
                st_val[q] = vals[j];
                if (loc >= 0) touch(static_cast<uint32_t>(loc));
            }
            __syncthreads();
            for (int p = 0; p < np; ++p) {
                for (uint32_t q = p_sof[p] + threadIdx.x; q < p_sof[p + 1]; q += kBlock) {
                    const uint16_t loc = st_loc[q];
                    if (loc != 0xffffu) acc[loc] = acc[loc] + st_val[q];
                }
                __syncthreads();
            }
        } else {
            // many entries in this tile: apply packet by packet from global memory
            for (int p = 0; p < np; ++p) {
                const int64_t pb = pk_off[pg + p];
                for (uint32_t t = threadIdx.x; t < p_cnt[p]; t += kBlock) {
                    const int64_t j = p_lo[p] + t;
                    const int32_t loc = local_of(j, pb);
                    if (loc >= 0) {
                        touch(static_cast<uint32_t>(loc));
                        acc[loc] = acc[loc] + vals[j];
                    }
                }
                __syncthreads();
            }
        }
        __syncthreads();
    }
    if (!FUSED) {
        for (int t = threadIdx.x; t < kTile; t += kBlock)
            if (touched[t >> 5] & (1u << (t & 31))) G[lo + t] = acc[t];
        return;
    }
    // the whole tile, four positions per thread at a time (w, G 16-byte aligned,
    // lo a multiple of 4).  Reading w at the block's start instead, under the
    // packet search, measured slower (its registers cost a wave per SIMD).
    // All of a thread's w loads go out together.
    constexpr int kQuads = kTile / (4 * kBlock);
    static_assert(kTile % (4 * kBlock) == 0, "a tile is whole quads of every thread");
    const int64_t len = hi - lo;
    f4 wv[kQuads];
#pragma unroll
    for (int r = 0; r < kQuads; ++r) {
        const int t = 4 * (static_cast<int>(threadIdx.x) + r * kBlock);
        if (t + 4 <= len) wv[r] = ld4(reinterpret_cast<const f4*>(w + lo + t));
    }
#pragma unroll
    for (int r = 0; r < kQuads; ++r) {
        const int t = 4 * (static_cast<int>(threadIdx.x) + r * kBlock);
        if (t + 4 <= len) {
            const f4 a = {acc[t], acc[t + 1], acc[t + 2], acc[t + 3]};
            const f4 st = lr * a;
            st4_changed(wv[r] - st, wv[r], reinterpret_cast<f4*>(w + lo + t));
            if (G) st4(a, reinterpret_cast<f4*>(G + lo + t));
        } else if (t < len) {
            for (int c = 0; c < 4 && t + c < len; ++c) {
                const float st = lr * acc[t + c];
                w[lo + t + c] = w[lo + t + c] - st;
                if (G) G[lo + t + c] = acc[t + c];
            }
        }
    }
}

// ------------------------------------------------------------------ multi-tile decode
// Each block owns a run of consecutive tiles.  Every packet's position is
// searched once, for the block's first tile, and then carried from tile to
// tile in the registers of the packet's 16 lanes, so that a tile costs one
// round of loads: every packet's next 16 entries (index, the index before it,
// value), read together with the tile's w.  The entries below the tile's end
// (their count is the run of leading lanes found by a ballot) are applied to
// the tile's LDS sums in packet order without a barrier per packet: in each
// round every pending entry offers (round tag, packet-major slot) to its
// position with an LDS atomic min, and the entry holding the minimum adds; the
// tag of a later round is smaller, so older tags never win.  A position that
// several packets hit takes one round per packet, in packet order; the others
// all add in the first round.  A packet with 16 or more entries in one tile
// sends the whole tile down the dense path, which stages every entry from
// global memory in packet-major chunks and applies each chunk the same way.
constexpr int kMaxPk = 64;                        // packets whose cursors a block carries
constexpr int kDenseStage = 1024;                 // entries per staged chunk of a dense tile
constexpr int kWin = kSearchLanes;                // entries of a packet read per tile and round

// lower_bound(a[0..len), v) by the 16 lanes of a group (every lane of the wave
// must call it; inactive groups pass len = 0)
__device__ __forceinline__ int64_t group_lower_bound1(const int32_t* a, int64_t len, int64_t v, int gl) {
    const int shift = threadIdx.x & 48;
    Search s{0, len, v};
    while (__any(s.R - s.L > kSearchLanes)) search_round(a, s, gl, shift, false, 0, len);
    const int64_t p = s.L + gl;
    const bool b = p < s.R && static_cast<int64_t>(a[p]) < v;
    return s.L + __popc(static_cast<uint32_t>(__ballot(b) >> shift) & 0xffffu);
}

// Round tag of an LDS atomic-min key: later rounds get smaller tags.
__device__ __forceinline__ uint32_t round_key(uint32_t epoch, uint32_t slot) {
    return ((0xffffu - epoch) << 16) | slot;
}

// One entry's addition to the tile: the fused form sums from +0; the other
// loads G at a position's first touch in the tile (touched bit).
template <bool FUSED>
__device__ __forceinline__ bool apply_entry(float* acc, uint32_t* touched, const float* G, int64_t lo, uint32_t loc,
                                            float v) {
    if (FUSED) {
        acc[loc] = acc[loc] + v;
        return false;
    }
    const uint32_t bit = 1u << (loc & 31);
    const uint32_t old = atomicOr(&touched[loc >> 5], bit);
    const bool first = !(old & bit);
    const float base = first ? G[lo + loc] : acc[loc];
    acc[loc] = base + v;
    return first;  // this entry writes the position back once the tile is summed
}

#ifndef EFG_DECODE_WAVES
#define EFG_DECODE_WAVES 1
#endif
// The run of tiles of block b.  Blocks are dealt to the eight XCDs in turn
// (block b to XCD b mod 8); here the blocks of one XCD take consecutive runs,
// so the bound searches of neighbouring runs, which probe nearby lines of
// every packet's indices, meet in that XCD's L2 instead of eight.  A
// bijection of [0, nb) for any nb.
__device__ __forceinline__ int64_t xcd_run(int64_t b, int64_t nb) {
    constexpr int64_t kXcds = 8;
    const int64_t q = nb / kXcds, rem = nb % kXcds, x = b % kXcds, j = b / kXcds;
    return x * q + min(x, rem) + j;
}
template <bool FUSED, int SLOTS>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(EFG_DECODE_WAVES))) void k_decode_tiles(float* __restrict__ G, int64_t n, int32_t npk,
                                                         const float* __restrict__ vals,
                                                         const int32_t* __restrict__ idx,
                                                         const int64_t* __restrict__ pk_off, float* __restrict__ w,
                                                         float lr, int64_t ntiles) {
    __shared__ float acc[kTile];
    __shared__ uint32_t own[kTile];
    __shared__ uint32_t touched[kTile / 32];
    __shared__ uint16_t st_loc[kDenseStage];
    __shared__ float st_val[kDenseStage];
    __shared__ uint32_t p_cnt[kMaxPk], p_sof[kMaxPk + 1];
    __shared__ int64_t p_beg[kMaxPk];
    __shared__ uint32_t lds[kBlock / kWave + 1];

    const int64_t run = xcd_run(blockIdx.x, gridDim.x);
    const int64_t t0 = run * ntiles / gridDim.x;
    const int64_t t1 = (run + 1) * ntiles / gridDim.x;
    const int tid = threadIdx.x, grp = tid / kSearchLanes, gl = tid % kSearchLanes;
    const int g0 = static_cast<int>(lane()) & ~(kSearchLanes - 1);  // the group's first lane in the wave
    for (int i = tid; i < kTile; i += kBlock) {
        own[i] = 0xffffffffu;
        if (FUSED) acc[i] = 0.0f;
    }
    if (!FUSED)
        for (int i = tid; i < kTile / 32; i += kBlock) touched[i] = 0;

    // packet grp + 16 u of lane group grp: entries [pb, pe), next entry cur,
    // index of the entry before cur (last; -1 if none: indices are >= 0)
    int64_t pb[SLOTS], pe[SLOTS], cur[SLOTS];
    int64_t last[SLOTS];
    {
        const int64_t lo0 = t0 * kTile;
#pragma unroll
        for (int u = 0; u < SLOTS; ++u) {
            const int p = grp + kPkGroup * u;
            pb[u] = pe[u] = 0;
            if (p < npk) {
                pb[u] = pk_off[p];
                pe[u] = max(pk_off[p + 1], pb[u]);
            }
            int64_t a, b;
            group_lower_bound2(idx + pb[u], pe[u] - pb[u], n, lo0, lo0, gl, &a, &b);
            cur[u] = pb[u] + a;
            last[u] = -1;
            if (cur[u] > pb[u]) last[u] = idx[cur[u] - 1];
        }
    }
    __syncthreads();

    constexpr int kQuads = kTile / (4 * kBlock);
    static_assert(kTile % (4 * kBlock) == 0, "a tile is whole quads of every thread");
    uint32_t epoch = 0;
    // after each round (every thread, uniformly): the next tag; when the 16-bit
    // tags run out, every position's key goes back above all tags
    auto next_round = [&]() {
        if (++epoch == 0x10000u) {
            __syncthreads();
            for (int i = tid; i < kTile; i += kBlock) own[i] = 0xffffffffu;
            epoch = 0;
            __syncthreads();
        }
    };
    // Loads of a tile, issued as early as their inputs allow: w needs only the
    // tile, the entry window of a packet its cursor after the tile before.
    auto load_w = [&](int64_t t, f4 (&wv)[kQuads]) {
        const int64_t lo = t * kTile, len = min(lo + kTile, n) - lo;
#pragma unroll
        for (int r = 0; r < kQuads; ++r) {
            const int q = 4 * (tid + r * kBlock);
            if (q + 4 <= len) wv[r] = ld4(reinterpret_cast<const f4*>(w + lo + q));
        }
    };
    auto load_window = [&](int32_t (&x)[SLOTS], float (&v)[SLOTS], bool (&in)[SLOTS]) {
#pragma unroll
        for (int u = 0; u < SLOTS; ++u) {
            const int64_t j = cur[u] + gl;
            in[u] = j < pe[u];
            x[u] = 0x7fffffff;
            v[u] = 0.0f;
            if (in[u]) {
                x[u] = idx[j];
                v[u] = vals[j];
            }
        }
    };
    f4 wA[kQuads];
    int32_t xA[SLOTS];
    float vA[SLOTS];
    bool inA[SLOTS];
    if (FUSED) load_w(t0, wA);
    load_window(xA, vA, inA);
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t lo = t * kTile, hi = min(lo + kTile, n);
        const int64_t len = hi - lo;
        const bool more = t + 1 < t1;
        // the next tile's w, in flight while this tile is summed and written
        f4 wB[kQuads];
        if (FUSED && more) load_w(t + 1, wB);
        uint32_t lead[SLOTS];
        bool full = false;
#pragma unroll
        for (int u = 0; u < SLOTS; ++u) {
            const bool lt = inA[u] && xA[u] < hi;
            const uint32_t m = static_cast<uint32_t>(__ballot(lt) >> (tid & 48)) & 0xffffu;
            lead[u] = __ffs(~m | 0x10000u) - 1;  // leading lanes below hi (16: window full)
            full |= lead[u] == kWin;
        }
        const bool dense = __syncthreads_or(full);
        int32_t xB[SLOTS];
        float vB[SLOTS];
        bool inB[SLOTS];
        uint32_t back[SLOTS];  // positions this lane writes back (accumulate only; 0xffffffff: none)
#pragma unroll
        for (int u = 0; u < SLOTS; ++u) back[u] = 0xffffffffu;
        if (!dense) {
            // each lane applies its own entry: valid when in [lo, hi) (so in [0, n))
            // and above the entry before it in its packet
            bool pend[SLOTS];
            uint32_t loc[SLOTS];
            float val[SLOTS];
            bool anyp = false;
#pragma unroll
            for (int u = 0; u < SLOTS; ++u) {
                const int64_t prev = __shfl_up(xA[u], 1, kSearchLanes);
                const int64_t before = gl == 0 ? last[u] : prev;
                pend[u] = static_cast<uint32_t>(gl) < lead[u] && xA[u] >= lo && xA[u] > before;
                loc[u] = pend[u] ? static_cast<uint32_t>(xA[u] - lo) : 0u;
                val[u] = vA[u];
                anyp |= pend[u];
                const int32_t lx = __shfl(xA[u], g0 + static_cast<int>(lead[u] > 0 ? lead[u] - 1 : 0), kWave);
                if (lead[u] > 0) last[u] = lx;
                cur[u] += lead[u];
            }
            // the next tile's windows go out before this tile's sums and stores
            if (more) load_window(xB, vB, inB);
            while (__syncthreads_or(anyp)) {
#pragma unroll
                for (int u = 0; u < SLOTS; ++u)
                    if (pend[u]) atomicMin(&own[loc[u]], round_key(epoch, static_cast<uint32_t>((grp + kPkGroup * u) * kWin + gl)));
                __syncthreads();
                anyp = false;
#pragma unroll
                for (int u = 0; u < SLOTS; ++u) {
                    if (pend[u] && own[loc[u]] == round_key(epoch, static_cast<uint32_t>((grp + kPkGroup * u) * kWin + gl))) {
                        if (apply_entry<FUSED>(acc, touched, G, lo, loc[u], val[u])) back[u] = loc[u];
                        pend[u] = false;
                    }
                    anyp |= pend[u];
                }
                next_round();
            }
        } else {
            // dense tile: every packet's entries below hi, staged from global
            // memory in packet-major chunks
            uint32_t cnt[SLOTS];
#pragma unroll
            for (int u = 0; u < SLOTS; ++u) {
                const bool f = lead[u] == kWin;
                const int64_t from = cur[u] + (f ? kWin : 0);
                const int64_t e = group_lower_bound1(idx + from, f ? pe[u] - from : 0, hi, gl);
                cnt[u] = lead[u] + static_cast<uint32_t>(f ? e : 0);
                const int p = grp + kPkGroup * u;
                if (gl == 0 && p < npk) {
                    p_cnt[p] = cnt[u];
                    p_beg[p] = cur[u];
                }
            }
            __syncthreads();
            const uint32_t c = tid < npk ? p_cnt[tid] : 0u;
            uint32_t total;
            const uint32_t ex = block_excl_scan<kBlock>(c, lds, &total);
            if (tid < npk) p_sof[tid] = ex;
            if (tid == 0) p_sof[npk] = total;
            __syncthreads();
            for (uint32_t cb = 0; cb < total; cb += kDenseStage) {
                const uint32_t ce = min(total, cb + kDenseStage);
                for (uint32_t q = cb + tid; q < ce; q += kBlock) {
                    const int p = upper_index(p_sof, npk, q);
                    const int64_t j = p_beg[p] + (q - p_sof[p]);
                    const int64_t xi = idx[j];
                    const int64_t before = j > pk_off[p] ? static_cast<int64_t>(idx[j - 1]) : -1;
                    const bool ok = xi >= lo && xi < hi && xi > before;
                    st_loc[q - cb] = ok ? static_cast<uint16_t>(xi - lo) : 0xffffu;
                    st_val[q - cb] = vals[j];
                }
                __syncthreads();
                constexpr int kPer = kDenseStage / kBlock;
                bool pend[kPer];
                bool anyp = false;
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const uint32_t q = tid + i * kBlock;
                    pend[i] = cb + q < ce && st_loc[q] != 0xffffu;
                    anyp |= pend[i];
                }
                while (__syncthreads_or(anyp)) {
#pragma unroll
                    for (int i = 0; i < kPer; ++i)
                        if (pend[i]) atomicMin(&own[st_loc[tid + i * kBlock]], round_key(epoch, tid + i * kBlock));
                    __syncthreads();
                    anyp = false;
#pragma unroll
                    for (int i = 0; i < kPer; ++i) {
                        const uint32_t q = tid + i * kBlock;
                        if (pend[i] && own[st_loc[q]] == round_key(epoch, q)) {
                            apply_entry<FUSED>(acc, touched, G, lo, st_loc[q], st_val[q]);
                            pend[i] = false;
                        }
                        anyp |= pend[i];
                    }
                    next_round();
                }
                __syncthreads();  // the chunk's staging area is reused by the next chunk
            }
#pragma unroll
            for (int u = 0; u < SLOTS; ++u) {
                if (cnt[u] > 0) last[u] = idx[cur[u] + cnt[u] - 1];
                cur[u] += cnt[u];
            }
            if (more) load_window(xB, vB, inB);
        }
        __syncthreads();
        if (FUSED) {
            // the whole tile: G (if given) = the sum, w -= fl(lr * G); the sums go
            // back to +0 for the next tile
#pragma unroll
            for (int r = 0; r < kQuads; ++r) {
                const int q = 4 * (tid + r * kBlock);
                if (q + 4 <= len) {
                    const f4 a = *reinterpret_cast<const f4*>(&acc[q]);
                    *reinterpret_cast<f4*>(&acc[q]) = f4{0.f, 0.f, 0.f, 0.f};
                    const f4 st = lr * a;
                    st4_changed(wA[r] - st, wA[r], reinterpret_cast<f4*>(w + lo + q));
                    if (G) st4(a, reinterpret_cast<f4*>(G + lo + q));
                } else if (q < len) {
                    for (int c = 0; c < 4 && q + c < len; ++c) {
                        const float st = lr * acc[q + c];
                        w[lo + q + c] = w[lo + q + c] - st;
                        if (G) G[lo + q + c] = acc[q + c];
                        acc[q + c] = 0.0f;
                    }
                }
            }
        } else {
            if (dense) {
                for (int i = tid; i < kTile; i += kBlock)
                    if (touched[i >> 5] & (1u << (i & 31))) G[lo + i] = acc[i];
                __syncthreads();
            } else {
                // each position by the entry that touched it first
#pragma unroll
                for (int u = 0; u < SLOTS; ++u)
                    if (back[u] != 0xffffffffu) G[lo + back[u]] = acc[back[u]];
            }
            for (int i = tid; i < kTile / 32; i += kBlock) touched[i] = 0;
        }
        __syncthreads();
        if (more) {
#pragma unroll
            for (int r = 0; r < kQuads; ++r) wA[r] = wB[r];
#pragma unroll
            for (int u = 0; u < SLOTS; ++u) {
                xA[u] = xB[u];
                vA[u] = vB[u];
                inA[u] = inB[u];
            }
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_sgd(float* __restrict__ w, const float* __restrict__ G, int64_t n,
                                                float lr) {
    const int64_t nv = n >> 2;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    f4* w4 = reinterpret_cast<f4*>(w);
    const f4* g4 = reinterpret_cast<const f4*>(G);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < nv; i += stride) {
        const f4 gv = ld4(g4 + i);
        const f4 wv = ld4(w4 + i);
        const f4 st = lr * gv;
        st4_changed(wv - st, wv, w4 + i);
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        const int64_t j = nv * 4 + threadIdx.x;
        const float st = lr * G[j];
        w[j] = w[j] - st;
    }
}

// Blocks of the multi-tile kernel that the GPU holds at once (its LDS use
// sets that; at most EFG_DECODE_PER_CU per CU when that is set), asked once
// per kernel and device.
#ifndef EFG_DECODE_PER_CU
#define EFG_DECODE_PER_CU 0
#endif
template <bool FUSED, int SLOTS>
static int resident_blocks(int64_t* out) {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(EF_EHIP, "decode: no current device");
    if (!cached[dev]) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_tiles<FUSED, SLOTS>, kBlock, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return fail(EF_EHIP, "decode: occupancy query failed");
        if (EFG_DECODE_PER_CU > 0) per_cu = std::min(per_cu, EFG_DECODE_PER_CU);
        cached[dev] = std::max(1, per_cu) * std::max(1, cus);
    }
    *out = cached[dev];
    return EF_OK;
}

// The tiles of G split among the blocks the GPU holds at once, each block a
// run of consecutive tiles; more packets than one block carries take the
// one-tile-per-block kernel.
template <bool FUSED>
static int launch_decode(const char* label, float* G, int64_t n, int32_t npk, const float* vals,
                         const int32_t* idx, const int64_t* pk_off, float* w, float lr, hipStream_t s) {
    const int64_t ntiles = cdiv(n, kTile);
    if (npk > kMaxPk)
        return launch(label, k_decode<FUSED>, dim3(static_cast<unsigned>(ntiles)), dim3(kBlock), s, G, n, npk,
                      vals, idx, pk_off, w, lr);
    int64_t res = 0;
    if (npk <= kPkGroup) {
        EF_TRY((resident_blocks<FUSED, 1>(&res)));
        return launch(label, k_decode_tiles<FUSED, 1>, dim3(static_cast<unsigned>(std::min(ntiles, res))),
                      dim3(kBlock), s, G, n, npk, vals, idx, pk_off, w, lr, ntiles);
    }
    EF_TRY((resident_blocks<FUSED, kMaxPk / kPkGroup>(&res)));
    return launch(label, k_decode_tiles<FUSED, kMaxPk / kPkGroup>, dim3(static_cast<unsigned>(std::min(ntiles, res))),
                  dim3(kBlock), s, G, n, npk, vals, idx, pk_off, w, lr, ntiles);
}

}  // namespace decode
}  // namespace efg

using namespace efg;

extern "C" int sparse_decode_accumulate(float* G, int64_t n, int32_t npk, const float* vals, const int32_t* idx,
                                        const int64_t* pk_off, uint32_t* invalid, void* stream) {
    if (n < 0 || n > kMaxElems) return fail(EF_EINVAL, "n=%lld outside [0, 2^31-1]", (long long)n);
    if (npk < 0) return fail(EF_EINVAL, "npk must be >= 0");
    if (npk > 0 && (!vals || !idx || !pk_off)) return fail(EF_EINVAL, "vals, idx and pk_off must not be NULL");
    if (n > 0 && !G) return fail(EF_EINVAL, "G must not be NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (invalid) {
        EF_TRY(launch("decode_zero", decode::k_zero_u32, dim3(1), dim3(1), s, invalid));
        if (npk > 0)
            EF_TRY(launch("decode_validate", decode::k_validate, dim3(static_cast<unsigned>(npk)), dim3(decode::kBlock),
                          s, n, idx, pk_off, invalid));
    }
    if (n == 0 || npk == 0) return EF_OK;
    return decode::launch_decode<false>("decode_scatter", G, n, npk, vals, idx, pk_off, nullptr, 0.0f, s);
}

extern "C" int sparse_decode_sgd(float* w, float* G, int64_t n, int32_t npk, const float* vals, const int32_t* idx,
                                 const int64_t* pk_off, float lr, uint32_t* invalid, void* stream) {
    if (n < 0 || n > kMaxElems) return fail(EF_EINVAL, "n=%lld outside [0, 2^31-1]", (long long)n);
    if (npk < 0) return fail(EF_EINVAL, "npk must be >= 0");
    if (npk > 0 && (!vals || !idx || !pk_off)) return fail(EF_EINVAL, "vals, idx and pk_off must not be NULL");
    if (n > 0 && !w) return fail(EF_EINVAL, "w must not be NULL");
    if (n > 0 && (!aligned16(w) || (G && !aligned16(G)))) return fail(EF_EINVAL, "w and G must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (invalid) {
        EF_TRY(launch("decode_zero", decode::k_zero_u32, dim3(1), dim3(1), s, invalid));
        if (npk > 0)
            EF_TRY(launch("decode_validate", decode::k_validate, dim3(static_cast<unsigned>(npk)), dim3(decode::kBlock),
                          s, n, idx, pk_off, invalid));
    }
    if (n == 0) return EF_OK;
    return decode::launch_decode<true>("decode_sgd", G, n, npk, vals, idx, pk_off, w, lr, s);
}

extern "C" int sgd_apply(float* w, const float* G, int64_t n, float lr, void* stream) {
    if (n < 0) return fail(EF_EINVAL, "n must be >= 0");
    if (n == 0) return EF_OK;
    if (!w || !G) return fail(EF_EINVAL, "w and G must not be NULL");
    if (!aligned16(w) || !aligned16(G)) return fail(EF_EINVAL, "w and G must be 16-byte aligned");
    int64_t grid = cdiv((n >> 2) + 1, decode::kBlock);
    if (grid > 16384) grid = 16384;
    return launch("sgd_apply", decode::k_sgd, dim3(static_cast<unsigned>(grid)), dim3(decode::kBlock),
                  static_cast<hipStream_t>(stream), w, G, n, lr);
}
