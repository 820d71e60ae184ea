// Receiver side: sparse packets summed into a dense buffer, then the SGD update.
//
// "Gradient sparsification" page, basic-principle section (values of all
// workers that share an index are added) and step-by-step algorithm steps 6-7
// (aggregate, then w = w - lr * G).
//
// Decode without float atomics and in packet order: each block owns one tile
// of 4096 consecutive positions of G.  For every packet, 16 lanes search the
// packet's (ascending) index list together for the entries that land in the
// tile, stage them in LDS, load G once for every touched position, add the
// packets one after another in LDS (a barrier between packets keeps the
// order), and write every touched position back once.  The sum at each index
// is therefore ((G + v_p0) + v_p1) + ... in packet order, bit for bit.
// The block's time is a chain of dependent loads (packet bounds, search,
// entries, G), so what counts is how many blocks a CU holds at once: a 4096
// tile and 512 staged entries (20 KB of LDS, up to eight blocks per CU) took
// 48 us on the 16-packet 25.6M workload, against 62 us for 8192 and 2048
// (45 KB, three per CU); tiles of 2048 to 8192 and stages of 256 to 2048
// were tried.  A tile whose packets hold more than 512 entries in it takes
// the slower path that adds them from global memory.
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
        if (t + 4 <= len) wv[r] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(w + lo + t));
    }
#pragma unroll
    for (int r = 0; r < kQuads; ++r) {
        const int t = 4 * (static_cast<int>(threadIdx.x) + r * kBlock);
        if (t + 4 <= len) {
            const f4 a = {acc[t], acc[t + 1], acc[t + 2], acc[t + 3]};
            const f4 st = lr * a;
            __builtin_nontemporal_store(wv[r] - st, reinterpret_cast<f4*>(w + lo + t));
            if (G) __builtin_nontemporal_store(a, reinterpret_cast<f4*>(G + lo + t));
        } else if (t < len) {
            for (int c = 0; c < 4 && t + c < len; ++c) {
                const float st = lr * acc[t + c];
                w[lo + t + c] = w[lo + t + c] - st;
                if (G) G[lo + t + c] = acc[t + c];
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
        const f4 gv = __builtin_nontemporal_load(g4 + i);
        const f4 wv = __builtin_nontemporal_load(w4 + i);
        const f4 st = lr * gv;
        __builtin_nontemporal_store(wv - st, w4 + i);
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        const int64_t j = nv * 4 + threadIdx.x;
        const float st = lr * G[j];
        w[j] = w[j] - st;
    }
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
    return launch("decode_scatter", decode::k_decode<false>, dim3(static_cast<unsigned>(cdiv(n, decode::kTile))),
                  dim3(decode::kBlock), s, G, n, npk, vals, idx, pk_off, static_cast<float*>(nullptr), 0.0f);
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
    return launch("decode_sgd", decode::k_decode<true>, dim3(static_cast<unsigned>(cdiv(n, decode::kTile))),
                  dim3(decode::kBlock), s, G, n, npk, vals, idx, pk_off, w, lr);
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
