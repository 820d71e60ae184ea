// Receiver side: sparse packets summed into a dense buffer, then the SGD update.
//
// "Gradient sparsification" page, basic-principle section (values of all
// workers that share an index are added) and step-by-step algorithm steps 6-7
// (aggregate, then w = w - lr * G).
//
// Decode without float atomics and in packet order: each block owns one tile
// of 8192 consecutive positions of G (fastest of 1024-16384 on MI355X).  For
// every packet, 16 lanes search the packet's (ascending) index list together
// for the entries that land in the tile,
// stages them in LDS, loads G once for every touched position, adds the
// packets one after another in LDS (a barrier between packets keeps the
// order), and writes every touched position back once.  The sum at each index
// is therefore ((G + v_p0) + v_p1) + ... in packet order, bit for bit.
#include "common.hpp"

namespace efg {
namespace decode {

constexpr int kBlock = 256;
#ifndef EFG_DECODE_TILE
#define EFG_DECODE_TILE 8192
#endif
constexpr int kTile = EFG_DECODE_TILE;               // positions of G per block
constexpr int kStage = 2048;
constexpr int kSearchLanes = 16;                     // lanes that search one packet together
constexpr int kPkGroup = kBlock / kSearchLanes;      // packets searched at once per block

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

// lower_bound(a[0..len), v) computed by the 16 lanes of one aligned lane group
// (gl = lane within the group): each round probes the last element of 16
// equal sub-ranges and keeps the first one that reaches v, so a search takes
// about log16(len) dependent loads instead of log2(len).  Every lane of the
// wave must call it (it ballots); inactive groups pass len = 0.  For an
// unsorted list the result is still some position in [0, len].
__device__ __forceinline__ int64_t group_lower_bound(const int32_t* a, int64_t len, int64_t v, int gl) {
    const int shift = threadIdx.x & 48;  // this group's 16 bits of the wave's ballot
    int64_t L = 0, R = len;
    while (__any(R - L > kSearchLanes)) {
        const bool more = R - L > kSearchLanes;
        const int64_t step = more ? (R - L + kSearchLanes - 1) / kSearchLanes : 0;
        const int64_t pos = L + static_cast<int64_t>(gl + 1) * step - 1;
        const bool below = more && pos < R && static_cast<int64_t>(a[pos]) < v;
        const uint32_t m = static_cast<uint32_t>(__ballot(below) >> shift) & 0xffffu;
        if (more) {
            const int64_t c = __popc(m);
            const int64_t nl = min(L + c * step, R);
            R = min(L + (c + 1) * step, R);
            L = nl;
        }
    }
    const int64_t pos = L + gl;
    const bool below = pos < R && static_cast<int64_t>(a[pos]) < v;
    return L + __popc(static_cast<uint32_t>(__ballot(below) >> shift) & 0xffffu);
}

__global__ __launch_bounds__(kBlock) void k_decode(float* __restrict__ G, int64_t n, int32_t npk,
                                                   const float* __restrict__ vals, const int32_t* __restrict__ idx,
                                                   const int64_t* __restrict__ pk_off) {
    __shared__ float acc[kTile];
    __shared__ uint32_t touched[kTile / 32];
    __shared__ uint16_t st_loc[kStage];
    __shared__ float st_val[kStage];
    __shared__ int64_t p_lo[kPkGroup];
    __shared__ uint32_t p_cnt[kPkGroup], p_sof[kPkGroup + 1];
    __shared__ uint32_t lds[kBlock / kWave + 1];

    const int64_t lo = static_cast<int64_t>(blockIdx.x) * kTile;
    const int64_t hi = min(lo + kTile, n);
    for (int i = threadIdx.x; i < kTile / 32; i += kBlock) touched[i] = 0;
    __syncthreads();

    // first touch of a position loads G; later touches add in LDS
    auto touch = [&](uint32_t loc) {
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
            const int64_t a = group_lower_bound(idx + pb, len, lo, gl);
            const int64_t b = group_lower_bound(idx + pb, len, hi, gl);
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
    for (int t = threadIdx.x; t < kTile; t += kBlock)
        if (touched[t >> 5] & (1u << (t & 31))) G[lo + t] = acc[t];
}

typedef float f4 __attribute__((ext_vector_type(4)));

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
    return launch("decode_scatter", decode::k_decode, dim3(static_cast<unsigned>(cdiv(n, decode::kTile))),
                  dim3(decode::kBlock), s, G, n, npk, vals, idx, pk_off);
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
