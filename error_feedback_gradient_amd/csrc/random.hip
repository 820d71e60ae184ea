// Random magnitude-proportional sparsification with error feedback, gfx950.
//
// "梯度稀疏化" page, section "随机稀疏化" (random sparsification): each element
// survives with a probability proportional to its magnitude, normalised so
// that k survive on average; it sits inside the page's generic error
// compensation loop (section "误差补偿": add the residual, sparsify, keep in
// the residual what was not sent).
//
// Per call, with x = g + e, S = sum of |x| over the finite x (exact, rounded
// to float64 and then to float32: S32):
//   p_i = min(1, (float(k) * |x_i|) / S32)  (float32; 0 for non-finite x_i)
//   u_i = word (i mod 4) of Philox4x32-10(counter {i/4, 0, step lo, step hi},
//         key {seed lo, seed hi}), top 24 bits times 2^-24
//   kept iff u_i < p_i; kept elements are sent unscaled in index order (the
//   first cap of them), their residual becomes +0; all others keep e = x.
//
// Passes (one wave per region of kRegion elements in the streaming ones):
//   k_rs_sample        (speculative calls) sums |x| over a fixed strided sample
//                      of chunks of 256 elements, one float64 per chunk
//   k_rs_sample_total  starts the call state; S_lo = 7/8 of n times the
//                      smallest of 16 group means of the sample: a likely
//                      lower bound of S, checked once S is known
//   k_rs_accum   x = g + e written into e; float64 sums of |x| per lane,
//                folded per block (12 B per element).  A speculative call
//                also draws u for every element and appends each element
//                that could be kept if S were S_lo to its region's slot of
//                kSlot (x, i) pairs, in index order
//   k_rs_total   sums the wave partials and certifies float32(S) from a
//                rigorous error bound; only when the bound straddles a
//                float32 rounding boundary (or on EF_FLAG_FORCE_FALLBACK)
//                do k_rs_exact / k_rs_exact_total re-read x and sum it
//                exactly with integer accumulators (4 B per element, rare)
//   The slots decide when the call was speculative, no slot overflowed and
//   S32 >= S_lo: correctly rounded division is monotone in the divisor, so
//   then every kept element is a candidate.  Otherwise (or on
//   EF_FLAG_FORCE_FALLBACK) the second pass runs:
//   k_rs_mark    reads x, draws u with one Philox call per 4 elements, writes
//                the keep bitmap and per-region counts (4 B + 1 bit per element)
//   k_rs_filter  (slots) the exact decision for each candidate: a 64-bit keep
//                mask and the kept count per region
//   k_rs_scan_tiles, k_excl_scan  region counts -> output offsets, the kept count
//   k_rs_write   per region, the kept elements (from the slot and its mask, or
//                from the bitmap) -> (x, i) at their index-ordered place,
//                e[i] = +0
// Each kernel reads the decision from the call state, so the path not taken
// costs one early exit per block.
// Every product, quotient and sum is rounded on its own (-ffp-contract=off,
// IEEE division, denormals kept).
#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace efg {
namespace rs {

// Shapes measured on MI355X (sweep over blocks 256-1024, regions 2048-8192,
// unrolls 4-16): the streaming passes work on regions of EFG_RS_REGION
// elements per wave; k_rs_accum issues EFG_RS_ACC_UNROLL float4 loads of g
// and of e at once, then draws their Philox words while the loads are in
// flight (the draws depend on the index only), then uses both.  Philox is 20
// 64-bit multiply-adds per 4 elements; hidden under the loads' latency that
// way, with 8 loads per array (150 VGPRs, 3 waves per SIMD), the pass costs
// 2.57 ms at N = 1.3e9 against 2.75 ms when each float4's draw followed its
// data (16 loads per array, 2 waves per SIMD; 16 with the draws first spills).
// Without the draws (calls that take the second pass) 16 loads per array stay
// best: EFG_RS_PLAIN_UNROLL.
#ifndef EFG_RS_BLOCK
#define EFG_RS_BLOCK 512
#endif
#ifndef EFG_RS_REGION
#define EFG_RS_REGION 4096
#endif
#ifndef EFG_RS_ACC_UNROLL
#define EFG_RS_ACC_UNROLL 8
#endif
#ifndef EFG_RS_PLAIN_UNROLL
#define EFG_RS_PLAIN_UNROLL 16
#endif
#ifndef EFG_RS_MARK_UNROLL
#define EFG_RS_MARK_UNROLL 4
#endif
constexpr int kBlock = EFG_RS_BLOCK;
constexpr int kWaves = kBlock / kWave;
constexpr int kRegion = EFG_RS_REGION;
constexpr int kUnroll = EFG_RS_ACC_UNROLL;         // k_rs_accum with the draws
constexpr int kPlainUnroll = EFG_RS_PLAIN_UNROLL;  // k_rs_accum without them
constexpr int kMarkUnroll = EFG_RS_MARK_UNROLL;
constexpr int kRegionWords = kRegion / 32;  // bitmap words per region
constexpr int kWordsPerLane = kRegionWords / kWave;
constexpr int kSlot = kWave;                // candidate entries per region: one per lane in k_rs_filter
static_assert(kRegion % 2048 == 0 && kRegion <= 8192,
              "a region is whole 32-bit words of 4-element lanes, 1 to 4 words per lane in k_rs_write");
static_assert(kRegion % (4 * kWave * kUnroll) == 0 && kRegion % (4 * kWave * kPlainUnroll) == 0 && kWaves <= 16 &&
                  kRegion / kWave / 4 <= 32,
              "the float64 error bound of k_rs_total counts at most 32 additions per lane accumulator, "
              "16 waves per block and 2^18 block partials");
static_assert(kRegionWords * 4 >= kSlot * 8, "a region's candidate slot fits in its bitmap slice");
constexpr int kLaneBlock = 256;    // threads of the one-lane-per-region filter
constexpr int kMaxBlocks = 4096;   // grid cap of the grid-stride region passes
constexpr int kTotalBlock = 1024;
constexpr int kExactWaves = 16384;  // grid of the exact-sum pass (grid-stride over regions)
constexpr int kExactBlock = 256;
constexpr int kBands = 8;  // exponent bands of 32 binades each
constexpr int kScanTile = 4 * kScanThreads;  // region counts per first-level scan block
// S_lo sample: chunks of 64 float4, at most kSampleMax of them, in
// kSampleGroups groups; calls with fewer than kSampleMin chunks, or with more
// than one kept element per kSpecRatio on average, take the two-pass path
constexpr int kSampleChunk = 4 * kWave;
constexpr int kSampleMax = 4096;
constexpr int kSampleMin = 256;
constexpr int kSampleGroups = 16;
constexpr int kSampleBlock = 256;
constexpr int64_t kSpecRatio = 512;
static_assert(kSampleGroups * kWave <= 1024 && kSampleMax % kSampleGroups == 0 && kSampleMin % kSampleGroups == 0,
              "one wave per sample group in k_rs_sample_total");

typedef float f4 __attribute__((ext_vector_type(4)));

struct State {
    double approx;      // float64 sum of the wave partials
    float s32;          // S32
    uint32_t uncertain; // 1: the exact pass decides S32
    uint32_t nonfinite; // non-finite x seen by k_rs_accum
    uint32_t kept;      // number kept (scan total)
    float slo;          // S_lo of a speculative call, 0 otherwise
    uint32_t overflow;  // 1: some candidate slot overflowed
    uint32_t pad[8];
};
static_assert(sizeof(State) == 64, "State is one 64-byte slot");

__device__ __forceinline__ bool finite(float x) { return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u; }

// The second pass is skipped iff this holds (read by every later kernel).
__device__ __forceinline__ bool use_slots(const State* st) {
    return st->slo > 0.0f && st->overflow == 0 && st->s32 >= st->slo;
}

__device__ __forceinline__ void start_state(State* st, float slo) {
    st->approx = 0.0;
    st->s32 = 0.0f;
    st->uncertain = 0;
    st->nonfinite = 0;
    st->kept = 0;
    st->slo = slo;
    st->overflow = 0;
}

__global__ void k_rs_init(State* st) { start_state(st, 0.0f); }

__device__ __forceinline__ double abs_finite(float x) { return finite(x) ? static_cast<double>(fabsf(x)) : 0.0; }

// Sample chunk j (of m) is chunk floor(j * nchunks / m) of the tensor's
// nchunks full chunks of kSampleChunk elements; one wave per chunk.
__global__ __launch_bounds__(kSampleBlock) void k_rs_sample(const float* __restrict__ g, const float* __restrict__ e,
                                                            int64_t nchunks, int32_t m, double* __restrict__ spart) {
    const int32_t j = static_cast<int32_t>(blockIdx.x) * (kSampleBlock / kWave) + threadIdx.x / kWave;
    if (j >= m) return;
    const int64_t c = static_cast<int64_t>(j) * nchunks / m;
    const int64_t i = c * kSampleChunk + 4 * lane();
    const f4 x = *reinterpret_cast<const f4*>(g + i) + *reinterpret_cast<const f4*>(e + i);
    double a = (abs_finite(x.x) + abs_finite(x.y)) + (abs_finite(x.z) + abs_finite(x.w));
    a = wave_sum(a);
    if (lane() == 0) spart[j] = a;
}

// S_lo from the chunk sums: wave q sums group q (m / kSampleGroups chunks).
// Any value is safe (the slots are checked against S32); a low one costs
// extra candidates, a high one the second pass.
__global__ __launch_bounds__(kSampleGroups * kWave) void k_rs_sample_total(const double* __restrict__ spart, int32_t m,
                                                                           int64_t n, State* __restrict__ st) {
    __shared__ double gsum[kSampleGroups];
    const int q = threadIdx.x / kWave;
    const int gs = m / kSampleGroups;
    double a = 0.0;
    for (int j = lane(); j < gs; j += kWave) a += spart[q * gs + j];
    a = wave_sum(a);
    if (lane() == 0) gsum[q] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        double mn = gsum[0];
        for (int i = 1; i < kSampleGroups; ++i) mn = fmin(mn, gsum[i]);
        const float slo = static_cast<float>(0.875 * static_cast<double>(n) * (mn / (static_cast<double>(gs) * kSampleChunk)));
        // the candidate test needs 1/S_lo as a normal float
        start_state(st, slo >= 0x1p-126f && slo <= 0x1p126f ? slo : 0.0f);
    }
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011) on counter c with key
// {k0, k1}; the key advances by the two Weyl constants after every round.
__device__ __forceinline__ void philox(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                       uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // one 32x32->64 product per multiplier (v_mad_u64_u32 gives both halves)
        const uint64_t p0 = static_cast<uint64_t>(c0) * 0xD2511F53u;
        const uint64_t p1 = static_cast<uint64_t>(c2) * 0xCD9E8D57u;
        const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = static_cast<uint32_t>(p1);
        c2 = n2;
        c3 = static_cast<uint32_t>(p0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// u for the 32-bit draw w: its top 24 bits times 2^-24
__device__ __forceinline__ float uniform24(uint32_t w) { return static_cast<float>(w >> 8) * 0x1p-24f; }

// Whether an element can be kept when S32 >= S_lo (rS = fl(1/S_lo), normal):
// fl(t * rS) is within a relative 2^-22 of fl(t / S_lo) >= fl(t / S32) when
// the quotient is normal, so the margin of 2^-20 keeps every such element; a
// draw u = 0 keeps any element with t > 0.  Over-inclusion only costs a slot.
__device__ __forceinline__ bool candidate(float x, float u, float kf, float rS) {
    if (!finite(x)) return false;
    const float t = kf * fabsf(x);
    if (u == 0.0f) return t > 0.0f;
    return u < (t * rS) * (1.0f + 0x1p-20f);
}

// Wave w owns elements [w*kRegion, min((w+1)*kRegion, n)).  Lane l of
// unroll step u holds float4 j = 64u + l of the region; a final partial
// float4 (only in the last region) is handled component by component.  Block
// b writes part[b], the sum of its waves' partials in wave order.  With SPEC
// (and S_lo set), the candidates of step u are appended to the region's slot
// after those of step u - 1, lanes in order, so the slot is in index order;
// ccnt[w] gets the slot's fill and st->overflow is raised past kSlot.
template <bool SPEC>
__global__ __launch_bounds__(kBlock) void k_rs_accum(const float* __restrict__ g, float* __restrict__ e, int64_t n,
                                                     double* __restrict__ part, State* __restrict__ st, float kf,
                                                     uint32_t key0, uint32_t key1, uint32_t step0, uint32_t step1,
                                                     uint2* __restrict__ slots, uint32_t* __restrict__ ccnt) {
    __shared__ double lsum[kWaves];
    __shared__ uint32_t lnf[kWaves];
    const int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int64_t beg = w * kRegion;
    const int l = lane();
    // four sequential float64 accumulators per lane: at most 32 additions each
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    uint32_t nf = 0;
    if (beg < n) {
        const float slo = SPEC ? st->slo : 0.0f;
        const bool spec = SPEC && slo > 0.0f;
        const float rS = spec ? 1.0f / slo : 0.0f;
        const uint32_t q0 = static_cast<uint32_t>(beg >> 2);
        uint2* slot = slots + w * kSlot;
        uint32_t cnt = 0;
        const int64_t len = min(static_cast<int64_t>(kRegion), n - beg);
        const int64_t nfull = len >> 2;
        const int64_t nv = (len + 3) >> 2;
        const f4* g4 = reinterpret_cast<const f4*>(g + beg);
        f4* e4 = reinterpret_cast<f4*>(e + beg);
        auto account = [&](double& a, float x) {
            if (finite(x)) a += static_cast<double>(fabsf(x));
            else ++nf;
        };
        auto iteration = [&](int64_t base, auto guard) {
            constexpr bool GUARD = decltype(guard)::value;
            constexpr int kU = SPEC ? kUnroll : kPlainUnroll;
            f4 gv[kU], ev[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t j = base + u * kWave + l;
                if (!GUARD || j < nfull) {
                    gv[u] = __builtin_nontemporal_load(g4 + j);
                    ev[u] = __builtin_nontemporal_load(e4 + j);
                }
            }
            // the draws depend on the index only: computed while the loads are in flight
            uint32_t pw[kU][4];
            if (spec) {
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    uint32_t c0 = q0 + static_cast<uint32_t>(base + u * kWave + l), c1 = 0u, c2 = step0, c3 = step1;
                    philox(c0, c1, c2, c3, key0, key1);
                    pw[u][0] = c0;
                    pw[u][1] = c1;
                    pw[u][2] = c2;
                    pw[u][3] = c3;
                }
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t j = base + u * kWave + l;
                f4 x = f4{0.f, 0.f, 0.f, 0.f};
                int valid = 4;  // components of this float4 inside the tensor
                if (!GUARD || j < nfull) {
                    x = gv[u] + ev[u];
                    __builtin_nontemporal_store(x, e4 + j);
                    account(a0, x.x);
                    account(a1, x.y);
                    account(a2, x.z);
                    account(a3, x.w);
                } else if (GUARD && j == nfull && nfull < nv) {
                    const int64_t i = beg + 4 * nfull;
                    valid = static_cast<int>(len - 4 * nfull);  // 1..3
                    x.x = g[i] + e[i];
                    e[i] = x.x;
                    account(a0, x.x);
                    if (valid > 1) {
                        x.y = g[i + 1] + e[i + 1];
                        e[i + 1] = x.y;
                        account(a1, x.y);
                    }
                    if (valid > 2) {
                        x.z = g[i + 2] + e[i + 2];
                        e[i + 2] = x.z;
                        account(a2, x.z);
                    }
                } else {
                    valid = 0;
                }
                if (spec) {
                    const float xs[4] = {x.x, x.y, x.z, x.w};
                    const uint32_t ws[4] = {pw[u][0], pw[u][1], pw[u][2], pw[u][3]};
                    bool hit[4];
                    uint64_t bal[4], any = 0;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        hit[t] = t < valid && candidate(xs[t], uniform24(ws[t]), kf, rS);
                        bal[t] = __ballot(hit[t]);
                        any |= bal[t];
                    }
                    if (any) {
                        // lane l's candidates follow those of lanes below l
                        uint32_t pos = cnt, tot = 0;
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            pos += count_below(bal[t]);
                            tot += popc64(bal[t]);
                        }
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            if (hit[t]) {
                                if (pos < kSlot)
                                    slot[pos] = make_uint2(__float_as_uint(xs[t]),
                                                           static_cast<uint32_t>(beg + 4 * j + t));
                                ++pos;
                            }
                        }
                        cnt += tot;
                    }
                }
            }
        };
        constexpr int64_t kStep = kWave * (SPEC ? kUnroll : kPlainUnroll);
        int64_t base = 0;
        for (; base + kStep <= nfull; base += kStep) iteration(base, std::false_type{});
        if (base < nv) iteration(base, std::true_type{});
        if (spec && l == 0) {
            ccnt[w] = cnt < kSlot ? cnt : kSlot;
            if (cnt > kSlot) atomicOr(&st->overflow, 1u);
        }
    }
    double a = (a0 + a1) + (a2 + a3);
    a = wave_sum(a);
    nf = wave_sum(nf);
    if (l == 0) {
        lsum[threadIdx.x / kWave] = a;
        lnf[threadIdx.x / kWave] = nf;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        uint32_t c = 0;
        for (int i = 0; i < kWaves; ++i) {
            t += lsum[i];
            c += lnf[i];
        }
        part[blockIdx.x] = t;
        if (c) atomicAdd(&st->nonfinite, c);
    }
}

// Sum of the block partials and the certified float32 rounding of the exact
// sum.  Every partial and sum is a sum of non-negative float64 values; along
// any path of the summation tree there are at most 32 + 2 (lane) + 6 (wave)
// + 16 (block of <= 16 waves) + 256 (thread's share of <= 2^18 partials) + 2
// + 6 + 16 (final block) = 336 additions,
// so the computed total t is within a relative 340 * 2^-53 < 2^-44 of the exact
// sum S (Higham, Accuracy and Stability of Numerical Algorithms, section 4.2).
// lo = t(1 - 2^-40) and hi = t(1 + 2^-40), each rounded once, then bracket S,
// and rounding to float64 then float32 is monotone: when lo and hi give the
// same float32 so does S.  Otherwise the exact pass decides.
__global__ __launch_bounds__(kTotalBlock) void k_rs_total(const double* __restrict__ part, int64_t np,
                                                          uint32_t force_exact, State* __restrict__ st,
                                                          float* __restrict__ sum_out,
                                                          uint32_t* __restrict__ nonfinite) {
    __shared__ double lsum[kTotalBlock / kWave];
    // four independent chains per thread keep four loads in flight
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    int64_t w = threadIdx.x;
    for (; w + 3 * kTotalBlock < np; w += 4 * kTotalBlock) {
        a0 += part[w];
        a1 += part[w + kTotalBlock];
        a2 += part[w + 2 * kTotalBlock];
        a3 += part[w + 3 * kTotalBlock];
    }
    for (; w < np; w += kTotalBlock) a0 += part[w];
    double a = (a0 + a1) + (a2 + a3);
    a = wave_sum(a);
    if (lane() == 0) lsum[threadIdx.x / kWave] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int i = 0; i < kTotalBlock / kWave; ++i) t += lsum[i];
        const double lo = t * (1.0 - 0x1p-40);
        const double hi = t * (1.0 + 0x1p-40);
        const float flo = static_cast<float>(lo), fhi = static_cast<float>(hi);
        const uint32_t unc = force_exact || __float_as_uint(flo) != __float_as_uint(fhi);
        st->approx = t;
        st->s32 = flo;
        st->uncertain = unc;
        if (sum_out) *sum_out = flo;
        if (nonfinite) *nonfinite = st->nonfinite;
    }
}

// Exact sum of |x| over the finite x, used when k_rs_total could not certify
// float32(S).  A finite float32 magnitude is M * 2^s * 2^-149 with an integer
// M < 2^24 and s = max(biased exponent, 1) - 1 in [0, 253]; band b = s / 32
// gathers M << (s mod 32) (< 2^55).  Each lane owns one uint64 per band in
// LDS and adds into it with non-returning LDS atomics (one per element, no
// band select in registers); after each region (64 elements per lane, so no
// band exceeds 2^61) the lane folds its bands into 32-bit halves summed in
// uint64 registers and clears them.  Wave w writes 16 uint64 (band b:
// low-half sum, high-half sum) to xpart[16 w ..].
__global__ __launch_bounds__(kExactBlock) void k_rs_exact(const float* __restrict__ x, int64_t n, int64_t nw,
                                                          const State* __restrict__ st,
                                                          uint64_t* __restrict__ xpart) {
    if (!st->uncertain) return;
    __shared__ unsigned long long lacc[kExactBlock / kWave][kBands][kWave];
    const int wv = threadIdx.x / kWave;
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * (kExactBlock / kWave) + wv;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * (kExactBlock / kWave);
    const int l = lane();
    uint64_t wlo[kBands], whi[kBands];
#pragma unroll
    for (int b = 0; b < kBands; ++b) {
        wlo[b] = whi[b] = 0;
        lacc[wv][b][l] = 0;
    }
    auto add = [&](float v) {
        const uint32_t u = __float_as_uint(v) & 0x7fffffffu;
        const uint32_t ex = u >> 23;
        if (ex == 0xffu) return;
        const uint32_t s = ex ? ex - 1 : 0;
        const unsigned long long m = static_cast<unsigned long long>((u & 0x7fffffu) | (ex ? 0x800000u : 0u))
                                     << (s & 31u);
        atomicAdd(&lacc[wv][s >> 5][l], m);
    };
    constexpr int kVec = kRegion / 4 / kWave;  // float4 per lane and region
    for (int64_t r = w0; r < nw; r += stride) {
        const int64_t beg = r * kRegion;
        const int64_t len = min(static_cast<int64_t>(kRegion), n - beg);
        const int64_t nfull = len >> 2;
        const f4* x4 = reinterpret_cast<const f4*>(x + beg);
        f4 v[kVec];
#pragma unroll
        for (int u = 0; u < kVec; ++u) {
            const int64_t j = u * kWave + l;
            v[u] = j < nfull ? __builtin_nontemporal_load(x4 + j) : f4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kVec; ++u) {
            add(v[u].x);
            add(v[u].y);
            add(v[u].z);
            add(v[u].w);
        }
        if (l < len - 4 * nfull) add(x[beg + 4 * nfull + l]);  // at most 3 trailing elements
#pragma unroll
        for (int b = 0; b < kBands; ++b) {
            const unsigned long long a = lacc[wv][b][l];
            lacc[wv][b][l] = 0;
            wlo[b] += a & 0xffffffffull;
            whi[b] += a >> 32;
        }
    }
#pragma unroll
    for (int b = 0; b < kBands; ++b) {
        wlo[b] = wave_sum(wlo[b]);
        whi[b] = wave_sum(whi[b]);
    }
    if (l == 0) {
#pragma unroll
        for (int b = 0; b < kBands; ++b) {
            xpart[16 * w0 + 2 * b] = wlo[b];
            xpart[16 * w0 + 2 * b + 1] = whi[b];
        }
    }
}

// Bits [p, p + 64) of the integer held in 32-bit limbs L[0..nl) (bits below
// 0 read as zero); *below gets whether any bit under p is set.
__device__ uint64_t window64(const uint64_t* L, int nl, int p, bool* below) {
    uint64_t r = 0;
    bool any = false;
    for (int j = 0; j < nl; ++j) {
        const int sh = 32 * j - p;  // where limb bit 0 lands in the window
        if (sh <= -32) {
            any |= L[j] != 0;
        } else if (sh < 0) {
            r |= L[j] >> (-sh);
            any |= (L[j] & ((1ull << (-sh)) - 1)) != 0;
        } else if (sh < 64) {
            r |= L[j] << sh;
        }
    }
    *below = any;
    return r;
}

// Totals the exact band sums and rounds them to float64 (nearest, ties to
// even), then to float32.
constexpr int kLimbs = 12;
__global__ __launch_bounds__(16 * kWave) void k_rs_exact_total(const uint64_t* __restrict__ xpart, int64_t nwx,
                                                               State* __restrict__ st, float* __restrict__ sum_out) {
    if (!st->uncertain) return;
    __shared__ uint64_t tot[16];
    {
        // wave q sums column q of the wave partials
        const int q = threadIdx.x / kWave;
        uint64_t a = 0;
        for (int64_t w = lane(); w < nwx; w += kWave) a += xpart[16 * w + q];
        a = wave_sum(a);
        if (lane() == 0) tot[q] = a;
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    // band b is (lo + hi * 2^32) * 2^(32 b) in units of 2^-149
    uint64_t L[kLimbs];
    for (int j = 0; j < kLimbs; ++j) L[j] = 0;
    for (int b = 0; b < kBands; ++b) {
        L[b] += tot[2 * b];
        L[b + 1] += tot[2 * b + 1];
    }
    for (int j = 0; j + 1 < kLimbs; ++j) {
        L[j + 1] += L[j] >> 32;
        L[j] &= 0xffffffffull;
    }
    int top = -1;
    for (int j = kLimbs - 1; j >= 0; --j) {
        if (L[j]) {
            top = 32 * j + 63 - __clzll(L[j]);
            break;
        }
    }
    double S = 0.0;
    if (top >= 0) {
        bool below = false;
        const uint64_t W = window64(L, kLimbs, top - 63, &below);  // bit 63 of W is the leading bit
        if (top < 53) {
            S = ldexp(static_cast<double>(W >> (63 - top)), -149);  // every bit fits: exact
        } else {
            uint64_t mant = W >> 11;
            const bool guard = (W >> 10) & 1u;
            const bool sticky = below || (W & 0x3ffull) != 0;
            if (guard && (sticky || (mant & 1u))) ++mant;
            S = ldexp(static_cast<double>(mant), top - 52 - 149);
        }
    }
    st->approx = S;
    st->s32 = static_cast<float>(S);
    if (sum_out) *sum_out = st->s32;
}

// The decision u < min(1, fl(t / S)) with t = fl(k |x|), for the four
// elements of one float4.  When rS = fl(1/S) is a normal float (fast),
// pa = fl(t * rS) is within a relative 2^-22 of the correctly rounded quotient
// whenever u is a positive draw (u >= 2^-24, so only quotients in the normal
// range matter): u < pa (1 - 2^-20) proves u < quotient and u >= pa (1 + 2^-20)
// proves the opposite, each product rounded once.  Draws within that margin,
// u = 0 and every element of a non-fast call take the correctly rounded
// division (rare: the branch is skipped when no lane of the wave needs it).
// The clip at 1 never changes the outcome (u < 1).
__device__ __forceinline__ uint32_t keep_nibble(const float (&x)[4], const uint32_t (&word)[4], float kf, float S,
                                                float rS, bool fast) {
    uint32_t nib = 0, unsure = 0;
    float t[4], u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        t[i] = kf * fabsf(x[i]);
        u[i] = static_cast<float>(word[i] >> 8) * 0x1p-24f;
        const float pa = t[i] * rS;
        const bool ok = finite(x[i]);
        const bool yes = fast && u[i] > 0.0f && u[i] < pa * (1.0f - 0x1p-20f);
        const bool no = fast && u[i] > 0.0f && u[i] >= pa * (1.0f + 0x1p-20f);
        nib |= (ok && yes ? 1u : 0u) << i;
        unsure |= (ok && !yes && !no ? 1u : 0u) << i;
    }
    if (unsure) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if ((unsure >> i) & 1u) {
                float p = t[i] / S;
                if (p > 1.0f) p = 1.0f;
                nib |= (u[i] < p ? 1u : 0u) << i;
            }
        }
    }
    return nib;
}

__device__ __forceinline__ void mark_region(const float* __restrict__ x, int64_t n, int64_t w, float kf,
                                            uint32_t key0, uint32_t key1, uint32_t step0, uint32_t step1, float S,
                                            float rS, bool fast, uint32_t* __restrict__ bm,
                                            uint32_t* __restrict__ cnt, int l) {
    const int64_t beg = w * kRegion;
    const int64_t len = min(static_cast<int64_t>(kRegion), n - beg);
    const int64_t nfull = len >> 2;
    const int64_t nv = (len + 3) >> 2;
    const f4* x4 = reinterpret_cast<const f4*>(x + beg);
    uint32_t* bw = bm + (beg >> 5);
    const uint32_t q0 = static_cast<uint32_t>(beg >> 2);
    uint32_t count = 0;
    auto iteration = [&](int64_t base, auto guard) {
        constexpr bool GUARD = decltype(guard)::value;
        f4 xv[kMarkUnroll];
#pragma unroll
        for (int u = 0; u < kMarkUnroll; ++u) {
            const int64_t j = base + u * kWave + l;
            if (!GUARD || j < nfull) {
                xv[u] = __builtin_nontemporal_load(x4 + j);
            } else {
                xv[u] = f4{0.f, 0.f, 0.f, 0.f};
                if (j == nfull) {
                    const int64_t rem = len - 4 * nfull;  // 0..3 valid components
                    if (rem > 0) xv[u].x = x[beg + 4 * nfull];
                    if (rem > 1) xv[u].y = x[beg + 4 * nfull + 1];
                    if (rem > 2) xv[u].z = x[beg + 4 * nfull + 2];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kMarkUnroll; ++u) {
            const int64_t j = base + u * kWave + l;
            uint32_t c0 = q0 + static_cast<uint32_t>(j), c1 = 0u, c2 = step0, c3 = step1;
            philox(c0, c1, c2, c3, key0, key1);
            const float xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
            const uint32_t ws[4] = {c0, c1, c2, c3};
            uint32_t nib = keep_nibble(xs, ws, kf, S, rS, fast);
            if (GUARD && j >= nv) nib = 0;  // zero-filled components of a partial float4 have p = 0 anyway
            count += __popc(nib);
            uint32_t word = nib << (4 * (l & 7));
            word |= __shfl_xor(word, 1, kWave);
            word |= __shfl_xor(word, 2, kWave);
            word |= __shfl_xor(word, 4, kWave);
            const int64_t j8 = base + u * kWave + (l & ~7);  // first float4 of this word
            if ((l & 7) == 0 && (!GUARD || j8 < nv)) bw[j8 >> 3] = word;
        }
    };
    constexpr int64_t kStep = kWave * kMarkUnroll;
    int64_t base = 0;
    for (; base + kStep <= nfull; base += kStep) iteration(base, std::false_type{});
    if (base < nv) iteration(base, std::true_type{});
    count = wave_sum(count);
    if (l == 0) cnt[w] = count;
}

// Decisions for the regions of wave w (grid-stride).  Lane l of unroll step u
// holds float4 j (elements 4j..4j+3 of the region, one Philox call); eight
// neighbouring lanes OR their nibbles into one 32-bit bitmap word (bit i mod 32
// of word i / 32).
__global__ __launch_bounds__(kBlock) void k_rs_mark(const float* __restrict__ x, int64_t n, float kf, uint32_t key0,
                                                    uint32_t key1, uint32_t step0, uint32_t step1,
                                                    const State* __restrict__ st, uint32_t* __restrict__ bm,
                                                    uint32_t* __restrict__ cnt) {
    if (use_slots(st)) return;
    const int l = lane();
    const float S = st->s32;
    const float rS = 1.0f / S;
    // 1/S normal: S in [2^-126, 2^126]
    const bool fast = S >= 0x1p-126f && S <= 0x1p126f;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
    for (int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / kWave; w * kRegion < n; w += stride)
        mark_region(x, n, w, kf, key0, key1, step0, step1, S, rS, fast, bm, cnt, l);
}

// One lane per region r: the exact decision for each of its ccnt[r]
// candidates; kmask[r] gets the kept slot entries, cnt[r] their number.
constexpr int kFilterBatch = 8;  // candidates of a region whose slot entries are read at once
__global__ __launch_bounds__(kLaneBlock) void k_rs_filter(const uint2* __restrict__ slots,
                                                          const uint32_t* __restrict__ ccnt, int64_t nw, float kf,
                                                          uint32_t key0, uint32_t key1, uint32_t step0,
                                                          uint32_t step1, const State* __restrict__ st,
                                                          uint64_t* __restrict__ kmask, uint32_t* __restrict__ cnt) {
    if (!use_slots(st)) return;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kLaneBlock + threadIdx.x;
    if (r >= nw) return;
    const float S = st->s32;
    const uint32_t c = ccnt[r];
    const uint2* sl = slots + r * kSlot;
    uint64_t m = 0;
    for (uint32_t j0 = 0; j0 < c; j0 += kFilterBatch) {
        // all loads issued before any is used: past the count reads the last candidate
        uint2 v[kFilterBatch];
#pragma unroll
        for (int t = 0; t < kFilterBatch; ++t) v[t] = sl[min(j0 + t, c - 1)];
#pragma unroll
        for (int t = 0; t < kFilterBatch; ++t) {
            if (j0 + t < c) {
                const uint32_t i = v[t].y;
                uint32_t c0 = i >> 2, c1 = 0u, c2 = step0, c3 = step1;
                philox(c0, c1, c2, c3, key0, key1);
                const uint32_t q = i & 3u;
                const uint32_t word = q == 0 ? c0 : q == 1 ? c1 : q == 2 ? c2 : c3;
                float p = (kf * fabsf(__uint_as_float(v[t].x))) / S;
                if (p > 1.0f) p = 1.0f;
                if (uniform24(word) < p) m |= 1ull << (j0 + t);
            }
        }
    }
    kmask[r] = m;
    cnt[r] = popc64(m);
}

// Kept elements -> output slots (region start) + rank; slots below cap get
// (x, i) and e[i] = +0.  When the candidate slots decide, one lane per region
// walks its keep mask; otherwise one wave per region reads its bitmap words
// (kWordsPerLane per lane, in order).  Both grid-stride.
constexpr int kWriteBatch = 4;  // kept entries of a region whose slot entries are read at once
__global__ __launch_bounds__(kBlock) void k_rs_write(float* __restrict__ e, int64_t n, int64_t nw,
                                                     const uint32_t* __restrict__ bm, const uint2* __restrict__ slots,
                                                     const uint64_t* __restrict__ kmask,
                                                     const uint32_t* __restrict__ off,
                                                     const uint32_t* __restrict__ tsum,
                                                     const State* __restrict__ st, float* __restrict__ vals,
                                                     int32_t* __restrict__ idx, int64_t cap) {
    if (use_slots(st)) {
        const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
        for (int64_t r = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; r < nw; r += stride) {
            uint64_t m = kmask[r];
            if (!m) continue;
            int64_t pos = off[r] + tsum[r / kScanTile];
            const uint2* sl = slots + r * kSlot;
            while (m && pos < cap) {
                // the next kWriteBatch kept entries' slot reads go out together;
                // past the last kept one, the first is read again and not used
                uint2 c[kWriteBatch];
                uint64_t mm = m;
                const int first = __ffsll(static_cast<unsigned long long>(m)) - 1;
#pragma unroll
                for (int t = 0; t < kWriteBatch; ++t) {
                    c[t] = sl[mm ? __ffsll(static_cast<unsigned long long>(mm)) - 1 : first];
                    mm &= mm - 1;
                }
#pragma unroll
                for (int t = 0; t < kWriteBatch; ++t) {
                    if (m && pos < cap) {
                        vals[pos] = __uint_as_float(c[t].x);
                        idx[pos] = static_cast<int32_t>(c[t].y);
                        e[c[t].y] = 0.0f;
                        m &= m - 1;
                        ++pos;
                    }
                }
            }
        }
        return;
    }
    const int l = lane();
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
    for (int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / kWave; w < nw; w += stride) {
        const int64_t beg = w * kRegion;
        const uint32_t o = off[w] + tsum[w / kScanTile];
        const uint32_t o_next = w + 1 < nw ? off[w + 1] + tsum[(w + 1) / kScanTile] : st->kept;
        if (o_next == o || static_cast<int64_t>(o) >= cap) continue;
        const int64_t len = min(static_cast<int64_t>(kRegion), n - beg);
        const int64_t nwords = (len + 31) >> 5;
        const uint32_t* bw = bm + (beg >> 5);
        uint32_t wd[kWordsPerLane];
        uint32_t c = 0;
#pragma unroll
        for (int q = 0; q < kWordsPerLane; ++q) {
            const int64_t wi = kWordsPerLane * l + q;
            wd[q] = wi < nwords ? bw[wi] : 0u;
            c += __popc(wd[q]);
        }
        int64_t pos = static_cast<int64_t>(o) + (wave_incl_scan(c) - c);
#pragma unroll
        for (int q = 0; q < kWordsPerLane; ++q) {
            uint32_t v = wd[q];
            while (v) {
                const int b = __ffs(v) - 1;
                v &= v - 1;
                if (pos < cap) {
                    const int64_t i = beg + 32 * (kWordsPerLane * l + q) + b;
                    vals[pos] = e[i];
                    idx[pos] = static_cast<int32_t>(i);
                    e[i] = 0.0f;
                }
                ++pos;
            }
        }
    }
}

// First level of the region-count scan: block t scans counts
// [t*kScanTile, (t+1)*kScanTile) in place (exclusive) and writes its total to
// tsum[t]; k_excl_scan then scans tsum, and region w starts at
// cnt[w] + tsum[w / kScanTile].
__global__ __launch_bounds__(kScanThreads) void k_rs_scan_tiles(uint32_t* __restrict__ cnt, int64_t nw,
                                                                uint32_t* __restrict__ tsum) {
    __shared__ uint32_t lds[kScanThreads / kWave + 1];
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kScanTile + 4 * threadIdx.x;
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = t0 + q < nw ? cnt[t0 + q] : 0u;
    uint32_t total;
    uint32_t run = block_excl_scan<kScanThreads>(v[0] + v[1] + v[2] + v[3], lds, &total);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (t0 + q < nw) cnt[t0 + q] = run;
        run += v[q];
    }
    if (threadIdx.x == 0) tsum[blockIdx.x] = total;
}

__global__ void k_rs_empty(int64_t* count_out, float* sum_out, uint32_t* nonfinite) {
    *count_out = 0;
    if (sum_out) *sum_out = 0.0f;
    if (nonfinite) *nonfinite = 0;
}

struct Layout {
    int64_t nw, nb, ntiles;  // regions, accumulation blocks, scan tiles
    int64_t nchunks;         // full sample chunks
    int32_t m;               // sample chunks (0: the call is not speculative)
    size_t state, part, cnt, ccnt, kmask, tsum, xpart, spart, bm, total;
};

// The slots of a speculative call and the bitmap of the second pass share
// memory: the bitmap is written only when the slots were given up.
inline Layout layout_for(int64_t n) {
    Layout L{};
    L.nw = std::max<int64_t>(1, cdiv(n, kRegion));
    L.nb = std::max<int64_t>(1, cdiv(n, static_cast<int64_t>(kRegion) * kWaves));
    L.ntiles = cdiv(L.nw, kScanTile);
    L.nchunks = n / kSampleChunk;
    L.m = L.nchunks < kSampleMin ? 0
                                 : static_cast<int32_t>(std::min<int64_t>(kSampleMax, L.nchunks) / kSampleGroups *
                                                        kSampleGroups);
    size_t o = 0;
    L.state = o;
    o += 256;
    L.part = o;
    o = round_up(o + static_cast<size_t>(L.nb) * sizeof(double), 256);
    L.cnt = o;
    o = round_up(o + static_cast<size_t>(L.nw) * sizeof(uint32_t), 256);
    L.ccnt = o;
    o = round_up(o + static_cast<size_t>(L.nw) * sizeof(uint32_t), 256);
    L.kmask = o;
    o = round_up(o + static_cast<size_t>(L.nw) * sizeof(uint64_t), 256);
    L.tsum = o;
    o = round_up(o + static_cast<size_t>(L.ntiles) * sizeof(uint32_t), 256);
    L.xpart = o;
    o = round_up(o + static_cast<size_t>(kExactWaves) * 16 * sizeof(uint64_t), 256);
    L.spart = o;
    o = round_up(o + static_cast<size_t>(kSampleMax) * sizeof(double), 256);
    L.bm = o;
    o = round_up(o + static_cast<size_t>(L.nw) * kRegionWords * sizeof(uint32_t), 256);
    L.total = o;
    return L;
}

}  // namespace rs
}  // namespace efg

using namespace efg;

extern "C" size_t ef_random_sparsify_workspace_bytes(int64_t n) {
    if (n < 0 || n > kMaxElems) return 0;
    return rs::layout_for(n).total;
}

extern "C" int ef_random_sparsify(const float* g, float* e, int64_t n, int64_t k, uint64_t seed, uint64_t step,
                                  float* vals, int32_t* idx, int64_t cap, int64_t* count_out, float* sum_out,
                                  uint32_t* nonfinite, void* ws, size_t ws_bytes, uint32_t flags, void* stream) {
    if (n < 0 || n > kMaxElems) return fail(EF_EINVAL, "n=%lld outside [0, 2^31-1]", (long long)n);
    if (k < 0 || k > kMaxElems) return fail(EF_EINVAL, "k=%lld outside [0, 2^31-1]", (long long)k);
    if (cap < 0) return fail(EF_EINVAL, "cap must be >= 0");
    if (flags & ~EF_FLAG_FORCE_FALLBACK) return fail(EF_EINVAL, "unknown flags 0x%x", flags);
    if (!count_out) return fail(EF_EINVAL, "count_out must not be NULL");
    if (n > 0 && (!g || !e)) return fail(EF_EINVAL, "g and e must not be NULL");
    if (n > 0 && (!aligned16(g) || !aligned16(e))) return fail(EF_EINVAL, "g and e must be 16-byte aligned");
    if (cap > 0 && (!vals || !idx)) return fail(EF_EINVAL, "vals and idx must not be NULL when cap > 0");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 0) return launch("rs_empty", rs::k_rs_empty, dim3(1), dim3(1), s, count_out, sum_out, nonfinite);
    const rs::Layout L = rs::layout_for(n);
    if (!ws || ws_bytes < L.total)
        return fail(EF_EWS, "ef_random_sparsify: needs %zu bytes of workspace", L.total);
    if (!aligned256(ws)) return fail(EF_EINVAL, "workspace must be 256-byte aligned");
    uint8_t* base = static_cast<uint8_t*>(ws);
    rs::State* st = reinterpret_cast<rs::State*>(base + L.state);
    double* part = reinterpret_cast<double*>(base + L.part);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(base + L.cnt);
    uint32_t* ccnt = reinterpret_cast<uint32_t*>(base + L.ccnt);
    uint64_t* kmask = reinterpret_cast<uint64_t*>(base + L.kmask);
    uint32_t* tsum = reinterpret_cast<uint32_t*>(base + L.tsum);
    uint64_t* xpart = reinterpret_cast<uint64_t*>(base + L.xpart);
    double* spart = reinterpret_cast<double*>(base + L.spart);
    uint32_t* bm = reinterpret_cast<uint32_t*>(base + L.bm);
    uint2* slots = reinterpret_cast<uint2*>(base + L.bm);
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(cdiv(L.nw, rs::kWaves), rs::kMaxBlocks));
    const unsigned agrid = static_cast<unsigned>(L.nb);
    const unsigned xgrid =
        static_cast<unsigned>(cdiv(std::min<int64_t>(rs::kExactWaves, L.nw), rs::kExactBlock / kWave));
    const int64_t nwx = static_cast<int64_t>(xgrid) * (rs::kExactBlock / kWave);
    const float kf = static_cast<float>(k);
    const uint32_t key0 = static_cast<uint32_t>(seed), key1 = static_cast<uint32_t>(seed >> 32);
    const uint32_t step0 = static_cast<uint32_t>(step), step1 = static_cast<uint32_t>(step >> 32);
    // speculative: enough elements to sample, few kept per region on average
    const bool spec = !(flags & EF_FLAG_FORCE_FALLBACK) && L.m > 0 && k <= n / rs::kSpecRatio;
    if (spec) {
        EF_TRY(launch("rs_sample", rs::k_rs_sample, dim3(static_cast<unsigned>(cdiv(L.m, rs::kSampleBlock / kWave))),
                      dim3(rs::kSampleBlock), s, g, static_cast<const float*>(e), L.nchunks, L.m, spart));
        EF_TRY(launch("rs_sample_total", rs::k_rs_sample_total, dim3(1), dim3(rs::kSampleGroups * kWave), s,
                      static_cast<const double*>(spart), L.m, n, st));
        EF_TRY(launch("rs_accum", rs::k_rs_accum<true>, dim3(agrid), dim3(rs::kBlock), s, g, e, n, part, st, kf,
                      key0, key1, step0, step1, slots, ccnt));
    } else {
        EF_TRY(launch("rs_init", rs::k_rs_init, dim3(1), dim3(1), s, st));
        EF_TRY(launch("rs_accum", rs::k_rs_accum<false>, dim3(agrid), dim3(rs::kBlock), s, g, e, n, part, st, kf,
                      key0, key1, step0, step1, slots, ccnt));
    }
    EF_TRY(launch("rs_total", rs::k_rs_total, dim3(1), dim3(rs::kTotalBlock), s, static_cast<const double*>(part),
                  L.nb, static_cast<uint32_t>(flags & EF_FLAG_FORCE_FALLBACK), st, sum_out, nonfinite));
    EF_TRY(launch("rs_exact", rs::k_rs_exact, dim3(xgrid), dim3(rs::kExactBlock), s, static_cast<const float*>(e), n,
                  L.nw, static_cast<const rs::State*>(st), xpart));
    EF_TRY(launch("rs_exact_total", rs::k_rs_exact_total, dim3(1), dim3(16 * kWave), s,
                  static_cast<const uint64_t*>(xpart), nwx, st, sum_out));
    EF_TRY(launch("rs_mark", rs::k_rs_mark, dim3(grid), dim3(rs::kBlock), s, static_cast<const float*>(e), n, kf,
                  key0, key1, step0, step1, static_cast<const rs::State*>(st), bm, cnt));
    if (spec)
        EF_TRY(launch("rs_filter", rs::k_rs_filter, dim3(static_cast<unsigned>(cdiv(L.nw, rs::kLaneBlock))),
                      dim3(rs::kLaneBlock), s,
                      static_cast<const uint2*>(slots), static_cast<const uint32_t*>(ccnt), L.nw, kf, key0, key1,
                      step0, step1, static_cast<const rs::State*>(st), kmask, cnt));
    EF_TRY(launch("rs_scan_tiles", rs::k_rs_scan_tiles, dim3(static_cast<unsigned>(L.ntiles)), dim3(kScanThreads), s,
                  cnt, L.nw, tsum));
    EF_TRY(launch("rs_scan", k_excl_scan<uint32_t>, dim3(1), dim3(kScanThreads), s, tsum, L.ntiles, &st->kept,
                  count_out));
    return launch("rs_write", rs::k_rs_write, dim3(grid), dim3(rs::kBlock), s, e, n, L.nw,
                  static_cast<const uint32_t*>(bm), static_cast<const uint2*>(slots),
                  static_cast<const uint64_t*>(kmask), static_cast<const uint32_t*>(cnt),
                  static_cast<const uint32_t*>(tsum), static_cast<const rs::State*>(st), vals, idx, cap);
}
