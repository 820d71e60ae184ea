// 1-bit sign compression with averaged error feedback and momentum, gfx950.
//
// "1-bit Adam" page, sections 2.1 (sign quantisation, quantisation error and
// its averaged error buffer), 2.2 (momentum on the quantised gradient) and 3.2
// (clip before quantisation, NaN check after the error update, int8 storage);
// section 1 (32 bits -> 1 bit per element).
//
// One streaming pass, one wave per contiguous region: each lane handles one
// float4 of g, e and m per unroll step (128-bit non-temporal loads and
// stores), writes its four int8 signs as one 32-bit store, and pairs with its
// neighbour lane to form one byte of packed bits.  21.125 bytes move per
// element with both optional outputs (read g, e, m; write e, m, int8, 1 bit);
// 13.125 when m is NULL (compress only, the momentum follows the exchange).
// Every product and sum is rounded on its own: the library is compiled with
// -ffp-contract=off.
#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace efg {
namespace sign {

// Shape of the streaming kernel, measured on MI355X (fastest of a sweep over
// regions 2048-16384, unroll 2-16, blocks 256-1024): one wave per region of EFG_SIGN_REGION
// elements, EFG_SIGN_UNROLL float4 of each of g, e, m in flight per lane.
#ifndef EFG_SIGN_BLOCK
#define EFG_SIGN_BLOCK 512
#endif
#ifndef EFG_SIGN_REGION
#define EFG_SIGN_REGION 8192
#endif
#ifndef EFG_SIGN_UNROLL
#define EFG_SIGN_UNROLL 16
#endif
constexpr int kBlock = EFG_SIGN_BLOCK;
constexpr int kWaves = kBlock / kWave;
constexpr int kRegion = EFG_SIGN_REGION;  // multiple of 8 * 64
constexpr int kUnroll = EFG_SIGN_UNROLL;
static_assert(kRegion % 512 == 0, "regions must hold whole 8-element groups per lane pair");

typedef float f4 __attribute__((ext_vector_type(4)));

struct Out {
    float e, m;
    int s;
};

__device__ __forceinline__ Out step(float g, float e, float m, float beta1, float c, float clip) {
    float gc = g > clip ? clip : (g < -clip ? -clip : g);  // NaN passes through
    float x = gc + e;
    int s = (x > 0.0f) - (x < 0.0f);
    float q = static_cast<float>(s);
    float delta = x - q;
    float ea = beta1 * e;
    float eb = c * delta;
    float ma = beta1 * m;
    float mb = c * q;
    Out o;
    o.e = ea + eb;
    o.m = ma + mb;
    o.s = s;
    return o;
}

__device__ __forceinline__ uint32_t nonfinite2(float a, float b) {
    return ((__float_as_uint(a) & 0x7f800000u) == 0x7f800000u) + ((__float_as_uint(b) & 0x7f800000u) == 0x7f800000u);
}

__global__ void k_zero_u32(uint32_t* p) { *p = 0; }

// Elements [0, n8) (n8 = n rounded down to 8) in regions of kRegion per wave:
// lane l of unroll step u holds float4 j = base + 64u + l, i.e. elements
// 4j..4j+3; lanes 2i and 2i+1 together hold one whole output byte of bits.
// The last n - n8 elements are done by the first lane of wave 0.
// With STATS, wave w also writes part[w] = {sum e'^2, sum m'^2, #(+1), #(-1)}
// (float64, finite values only) for k_sign_stats.  Without MOM, m is neither
// read nor written (compress only; its terms count as zero).
template <bool STATS, bool MOM>
__global__ __launch_bounds__(kBlock) void k_sign(const float* __restrict__ g, float* __restrict__ e,
                                                 float* __restrict__ m, int64_t n, float beta1, float c,
                                                 float clip, int8_t* __restrict__ sgn, uint8_t* __restrict__ bits,
                                                 uint32_t* __restrict__ nonfinite, double4* __restrict__ part) {
    const int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int64_t n8 = n & ~static_cast<int64_t>(7);
    const int64_t beg = w * kRegion;
    if (beg >= n8 && w != 0) return;
    const int64_t end = min(beg + static_cast<int64_t>(kRegion), n8);
    const int l = lane();
    uint32_t nf = 0;
    double se = 0.0, sm = 0.0;
    uint32_t cp = 0, cn = 0;
    auto account = [&](const Out& o) {
        if (STATS) {
            if ((__float_as_uint(o.e) & 0x7f800000u) != 0x7f800000u) se += static_cast<double>(o.e) * o.e;
            if (MOM && (__float_as_uint(o.m) & 0x7f800000u) != 0x7f800000u) sm += static_cast<double>(o.m) * o.m;
            cp += o.s == 1;
            cn += o.s == -1;
        }
    };
    const int64_t nv = beg < end ? (end - beg) >> 2 : 0;  // even
    const f4* g4 = reinterpret_cast<const f4*>(g + beg);
    f4* e4 = reinterpret_cast<f4*>(e + beg);
    f4* m4 = MOM ? reinterpret_cast<f4*>(m + beg) : nullptr;
    uint32_t* s4 = sgn ? reinterpret_cast<uint32_t*>(sgn + beg) : nullptr;
    uint8_t* b8 = bits ? bits + (beg >> 3) : nullptr;
    auto iteration = [&](int64_t base, auto guard) {
        constexpr bool GUARD = decltype(guard)::value;
        f4 gv[kUnroll], ev[kUnroll], mv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = base + u * kWave + l;
            if (!GUARD || j < nv) {
                gv[u] = __builtin_nontemporal_load(g4 + j);
                ev[u] = __builtin_nontemporal_load(e4 + j);
                mv[u] = MOM ? __builtin_nontemporal_load(m4 + j) : f4{0.f, 0.f, 0.f, 0.f};
            } else {
                gv[u] = ev[u] = mv[u] = f4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = base + u * kWave + l;
            const bool ok = !GUARD || j < nv;
            const float ga[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
            const float ea[4] = {ev[u].x, ev[u].y, ev[u].z, ev[u].w};
            const float ma[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
            float eo[4], mo[4];
            uint32_t s4v = 0, nib = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const Out o = step(ga[t], ea[t], ma[t], beta1, c, clip);
                eo[t] = o.e;
                mo[t] = o.m;
                nf += ok ? nonfinite2(o.e, MOM ? o.m : 0.0f) : 0u;
                if (ok) account(o);
                s4v |= static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(o.s))) << (8 * t);
                nib |= (o.s == 1 ? 1u : 0u) << t;
            }
            const uint32_t hi = __shfl_xor(nib, 1, kWave);  // the odd lane's nibble
            if (ok) {
                __builtin_nontemporal_store(f4{eo[0], eo[1], eo[2], eo[3]}, e4 + j);
                if (MOM) __builtin_nontemporal_store(f4{mo[0], mo[1], mo[2], mo[3]}, m4 + j);
                // the int8 signs go out non-temporal like e and m (1.254 -> 1.227
                // ms at N = 340M); the bits bytes stay plain stores, which the
                // L2 merges into whole lines (non-temporal: 1.273 ms)
                if (s4) __builtin_nontemporal_store(s4v, s4 + j);
                if (b8 && !(l & 1)) b8[j >> 1] = static_cast<uint8_t>(nib | (hi << 4));
            }
        }
    };
    constexpr int64_t kStep = kWave * kUnroll;
    const int64_t nfull = nv / kStep * kStep;
    for (int64_t base = 0; base < nfull; base += kStep) iteration(base, std::false_type{});
    if (nfull < nv) iteration(nfull, std::true_type{});
    // the last n % 8 elements: one lane, one partial byte
    if (w == 0 && l == 0 && n8 < n) {
        uint32_t byte = 0;
        for (int64_t j = n8; j < n; ++j) {
            const Out o = step(g[j], e[j], MOM ? m[j] : 0.0f, beta1, c, clip);
            e[j] = o.e;
            if (MOM) m[j] = o.m;
            nf += nonfinite2(o.e, MOM ? o.m : 0.0f);
            account(o);
            if (sgn) sgn[j] = static_cast<int8_t>(o.s);
            byte |= (o.s == 1 ? 1u : 0u) << (j & 7);
        }
        if (bits) bits[n8 >> 3] = static_cast<uint8_t>(byte);
    }
    if (nonfinite) {
        nf = wave_sum(nf);
        if (l == 0 && nf) atomicAdd(nonfinite, nf);
    }
    if (STATS) {
        se = wave_sum(se);
        sm = wave_sum(sm);
        cp = wave_sum(cp);
        cn = wave_sum(cn);
        if (l == 0) part[w] = make_double4(se, sm, static_cast<double>(cp), static_cast<double>(cn));
    }
}

// Sums the per-wave statistics in a fixed order: stats = {sum e'^2, sum m'^2, #(+1), #(-1)}.
constexpr int kStatsBlock = 1024;
__global__ __launch_bounds__(kStatsBlock) void k_sign_stats(const double4* __restrict__ part, int64_t nw,
                                                            double* __restrict__ stats) {
    __shared__ double4 lsum[kStatsBlock / kWave];
    double4 a = make_double4(0.0, 0.0, 0.0, 0.0);
    for (int64_t w = threadIdx.x; w < nw; w += kStatsBlock) {
        a.x += part[w].x;
        a.y += part[w].y;
        a.z += part[w].z;
        a.w += part[w].w;
    }
    a.x = wave_sum(a.x);
    a.y = wave_sum(a.y);
    a.z = wave_sum(a.z);
    a.w = wave_sum(a.w);
    if (lane() == 0) lsum[threadIdx.x / kWave] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        double4 t = make_double4(0.0, 0.0, 0.0, 0.0);
        for (int i = 0; i < kStatsBlock / kWave; ++i) {
            t.x += lsum[i].x;
            t.y += lsum[i].y;
            t.z += lsum[i].z;
            t.w += lsum[i].w;
        }
        stats[0] = t.x;
        stats[1] = t.y;
        stats[2] = t.z;
        stats[3] = t.w;
    }
}

inline int64_t waves_for(int64_t n) { return std::max<int64_t>(1, cdiv(n & ~static_cast<int64_t>(7), kRegion)); }

}  // namespace sign
}  // namespace efg

using namespace efg;

extern "C" size_t ef_sign_workspace_bytes(int64_t n) {
    if (n < 0) return 0;
    return static_cast<size_t>(sign::waves_for(n)) * sizeof(double4);
}

extern "C" int ef_sign_compress(const float* g, float* e, float* m, int64_t n, float beta1, float clip,
                                int8_t* sign_out, uint8_t* bits, uint32_t* nonfinite, double* stats, void* ws,
                                size_t ws_bytes, void* stream) {
    if (n < 0 || n > kMaxElems) return fail(EF_EINVAL, "n=%lld outside [0, 2^31-1]", (long long)n);
    if (!(beta1 >= 0.0f && beta1 <= 1.0f)) return fail(EF_EINVAL, "beta1 must lie in [0, 1]");
    if (!(clip > 0.0f)) return fail(EF_EINVAL, "clip must be > 0 (+inf disables clipping)");
    if (n > 0 && (!g || !e)) return fail(EF_EINVAL, "g and e must not be NULL");
    if (n > 0 && (!aligned16(g) || !aligned16(e) || (m && !aligned16(m))))
        return fail(EF_EINVAL, "g, e and m must be 16-byte aligned");
    if (sign_out && (reinterpret_cast<uintptr_t>(sign_out) & 3u))
        return fail(EF_EINVAL, "sign_out must be 4-byte aligned");
    if (stats) {
        const size_t need = ef_sign_workspace_bytes(n);
        if (!ws || ws_bytes < need) return fail(EF_EWS, "ef_sign_compress: statistics need %zu bytes of workspace", need);
        if (reinterpret_cast<uintptr_t>(ws) & 31u) return fail(EF_EINVAL, "workspace must be 32-byte aligned");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (nonfinite) EF_TRY(launch("sign_zero", sign::k_zero_u32, dim3(1), dim3(1), s, nonfinite));
    const float c = 1.0f - beta1;
    const int64_t waves = sign::waves_for(n);
    const int64_t grid = cdiv(waves, sign::kWaves);
    double4* part = static_cast<double4*>(ws);
    if (n > 0) {
        const dim3 gd(static_cast<unsigned>(grid)), bd(sign::kBlock);
        double4* p = stats ? part : nullptr;
        if (stats && m)
            EF_TRY(launch("sign_ef", sign::k_sign<true, true>, gd, bd, s, g, e, m, n, beta1, c, clip, sign_out, bits,
                          nonfinite, p));
        else if (stats)
            EF_TRY(launch("sign_ef", sign::k_sign<true, false>, gd, bd, s, g, e, m, n, beta1, c, clip, sign_out, bits,
                          nonfinite, p));
        else if (m)
            EF_TRY(launch("sign_ef", sign::k_sign<false, true>, gd, bd, s, g, e, m, n, beta1, c, clip, sign_out, bits,
                          nonfinite, p));
        else
            EF_TRY(launch("sign_ef", sign::k_sign<false, false>, gd, bd, s, g, e, m, n, beta1, c, clip, sign_out,
                          bits, nonfinite, p));
    }
    if (!stats) return EF_OK;
    return launch("sign_stats", sign::k_sign_stats, dim3(1), dim3(sign::kStatsBlock), s,
                  static_cast<const double4*>(part), n > 0 ? waves : static_cast<int64_t>(0), stats);
}
