// 1-bit sign compression with averaged error feedback and momentum, gfx950.
//
// "1-bit Adam" page, sections 2.1 (sign quantisation, quantisation error and
// its averaged error buffer), 2.2 (momentum on the quantised gradient) and 3.2
// (clip before quantisation, NaN check after the error update, int8 storage);
// section 1 (32 bits -> 1 bit per element).
//
// One streaming pass: each lane owns 8 consecutive elements (two 128-bit loads
// per array), so its 8 sign bits are exactly one output byte and its 8 int8
// signs one 64-bit store.  21.125 bytes move per element with both optional
// outputs (read g, e, m; write e, m, int8, 1 bit).  Every product and sum is
// rounded on its own: the library is compiled with -ffp-contract=off.
#include "common.hpp"

namespace efg {
namespace sign {

constexpr int kBlock = 256;
constexpr int kMaxGrid = 16384;

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

__global__ __launch_bounds__(kBlock) void k_sign(const float* __restrict__ g, float* __restrict__ e,
                                                 float* __restrict__ m, int64_t n, float beta1, float c,
                                                 float clip, int8_t* __restrict__ sgn, uint8_t* __restrict__ bits,
                                                 uint32_t* __restrict__ nonfinite) {
    const int64_t groups = n >> 3;  // full groups of 8
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    uint32_t nf = 0;
    const f4* g4 = reinterpret_cast<const f4*>(g);
    f4* e4 = reinterpret_cast<f4*>(e);
    f4* m4 = reinterpret_cast<f4*>(m);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < groups; i += stride) {
        const f4 ga = __builtin_nontemporal_load(g4 + 2 * i), gb = __builtin_nontemporal_load(g4 + 2 * i + 1);
        const f4 ea = __builtin_nontemporal_load(e4 + 2 * i), eb = __builtin_nontemporal_load(e4 + 2 * i + 1);
        const f4 ma = __builtin_nontemporal_load(m4 + 2 * i), mb = __builtin_nontemporal_load(m4 + 2 * i + 1);
        const float gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
        const float ev[8] = {ea.x, ea.y, ea.z, ea.w, eb.x, eb.y, eb.z, eb.w};
        const float mv[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
        float eo[8], mo[8];
        uint64_t s8 = 0;
        uint32_t byte = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const Out o = step(gv[t], ev[t], mv[t], beta1, c, clip);
            eo[t] = o.e;
            mo[t] = o.m;
            nf += nonfinite2(o.e, o.m);
            s8 |= static_cast<uint64_t>(static_cast<uint8_t>(static_cast<int8_t>(o.s))) << (8 * t);
            byte |= (o.s == 1 ? 1u : 0u) << t;
        }
        __builtin_nontemporal_store(f4{eo[0], eo[1], eo[2], eo[3]}, e4 + 2 * i);
        __builtin_nontemporal_store(f4{eo[4], eo[5], eo[6], eo[7]}, e4 + 2 * i + 1);
        __builtin_nontemporal_store(f4{mo[0], mo[1], mo[2], mo[3]}, m4 + 2 * i);
        __builtin_nontemporal_store(f4{mo[4], mo[5], mo[6], mo[7]}, m4 + 2 * i + 1);
        if (sgn) reinterpret_cast<uint64_t*>(sgn)[i] = s8;
        if (bits) bits[i] = static_cast<uint8_t>(byte);
    }
    // tail: the last n % 8 elements, handled by the first thread of block 0
    if (blockIdx.x == 0 && threadIdx.x == 0 && (n & 7)) {
        uint32_t byte = 0;
        for (int64_t j = groups * 8; j < n; ++j) {
            const Out o = step(g[j], e[j], m[j], beta1, c, clip);
            e[j] = o.e;
            m[j] = o.m;
            nf += nonfinite2(o.e, o.m);
            if (sgn) sgn[j] = static_cast<int8_t>(o.s);
            byte |= (o.s == 1 ? 1u : 0u) << (j & 7);
        }
        if (bits) bits[groups] = static_cast<uint8_t>(byte);
    }
    if (nonfinite) {
        nf = wave_sum(nf);
        if (lane() == 0 && nf) atomicAdd(nonfinite, nf);
    }
}

}  // namespace sign
}  // namespace efg

using namespace efg;

extern "C" int ef_sign_compress(const float* g, float* e, float* m, int64_t n, float beta1, float clip,
                                int8_t* sign_out, uint8_t* bits, uint32_t* nonfinite, void* stream) {
    if (n < 0 || n > kMaxElems) return fail(EF_EINVAL, "n=%lld outside [0, 2^31-1]", (long long)n);
    if (!(beta1 >= 0.0f && beta1 <= 1.0f)) return fail(EF_EINVAL, "beta1 must lie in [0, 1]");
    if (!(clip > 0.0f)) return fail(EF_EINVAL, "clip must be > 0 (+inf disables clipping)");
    if (n > 0 && (!g || !e || !m)) return fail(EF_EINVAL, "g, e and m must not be NULL");
    if (n > 0 && (!aligned16(g) || !aligned16(e) || !aligned16(m)))
        return fail(EF_EINVAL, "g, e and m must be 16-byte aligned");
    if (sign_out && (reinterpret_cast<uintptr_t>(sign_out) & 7u))
        return fail(EF_EINVAL, "sign_out must be 8-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (nonfinite) EF_TRY(launch("sign_zero", sign::k_zero_u32, dim3(1), dim3(1), s, nonfinite));
    if (n == 0) return EF_OK;
    const float c = 1.0f - beta1;
    const int64_t groups = n >> 3;
    int64_t grid = cdiv(groups > 0 ? groups : 1, sign::kBlock);
    if (grid > sign::kMaxGrid) grid = sign::kMaxGrid;
    return launch("sign_ef", sign::k_sign, dim3(static_cast<unsigned>(grid)), dim3(sign::kBlock), s, g, e, m, n,
                  beta1, c, clip, sign_out, bits, nonfinite);
}
