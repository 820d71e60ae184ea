// Adam warm-up step and 1-bit Adam compression-phase update, gfx950.
//
// "1-bit Adam" page: section 3.1 (the optimiser state holds momentum,
// variance, beta1, beta2, eps and the step count), section 2.2 (the momentum
// runs on the compressed gradient) and section 6.1 (the first steps train at
// full precision before the switch to 1-bit compression).  The variance and
// parameter rules follow textbook Adam (Kingma and Ba, ICLR 2015,
// Algorithm 1), with the bias corrections folded into two host scalars:
//   step_size = lr / (1 - beta1^t),  sqrt_bc2 = sqrt(1 - beta2^t_v)
//   w' = w - step_size * (m / (sqrt(v) / sqrt_bc2 + eps))
//
// ef_adam_step (warm-up, full precision, per element):
//   m' = beta1 m + (1 - beta1) g;  v' = beta2 v + (1 - beta2) (g g);  w' as above
//   reads g, m, v, w and writes m, v, w: 28 B per element.
// ef_onebit_adam_update (compression phase, after the workers' int8 signs
// were summed into qsum): ghat = qsum / nworkers;
//   m' = beta1 m + (1 - beta1) ghat;  v frozen (read only);  w' as above
//   reads qsum (1 B), m, v, w and writes m, w: 21 B per element.
// ef_onebit_adam_update_var: the same with v' = beta2 v + (1 - beta2) ghat^2
//   (every replica holds the same ghat, so this v stays shared too): 25 B.
// One streaming pass each, one wave per region, 128-bit non-temporal loads
// and stores.  Square root and divisions are correctly rounded; every other
// product and sum is rounded on its own (-ffp-contract=off).
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace efg {
namespace adam {

#ifndef EFG_ADAM_BLOCK
#define EFG_ADAM_BLOCK 512
#endif
#ifndef EFG_ADAM_REGION
#define EFG_ADAM_REGION 4096
#endif
#ifndef EFG_ADAM_UNROLL
#define EFG_ADAM_UNROLL 8
#endif
constexpr int kBlock = EFG_ADAM_BLOCK;
constexpr int kWaves = kBlock / kWave;
constexpr int kRegion = EFG_ADAM_REGION;
constexpr int kUnroll = EFG_ADAM_UNROLL;
static_assert(kRegion % 256 == 0, "regions hold whole float4 per lane");

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t nonfinite(float a) {
    return (__float_as_uint(a) & 0x7f800000u) == 0x7f800000u ? 1u : 0u;
}

__device__ __forceinline__ float param(float w, float m, float v, float step_size, float sqrt_bc2, float eps) {
    const float r = __builtin_sqrtf(v);
    const float q = r / sqrt_bc2;
    const float d = q + eps;
    const float u = m / d;
    const float s = step_size * u;
    return w - s;
}

struct Hyper {
    float beta1, c1, beta2, c2, step_size, sqrt_bc2, eps, inv_unused;
};

// One element.  VUPD: v takes gin^2 (warm-up, and the 1-bit step that keeps
// updating the variance with ghat^2); otherwise v is kept.
template <bool VUPD>
__device__ __forceinline__ void element(float gin, float& m, float& v, float& w, const Hyper& h, uint32_t& nf) {
    const float ma = h.beta1 * m;
    const float mb = h.c1 * gin;
    const float mn = ma + mb;
    float vn = v;
    if (VUPD) {
        const float g2 = gin * gin;
        const float va = h.beta2 * v;
        const float vb = h.c2 * g2;
        vn = va + vb;
    }
    const float wn = param(w, mn, vn, h.step_size, h.sqrt_bc2, h.eps);
    nf += nonfinite(mn) + nonfinite(wn) + (VUPD ? nonfinite(vn) : 0u);
    m = mn;
    v = vn;
    w = wn;
}

// Wave w owns elements [w*kRegion, min((w+1)*kRegion, n)); lane l of unroll
// step u holds float4 j = base + 64u + l of its region; a final partial float4
// (only in the last region) goes element by element.  ONEBIT reads the four
// int8 sums of a float4 as one 32-bit word (qsum is 4-byte aligned).  Without
// DIV the worker count is a power of two: qs * (1/N) is then exact and equals
// the correctly rounded qs / N.
template <bool ONEBIT, bool DIV, bool VUPD>
__global__ __launch_bounds__(kBlock) void k_adam(const float* __restrict__ g, const int8_t* __restrict__ qsum,
                                                 float nworkers, float* __restrict__ m, float* __restrict__ v,
                                                 float* __restrict__ w, int64_t n, Hyper h,
                                                 uint32_t* __restrict__ nonfinite_out) {
    const int64_t wv = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int64_t beg = wv * kRegion;
    if (beg >= n) return;
    const int64_t len = min(static_cast<int64_t>(kRegion), n - beg);
    const int64_t nfull = len >> 2;
    const int64_t nv = (len + 3) >> 2;
    const int l = lane();
    const f4* g4 = ONEBIT ? nullptr : reinterpret_cast<const f4*>(g + beg);
    const uint32_t* q4 = ONEBIT ? reinterpret_cast<const uint32_t*>(qsum + beg) : nullptr;
    f4* m4 = reinterpret_cast<f4*>(m + beg);
    f4* v4 = reinterpret_cast<f4*>(v + beg);
    f4* w4 = reinterpret_cast<f4*>(w + beg);
    uint32_t nf = 0;
    const float recip = 1.0f / nworkers;
    auto ghat = [&](float qs) -> float { return DIV ? qs / nworkers : qs * recip; };
    auto gin_of = [&](f4 gv, uint32_t qw, int t) -> float {
        if (ONEBIT) return ghat(static_cast<float>(static_cast<int8_t>(qw >> (8 * t))));
        return t == 0 ? gv.x : t == 1 ? gv.y : t == 2 ? gv.z : gv.w;
    };
    auto iteration = [&](int64_t base, auto guard) {
        constexpr bool GUARD = decltype(guard)::value;
        f4 gv[kUnroll], mv[kUnroll], vv[kUnroll], wv4[kUnroll];
        uint32_t qv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = base + u * kWave + l;
            if (!GUARD || j < nfull) {
                if (ONEBIT) qv[u] = __builtin_nontemporal_load(q4 + j);
                else gv[u] = __builtin_nontemporal_load(g4 + j);
                mv[u] = __builtin_nontemporal_load(m4 + j);
                vv[u] = __builtin_nontemporal_load(v4 + j);
                wv4[u] = __builtin_nontemporal_load(w4 + j);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = base + u * kWave + l;
            if (!GUARD || j < nfull) {
                float ma[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
                float va[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
                float wa[4] = {wv4[u].x, wv4[u].y, wv4[u].z, wv4[u].w};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    element<VUPD>(gin_of(ONEBIT ? f4{} : gv[u], ONEBIT ? qv[u] : 0u, t), ma[t], va[t], wa[t], h, nf);
                __builtin_nontemporal_store(f4{ma[0], ma[1], ma[2], ma[3]}, m4 + j);
                if (VUPD) __builtin_nontemporal_store(f4{va[0], va[1], va[2], va[3]}, v4 + j);
                __builtin_nontemporal_store(f4{wa[0], wa[1], wa[2], wa[3]}, w4 + j);
            } else if (GUARD && j == nfull && nfull < nv) {
                for (int64_t i = beg + 4 * nfull; i < beg + len; ++i) {
                    const float gin = ONEBIT ? ghat(static_cast<float>(qsum[i])) : g[i];
                    float mi = m[i], vi = v[i], wi = w[i];
                    element<VUPD>(gin, mi, vi, wi, h, nf);
                    m[i] = mi;
                    if (VUPD) v[i] = vi;
                    w[i] = wi;
                }
            }
        }
    };
    constexpr int64_t kStep = kWave * kUnroll;
    int64_t base = 0;
    for (; base + kStep <= nfull; base += kStep) iteration(base, std::false_type{});
    if (base < nv) iteration(base, std::true_type{});
    if (nonfinite_out) {
        nf = wave_sum(nf);
        if (l == 0 && nf) atomicAdd(nonfinite_out, nf);
    }
}

__global__ void k_zero_u32(uint32_t* p) { *p = 0; }

inline int64_t blocks_for(int64_t n) { return std::max<int64_t>(1, cdiv(cdiv(n, kRegion), kWaves)); }

inline int check_common(float* m, const float* v, float* w, int64_t n, float beta1, float step_size, float sqrt_bc2,
                        float eps) {
    if (n < 0 || n > kMaxElems) return fail(EF_EINVAL, "n=%lld outside [0, 2^31-1]", (long long)n);
    if (!(beta1 >= 0.0f && beta1 <= 1.0f)) return fail(EF_EINVAL, "beta1 must lie in [0, 1]");
    if (!(sqrt_bc2 > 0.0f) || !(eps >= 0.0f) || !(step_size == step_size))
        return fail(EF_EINVAL, "sqrt_bc2 must be > 0, eps >= 0 and step_size a number");
    if (n > 0 && (!m || !v || !w)) return fail(EF_EINVAL, "m, v and w must not be NULL");
    if (n > 0 && (!aligned16(m) || !aligned16(v) || !aligned16(w)))
        return fail(EF_EINVAL, "m, v and w must be 16-byte aligned");
    return EF_OK;
}

}  // namespace adam
}  // namespace efg

using namespace efg;

// Bias corrections of step t as the two host scalars of the update, in
// float64 from the float32 betas, each rounded once to float32.
extern "C" int ef_adam_scalars(double lr, float beta1, float beta2, int64_t t, int64_t t_v, float* step_size,
                               float* sqrt_bc2) {
    if (!step_size || !sqrt_bc2) return fail(EF_EINVAL, "ef_adam_scalars: outputs must not be NULL");
    if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
        return fail(EF_EINVAL, "ef_adam_scalars: betas must lie in [0, 1)");
    if (t < 1 || t_v < 1) return fail(EF_EINVAL, "ef_adam_scalars: steps count from 1");
    if (!isfinite(lr)) return fail(EF_EINVAL, "ef_adam_scalars: lr must be finite");
    const double bc1 = 1.0 - pow(static_cast<double>(beta1), static_cast<double>(t));
    const double bc2 = 1.0 - pow(static_cast<double>(beta2), static_cast<double>(t_v));
    *step_size = static_cast<float>(lr / bc1);
    *sqrt_bc2 = static_cast<float>(sqrt(bc2));
    return EF_OK;
}

extern "C" int ef_adam_step(const float* g, float* m, float* v, float* w, int64_t n, float beta1, float beta2,
                            float step_size, float sqrt_bc2, float eps, uint32_t* nonfinite, void* stream) {
    EF_TRY(adam::check_common(m, v, w, n, beta1, step_size, sqrt_bc2, eps));
    if (!(beta2 >= 0.0f && beta2 <= 1.0f)) return fail(EF_EINVAL, "beta2 must lie in [0, 1]");
    if (n > 0 && (!g || !aligned16(g))) return fail(EF_EINVAL, "g must be a 16-byte aligned pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (nonfinite) EF_TRY(launch("adam_zero", adam::k_zero_u32, dim3(1), dim3(1), s, nonfinite));
    if (n == 0) return EF_OK;
    const adam::Hyper h{beta1, 1.0f - beta1, beta2, 1.0f - beta2, step_size, sqrt_bc2, eps, 0.0f};
    return launch("adam_step", adam::k_adam<false, false, true>, dim3(static_cast<unsigned>(adam::blocks_for(n))),
                  dim3(adam::kBlock), s, g, static_cast<const int8_t*>(nullptr), 1.0f, m, v, w, n, h, nonfinite);
}

extern "C" int ef_onebit_adam_update(const int8_t* qsum, int32_t nworkers, float* m, const float* v, float* w,
                                     int64_t n, float beta1, float step_size, float sqrt_bc2, float eps,
                                     uint32_t* nonfinite, void* stream) {
    EF_TRY(adam::check_common(m, v, w, n, beta1, step_size, sqrt_bc2, eps));
    if (nworkers < 1 || nworkers > 127) return fail(EF_EINVAL, "nworkers must lie in [1, 127]");
    if (n > 0 && (!qsum || (reinterpret_cast<uintptr_t>(qsum) & 3u)))
        return fail(EF_EINVAL, "qsum must be a 4-byte aligned pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (nonfinite) EF_TRY(launch("onebit_zero", adam::k_zero_u32, dim3(1), dim3(1), s, nonfinite));
    if (n == 0) return EF_OK;
    const adam::Hyper h{beta1, 1.0f - beta1, 1.0f, 0.0f, step_size, sqrt_bc2, eps, 0.0f};
    const bool pow2 = (nworkers & (nworkers - 1)) == 0;
    return launch("onebit_update", pow2 ? adam::k_adam<true, false, false> : adam::k_adam<true, true, false>,
                  dim3(static_cast<unsigned>(adam::blocks_for(n))), dim3(adam::kBlock), s,
                  static_cast<const float*>(nullptr), qsum, static_cast<float>(nworkers), m, const_cast<float*>(v), w,
                  n, h, nonfinite);
}

extern "C" int ef_onebit_adam_update_var(const int8_t* qsum, int32_t nworkers, float* m, float* v, float* w,
                                         int64_t n, float beta1, float beta2, float step_size, float sqrt_bc2,
                                         float eps, uint32_t* nonfinite, void* stream) {
    EF_TRY(adam::check_common(m, v, w, n, beta1, step_size, sqrt_bc2, eps));
    if (!(beta2 >= 0.0f && beta2 <= 1.0f)) return fail(EF_EINVAL, "beta2 must lie in [0, 1]");
    if (nworkers < 1 || nworkers > 127) return fail(EF_EINVAL, "nworkers must lie in [1, 127]");
    if (n > 0 && (!qsum || (reinterpret_cast<uintptr_t>(qsum) & 3u)))
        return fail(EF_EINVAL, "qsum must be a 4-byte aligned pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (nonfinite) EF_TRY(launch("onebit_zero", adam::k_zero_u32, dim3(1), dim3(1), s, nonfinite));
    if (n == 0) return EF_OK;
    const adam::Hyper h{beta1, 1.0f - beta1, beta2, 1.0f - beta2, step_size, sqrt_bc2, eps, 0.0f};
    const bool pow2 = (nworkers & (nworkers - 1)) == 0;
    return launch("onebit_update_var", pow2 ? adam::k_adam<true, false, true> : adam::k_adam<true, true, true>,
                  dim3(static_cast<unsigned>(adam::blocks_for(n))), dim3(adam::kBlock), s,
                  static_cast<const float*>(nullptr), qsum, static_cast<float>(nworkers), m, v, w, n, h, nonfinite);
}
