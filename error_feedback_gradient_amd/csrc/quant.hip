// 8-bit quantisation of a sent packet, the error kept in the residual, gfx950.
//
// "Gradient sparsification" page, comparison with other compression
// techniques: top-k selection followed by 8-bit quantisation of the kept
// values.  One symmetric scale per packet: amax = largest finite |v|,
// inv = 127 / amax and scale = amax / 127 (correctly rounded float32
// divisions), q = rint(v * inv) clamped to [-127, 127], e[idx] = v - q*scale.
//
// Two kernels: per-block maxima of the finite magnitudes (compared as bit
// patterns, so the result does not depend on order), then the quantisation,
// where every block reduces the per-block maxima again so that no clearing
// launch is needed.  O(k) work: read v and idx, write q and one scattered e.
#include <algorithm>

#include "common.hpp"

namespace efg {
namespace quant {

constexpr int kBlock = 256;
constexpr int kMaxGrid = 1024;
#ifndef EFG_QUANT_PER
#define EFG_QUANT_PER 4
#endif
constexpr int kPer = EFG_QUANT_PER;  // entries per thread and step

__global__ __launch_bounds__(kBlock) void k_amax(const float* __restrict__ vals, int64_t k,
                                                 uint32_t* __restrict__ part) {
    __shared__ uint32_t w[kBlock / kWave];
    uint32_t m = 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    // kPer entries per thread and step, all loaded before any is used
    for (int64_t j0 = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j0 < k; j0 += stride * kPer) {
        float v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) v[u] = vals[min(j0 + u * stride, k - 1)];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const uint32_t key = key_of(v[u]);
            if (j0 + u * stride < k && key < 0x7f800000u) m = max(m, key);  // finite values only
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(m, d, kWave)));
    if (lane() == 0) w[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < kBlock / kWave; ++i) r = max(r, w[i]);
        part[blockIdx.x] = r;
    }
}

__global__ __launch_bounds__(kBlock) void k_quant(const float* __restrict__ vals, const int32_t* __restrict__ idx,
                                                  int64_t k, float* __restrict__ e, int64_t n,
                                                  int8_t* __restrict__ q, float* __restrict__ scale_out,
                                                  const uint32_t* __restrict__ part, int nparts) {
    __shared__ uint32_t w[kBlock / kWave];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += kBlock) m = max(m, part[i]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(m, d, kWave)));
    if (lane() == 0) w[threadIdx.x / kWave] = m;
    __syncthreads();
    uint32_t mk = 0;
    for (int i = 0; i < kBlock / kWave; ++i) mk = max(mk, w[i]);
    const float amax = __uint_as_float(mk);
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    const float scale = amax > 0.0f ? amax / 127.0f : 0.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = scale;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    // kPer entries per thread and step, all loaded before any is used, so
    // that a thread has kPer scattered residual writes in flight
    for (int64_t j0 = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j0 < k; j0 += stride * kPer) {
        float v[kPer];
        int32_t ix[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int64_t j = min(j0 + u * stride, k - 1);
            v[u] = vals[j];
            ix[u] = idx[j];
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int64_t j = j0 + u * stride;
            if (j >= k) break;
            int qi = 0;
            if (amax > 0.0f && key_of(v[u]) < 0x7f800000u) {
                const float t = v[u] * inv;
                float r = rintf(t);
                if (r != r) r = 0.0f;  // 0 * inf when amax is below 127 / FLT_MAX
                r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
                qi = static_cast<int>(r);
            }
            const float deq = static_cast<float>(qi) * scale;
            q[j] = static_cast<int8_t>(qi);
            const int64_t i = ix[u];
            if (i >= 0 && i < n) e[i] = v[u] - deq;
        }
    }
}

}  // namespace quant
}  // namespace efg

using namespace efg;

extern "C" size_t ef_quantize_workspace_bytes(int64_t k) {
    if (k < 0) return 0;
    return quant::kMaxGrid * sizeof(uint32_t);
}

extern "C" int ef_quantize_int8(const float* vals, const int32_t* idx, int64_t k, float* e, int64_t n, int8_t* q,
                                float* scale_out, void* ws, size_t ws_bytes, void* stream) {
    if (k < 0 || k > kMaxElems || n < 0 || n > kMaxElems) return fail(EF_EINVAL, "ef_quantize_int8: bad sizes");
    if (!scale_out) return fail(EF_EINVAL, "ef_quantize_int8: scale_out must not be NULL");
    if (k > 0 && (!vals || !idx || !e || !q)) return fail(EF_EINVAL, "ef_quantize_int8: NULL argument");
    const size_t need = ef_quantize_workspace_bytes(k);
    if (!ws || ws_bytes < need) return fail(EF_EWS, "ef_quantize_int8: workspace %zu < %zu bytes", ws_bytes, need);
    if (reinterpret_cast<uintptr_t>(ws) & 3u) return fail(EF_EINVAL, "ef_quantize_int8: workspace must be 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int grid = static_cast<int>(std::min<int64_t>(quant::kMaxGrid, std::max<int64_t>(1, cdiv(k, quant::kBlock))));
    uint32_t* part = static_cast<uint32_t*>(ws);
    EF_TRY(launch("quant_amax", quant::k_amax, dim3(grid), dim3(quant::kBlock), s, vals, k, part));
    return launch("quant_int8", quant::k_quant, dim3(grid), dim3(quant::kBlock), s, vals, idx, k, e, n, q, scale_out,
                  static_cast<const uint32_t*>(part), grid);
}
