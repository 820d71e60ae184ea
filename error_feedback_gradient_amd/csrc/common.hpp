// Shared host and device helpers of libefgrad (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <utility>

#include "efgrad.h"

namespace efg {

// ------------------------------------------------------------------ host side
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int check_launch(const char* label);

// Event pair of one launch when profiling is on (see ef_profile_enable): the
// launch records both with the dispatch itself (hipExtLaunchKernelGGL), so
// their interval is the kernel's own run, without marker packets around it.
// Nothing is recorded on a stream under graph capture.
struct ProfScope {
    hipEvent_t start = nullptr, stop = nullptr;
    ProfScope(const char* label, hipStream_t s);
};

template <typename... KArgs, typename... Args>
inline int launch(const char* label, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                  hipStream_t s, Args... args) {
    if (grid.x == 0 || grid.y == 0 || grid.z == 0) return EF_OK;
    ProfScope ps(label, s);
    if (ps.start)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ps.start, ps.stop, 0u, static_cast<KArgs>(args)...);
    else
        kernel<<<grid, block, 0, s>>>(static_cast<KArgs>(args)...);
    return check_launch(label);
}

#define EF_TRY(expr)                 \
    do {                             \
        int _rc = (expr);            \
        if (_rc != EF_OK) return _rc; \
    } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }
constexpr int64_t kMaxElems = 0x7fffffffLL;

// A few hundred host words passed to a kernel by value.
constexpr uint32_t kWordChunk = 500;
struct WordChunk {
    uint32_t n;
    uint32_t w[kWordChunk];
};

// Upload up to a few KB of host words into device memory through kernel
// arguments (copied by the runtime at launch, so the host buffer is free as
// soon as the call returns and no pinned staging or host wait is needed).
int upload_words(void* dst, const uint32_t* src, size_t nwords, hipStream_t s);
// Fill n bytes of device memory with zero using a kernel (no memset node).
int zero_bytes(void* dst, size_t n, hipStream_t s);

// ------------------------------------------------------------------ device side
constexpr int kWave = 64;

__device__ __forceinline__ uint32_t lane() { return __lane_id(); }

// number of set bits of m in lanes below the calling lane
__device__ __forceinline__ uint32_t count_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ uint32_t key_of(float x) { return __float_as_uint(x) & 0x7fffffffu; }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// inclusive scan over the 64 lanes
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    const uint32_t l = lane();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        uint32_t t = __shfl_up(v, d, kWave);
        if (l >= static_cast<uint32_t>(d)) v += t;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_incl_scan64(uint64_t v) {
    const uint32_t l = lane();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        uint32_t lo = __shfl_up(static_cast<uint32_t>(v), d, kWave);
        uint32_t hi = __shfl_up(static_cast<uint32_t>(v >> 32), d, kWave);
        uint64_t t = (static_cast<uint64_t>(hi) << 32) | lo;
        if (l >= static_cast<uint32_t>(d)) v += t;
    }
    return v;
}

// Exclusive scan over a block of NT threads (NT a multiple of 64, <= 1024).
// `lds` needs NT/64 + 1 slots.  Returns the exclusive prefix; *total gets the
// block sum.  Contains barriers: every thread of the block must call it.
template <int NT, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* lds, T* total) {
    constexpr int NW = NT / kWave;
    const uint32_t w = threadIdx.x / kWave;
    T incl;
    if constexpr (sizeof(T) == 8) incl = wave_incl_scan64(v);
    else incl = wave_incl_scan(v);
    if (lane() == kWave - 1) lds[w] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        T run = 0;
        for (int i = 0; i < NW; ++i) {
            T t = lds[i];
            lds[i] = run;
            run += t;
        }
        lds[NW] = run;
    }
    __syncthreads();
    T res = lds[w] + incl - v;
    *total = lds[NW];
    __syncthreads();
    return res;
}

// largest i in [0, n) with a[i] <= v, for a non-decreasing a with a[0] <= v
template <typename T>
__device__ __forceinline__ int upper_index(const T* a, int n, T v) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (a[mid] <= v) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Exclusive scan in place of a[0..m) (uint32 or uint64) by one block of
// kScanThreads threads, each summing a contiguous slice; total -> *tot (if
// set) and, converted, -> *tot64 (if set).
constexpr int kScanThreads = 1024;
template <typename T>
__global__ __launch_bounds__(kScanThreads) void k_excl_scan(T* __restrict__ a, int64_t m, T* __restrict__ tot,
                                                            int64_t* __restrict__ tot64) {
    __shared__ T lds[kScanThreads / kWave + 1];
    const int64_t per = (m + kScanThreads - 1) / kScanThreads;
    const int64_t i0 = per * threadIdx.x < m ? per * threadIdx.x : m;
    const int64_t i1 = i0 + per < m ? i0 + per : m;
    T sum = 0;
    for (int64_t i = i0; i < i1; ++i) sum += a[i];
    T total;
    T run = block_excl_scan<kScanThreads>(sum, lds, &total);
    for (int64_t i = i0; i < i1; ++i) {
        const T t = a[i];
        a[i] = run;
        run += t;
    }
    if (threadIdx.x == 0) {
        if (tot) *tot = total;
        if (tot64) *tot64 = static_cast<int64_t>(total);
    }
}

}  // namespace efg
