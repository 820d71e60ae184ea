// Error reporting, kernel timing and small device utilities of libefgrad.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace efg {

static thread_local std::string g_err = "no error";

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int check_launch(const char* label) {
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(EF_EHIP, "launch of %s failed: %s", label, hipGetErrorString(err));
    return EF_OK;
}

// ------------------------------------------------------------------ profiling
namespace {
struct ProfRec {
    std::string label;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
// read first by every launch, without the lock: launches do not serialise on
// the mutex while profiling is off
std::atomic<bool> g_prof_armed{false};
bool g_prof_on = false;
std::string g_prof_only;
std::vector<ProfRec> g_prof;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_prof_pool;

void prof_clear_locked() {
    for (auto& r : g_prof) g_prof_pool.emplace_back(r.start, r.stop);
    g_prof.clear();
}
}  // namespace

ProfScope::ProfScope(const char* label, hipStream_t s) {
    if (!g_prof_armed.load(std::memory_order_acquire)) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    if (!g_prof_only.empty() && !strstr(label, g_prof_only.c_str())) return;
    ProfRec r;
    r.label = label;
    if (!g_prof_pool.empty()) {
        r.start = g_prof_pool.back().first;
        r.stop = g_prof_pool.back().second;
        g_prof_pool.pop_back();
    } else {
        if (hipEventCreate(&r.start) != hipSuccess) return;
        if (hipEventCreate(&r.stop) != hipSuccess) { (void)hipEventDestroy(r.start); return; }
    }
    g_prof.push_back(r);
    start = r.start;
    stop = r.stop;
}

// ------------------------------------------------------------------ utilities
__global__ void k_upload(uint32_t* dst, WordChunk c) {
    for (uint32_t i = threadIdx.x; i < c.n; i += blockDim.x) dst[i] = c.w[i];
}

int upload_words(void* dst, const uint32_t* src, size_t nwords, hipStream_t s) {
    uint32_t* d = static_cast<uint32_t*>(dst);
    for (size_t at = 0; at < nwords; at += kWordChunk) {
        WordChunk c;
        c.n = static_cast<uint32_t>(nwords - at < kWordChunk ? nwords - at : kWordChunk);
        memcpy(c.w, src + at, c.n * sizeof(uint32_t));
        EF_TRY(launch("upload", k_upload, dim3(1), dim3(256), s, d + at, c));
    }
    return EF_OK;
}

__global__ void k_zero(uint8_t* dst, size_t n) {
    size_t nv = n / 16;
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nv; i += stride)
        d4[i] = make_uint4(0, 0, 0, 0);
    for (size_t i = nv * 16 + static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = 0;
}

int zero_bytes(void* dst, size_t n, hipStream_t s) {
    if (n == 0) return EF_OK;
    if (!aligned16(dst)) return fail(EF_EINVAL, "zero_bytes: destination not 16-byte aligned");
    int64_t blocks = cdiv(static_cast<int64_t>(n / 16 + 1), 256);
    if (blocks > 2048) blocks = 2048;
    return launch("zero", k_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), s,
                  static_cast<uint8_t*>(dst), n);
}

}  // namespace efg

extern "C" {

const char* ef_last_error(void) { return efg::g_err.c_str(); }

const char* ef_version(void) { return "efgrad 0.1 gfx950"; }

int ef_profile_enable(int on, const char* only) {
    std::lock_guard<std::mutex> lk(efg::g_prof_mu);
    efg::prof_clear_locked();
    efg::g_prof_on = on != 0;
    efg::g_prof_only = (on && only) ? only : "";
    efg::g_prof_armed.store(efg::g_prof_on, std::memory_order_release);
    return EF_OK;
}

int ef_profile_read(const char* name, double* total_ms, int64_t* launches) {
    if (!name || !total_ms || !launches) return efg::fail(EF_EINVAL, "ef_profile_read: null argument");
    std::lock_guard<std::mutex> lk(efg::g_prof_mu);
    double sum = 0.0;
    int64_t cnt = 0;
    for (auto& r : efg::g_prof) {
        if (r.label.find(name) == std::string::npos) continue;
        if (hipEventSynchronize(r.stop) != hipSuccess)
            return efg::fail(EF_EHIP, "ef_profile_read: event wait failed");
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
            return efg::fail(EF_EHIP, "ef_profile_read: elapsed time failed");
        sum += ms;
        ++cnt;
    }
    *total_ms = sum;
    *launches = cnt;
    return EF_OK;
}

}  // extern "C"
