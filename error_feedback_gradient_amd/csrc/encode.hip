// Index encodings of sparse packets, gfx950.
//
// "Gradient sparsification" page, index-encoding section: a bitmap with one
// bit per position, differences of consecutive indices in a variable-length
// code, and block-sparse marking (one bit per block, in-block positions only
// for non-empty blocks).
//
// Every variable-length output is built in three steps so that it is
// deterministic: per-chunk counts (one block per 4096 items), an exclusive
// scan of the chunk counts, then an ordered write where each thread owns 16
// consecutive items and a block scan gives its output offset.
#include <algorithm>

#include "common.hpp"

namespace efg {
namespace enc {

constexpr int kBlock = 256;
constexpr int kPer = 16;
constexpr int kChunk = kBlock * kPer;  // items per block-unit
constexpr int kMaxGrid = 4096;

inline unsigned grid_for(int64_t items, int64_t per_block) {
    int64_t g = cdiv(std::max<int64_t>(items, 1), per_block);
    return static_cast<unsigned>(std::min<int64_t>(g, kMaxGrid));
}

__global__ void k_zero_u32(uint32_t* p) { *p = 0; }

__global__ __launch_bounds__(kBlock) void k_fill_bytes(uint8_t* __restrict__ p, int64_t n, uint8_t v) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    const int64_t head = std::min<int64_t>(n, (16 - (reinterpret_cast<uintptr_t>(p) & 15u)) & 15u);
    const int64_t nv = (n - head) / 16;
    const uint32_t w = 0x01010101u * v;
    uint4* p4 = reinterpret_cast<uint4*>(p + head);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < nv; i += stride)
        p4[i] = make_uint4(w, w, w, w);
    if (blockIdx.x == 0) {
        if (threadIdx.x < head) p[threadIdx.x] = v;
        for (int64_t i = head + nv * 16 + threadIdx.x; i < n; i += kBlock) p[i] = v;
    }
}

// ------------------------------------------------------------------ bitmap
__global__ __launch_bounds__(kBlock) void k_bitmap_set(const int32_t* __restrict__ idx, int64_t k, int64_t n,
                                                       uint8_t* __restrict__ bits) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j < k; j += stride) {
        const int64_t i = idx[j];
        if (i < 0 || i >= n) continue;
        const int64_t byte = i >> 3;
        if (j > 0) {
            const int64_t ip = idx[j - 1];
            if (ip >= 0 && ip < n && (ip >> 3) == byte) continue;  // not the first entry of its byte
        }
        uint32_t v = 0;
        for (int64_t t = j; t < k && t < j + 8; ++t) {
            const int64_t it = idx[t];
            if (it < 0 || it >= n || (it >> 3) != byte) break;
            v |= 1u << (it & 7);
        }
        bits[byte] = static_cast<uint8_t>(v);
    }
}

// The thread's kPer bitmap bytes from byte b0, limited to nbits bits (bytes
// past the end count as 0).  All loads are issued before any is used: a byte
// past the end reads the last byte instead (nbits >= 1).
__device__ __forceinline__ void load_bits(const uint8_t* bits, int64_t nbits, int64_t b0, uint32_t (&v)[kPer]) {
    const int64_t nbytes = (nbits + 7) / 8;
#pragma unroll
    for (int t = 0; t < kPer; ++t) v[t] = bits[min(b0 + t, nbytes - 1)];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
        const int64_t valid = nbits - (b0 + t) * 8;
        v[t] = valid <= 0 ? 0u : valid < 8 ? v[t] & ((1u << valid) - 1u) : v[t];
    }
}

__global__ __launch_bounds__(kBlock) void k_bm_count(const uint8_t* __restrict__ bits, int64_t nbits,
                                                     int64_t nchunks, uint32_t* __restrict__ cnt) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        if (nbits == 0) {
            if (threadIdx.x == 0) cnt[c] = 0;
            continue;
        }
        uint32_t s = 0;
        const int64_t b0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        uint32_t v[kPer];
        load_bits(bits, nbits, b0, v);
#pragma unroll
        for (int t = 0; t < kPer; ++t) s += __popc(v[t]);
        uint32_t total;
        block_excl_scan<kBlock>(s, lds, &total);
        if (threadIdx.x == 0) cnt[c] = total;
    }
}

// writes set-bit positions (plus `add`, as int32) at out[off ...], bounded by cap;
// with `blk` set the positions go to a uint32 list instead
__global__ __launch_bounds__(kBlock) void k_bm_write(const uint8_t* __restrict__ bits, int64_t nbits,
                                                     int64_t nchunks, const uint32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ out, int64_t cap) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    if (nbits == 0) return;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t b0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        uint32_t v[kPer];
        load_bits(bits, nbits, b0, v);
        uint32_t s = 0;
#pragma unroll
        for (int t = 0; t < kPer; ++t) s += __popc(v[t]);
        uint32_t total;
        int64_t pos = static_cast<int64_t>(cnt[c]) + block_excl_scan<kBlock>(s, lds, &total);
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            uint32_t w = v[t];
            while (w) {
                const int b = __ffs(w) - 1;
                w &= w - 1;
                if (pos < cap) out[pos] = static_cast<int32_t>((b0 + t) * 8 + b);
                ++pos;
            }
        }
    }
}

// ------------------------------------------------------------------ delta
__device__ __forceinline__ uint32_t leb_len(uint32_t d) {
    return d < (1u << 7) ? 1u : d < (1u << 14) ? 2u : d < (1u << 21) ? 3u : d < (1u << 28) ? 4u : 5u;
}

// Differences idx[j] - idx[j - 1] (idx[-1] = 0) of the thread's kPer entries
// from j0; entries past k get 0 and are not used.  All loads are issued
// before any is used: a position outside [0, k) reads entry k - 1 (k >= 1).
__device__ __forceinline__ void load_deltas(const int32_t* idx, int64_t k, int64_t j0, uint32_t (&d)[kPer]) {
    int32_t v[kPer + 1];
#pragma unroll
    for (int t = 0; t <= kPer; ++t) v[t] = idx[min(max(j0 + t - 1, static_cast<int64_t>(0)), k - 1)];
    if (j0 == 0) v[0] = 0;
#pragma unroll
    for (int t = 0; t < kPer; ++t)
        d[t] = static_cast<uint32_t>(static_cast<int64_t>(v[t + 1]) - static_cast<int64_t>(v[t]));
}

__global__ __launch_bounds__(kBlock) void k_de_count(const int32_t* __restrict__ idx, int64_t k, int64_t nchunks,
                                                     uint32_t* __restrict__ cnt) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        if (k == 0) {
            if (threadIdx.x == 0) cnt[c] = 0;
            continue;
        }
        const int64_t j0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        uint32_t d[kPer];
        load_deltas(idx, k, j0, d);
        uint32_t s = 0;
#pragma unroll
        for (int t = 0; t < kPer; ++t) s += j0 + t < k ? leb_len(d[t]) : 0u;
        uint32_t total;
        block_excl_scan<kBlock>(s, lds, &total);
        if (threadIdx.x == 0) cnt[c] = total;
    }
}

__global__ __launch_bounds__(kBlock) void k_de_write(const int32_t* __restrict__ idx, int64_t k, int64_t nchunks,
                                                     const uint32_t* __restrict__ cnt, uint8_t* __restrict__ out) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    if (k == 0) return;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t j0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        uint32_t dl[kPer];
        load_deltas(idx, k, j0, dl);
        uint32_t s = 0;
#pragma unroll
        for (int t = 0; t < kPer; ++t) s += j0 + t < k ? leb_len(dl[t]) : 0u;
        uint32_t total;
        int64_t pos = static_cast<int64_t>(cnt[c]) + block_excl_scan<kBlock>(s, lds, &total);
        for (int t = 0; t < kPer && j0 + t < k; ++t) {
            uint32_t d = dl[t];
            for (;;) {
                const uint32_t low = d & 0x7fu;
                d >>= 7;
                if (d) {
                    out[pos++] = static_cast<uint8_t>(low | 0x80u);
                } else {
                    out[pos++] = static_cast<uint8_t>(low);
                    break;
                }
            }
        }
    }
}

// The thread's kPer stream bytes from b0 and the 5 before them (a varint that
// ends in the thread's range starts at most 4 bytes before it; one more byte
// tells whether it is longer than 5 bytes).  w[5 + t] is byte b0 + t; bytes
// before the stream read as 0 (no continuation bit), bytes past its end are
// not used.  All loads are issued before any is used: a position outside
// [0, nbytes) reads byte nbytes - 1 (nbytes >= 1).
constexpr int kWin = kPer + 5;
__device__ __forceinline__ void load_window(const uint8_t* in, int64_t nbytes, int64_t b0, uint32_t (&w)[kWin]) {
#pragma unroll
    for (int i = 0; i < kWin; ++i) w[i] = in[min(max(b0 - 5 + i, static_cast<int64_t>(0)), nbytes - 1)];
#pragma unroll
    for (int i = 0; i < 5; ++i)
        if (b0 - 5 + i < 0) w[i] = 0;
}

// value of the varint that ends at terminator byte w[p] (p >= 5): back over at
// most 4 continuation bytes, the first byte the least significant; sets *bad
// when the byte before those 4 continues it too (longer than 5 bytes)
__device__ __forceinline__ uint64_t varint_ending_at(const uint32_t (&w)[kWin], int p, bool* bad) {
    uint64_t v = w[p] & 0x7fu;
    bool cont = true;
#pragma unroll
    for (int j = 1; j <= 4; ++j) {
        cont = cont && (w[p - j] & 0x80u);
        if (cont) v = (v << 7) | (w[p - j] & 0x7fu);
    }
    if (cont && (w[p - 5] & 0x80u)) *bad = true;
    return v;
}

__global__ __launch_bounds__(kBlock) void k_dd_count(const uint8_t* __restrict__ in, int64_t nbytes,
                                                     int64_t nchunks, uint32_t* __restrict__ tcnt,
                                                     uint64_t* __restrict__ dsum, uint32_t* __restrict__ status) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    __shared__ uint64_t lds64[kBlock / kWave + 1];
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        if (nbytes == 0) {
            if (threadIdx.x == 0) {
                tcnt[c] = 0;
                dsum[c] = 0;
            }
            continue;
        }
        const int64_t b0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        uint32_t w[kWin];
        load_window(in, nbytes, b0, w);
        uint32_t s = 0;
        uint64_t d = 0;
        bool bad = false;
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            if (b0 + t < nbytes && !(w[5 + t] & 0x80u)) {
                ++s;
                d += varint_ending_at(w, 5 + t, &bad);
            }
        }
        if (bad && status) atomicOr(status, 1u);
        uint32_t total;
        uint64_t total64;
        block_excl_scan<kBlock>(s, lds, &total);
        block_excl_scan<kBlock>(d, lds64, &total64);
        if (threadIdx.x == 0) {
            tcnt[c] = total;
            dsum[c] = total64;
        }
    }
}

// Both chunk scans of the decoder (varint counts and delta sums) in one launch,
// then the stream checks: as many varints as k, and a terminated last varint.
__global__ __launch_bounds__(kScanThreads) void k_dd_scan(const uint8_t* __restrict__ in, int64_t nbytes, int64_t k,
                                                         int64_t nchunks, uint32_t* __restrict__ tcnt,
                                                         uint64_t* __restrict__ dsum,
                                                         uint32_t* __restrict__ status) {
    __shared__ uint32_t lds[kScanThreads / kWave + 1];
    __shared__ uint64_t lds64[kScanThreads / kWave + 1];
    const int64_t per = (nchunks + kScanThreads - 1) / kScanThreads;
    const int64_t i0 = min(nchunks, per * threadIdx.x), i1 = min(nchunks, i0 + per);
    uint32_t a = 0;
    uint64_t b = 0;
    for (int64_t i = i0; i < i1; ++i) {
        a += tcnt[i];
        b += dsum[i];
    }
    uint32_t ta;
    uint64_t tb;
    uint32_t ra = block_excl_scan<kScanThreads>(a, lds, &ta);
    uint64_t rb = block_excl_scan<kScanThreads>(b, lds64, &tb);
    for (int64_t i = i0; i < i1; ++i) {
        const uint32_t x = tcnt[i];
        const uint64_t y = dsum[i];
        tcnt[i] = ra;
        dsum[i] = rb;
        ra += x;
        rb += y;
    }
    if (threadIdx.x == 0 && status) {
        const bool bad = static_cast<int64_t>(ta) != k || (nbytes > 0 && (in[nbytes - 1] & 0x80u));
        if (bad) atomicOr(status, 1u);
    }
}

__global__ __launch_bounds__(kBlock) void k_dd_write(const uint8_t* __restrict__ in, int64_t nbytes,
                                                     int64_t nchunks, const uint32_t* __restrict__ tcnt,
                                                     const uint64_t* __restrict__ dsum, int64_t k,
                                                     int32_t* __restrict__ idx, uint32_t* __restrict__ status) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    __shared__ uint64_t lds64[kBlock / kWave + 1];
    if (nbytes == 0) return;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t b0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        uint32_t w[kWin];
        load_window(in, nbytes, b0, w);
        uint32_t s = 0;
        uint64_t d = 0;
        bool bad = false;
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            if (b0 + t < nbytes && !(w[5 + t] & 0x80u)) {
                ++s;
                d += varint_ending_at(w, 5 + t, &bad);
            }
        }
        uint32_t total;
        uint64_t total64;
        int64_t ord = static_cast<int64_t>(tcnt[c]) + block_excl_scan<kBlock>(s, lds, &total);
        uint64_t acc = dsum[c] + block_excl_scan<kBlock>(d, lds64, &total64);
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            if (b0 + t < nbytes && !(w[5 + t] & 0x80u)) {
                acc += varint_ending_at(w, 5 + t, &bad);
                if (acc > 0x7fffffffull) bad = true;
                if (ord < k) idx[ord] = static_cast<int32_t>(acc);
                ++ord;
            }
        }
        if (bad && status) atomicOr(status, 1u);
    }
}

// ------------------------------------------------------------------ blocks
// Encoder, for ascending indices in [0, n) (others are skipped and never cause a
// write outside the outputs).  One block per chunk of kChunk list entries;
// thread t holds entries [j0, j0 + kPer) of its chunk in registers (four
// 128-bit loads when idx is 16-byte aligned).  A "leader" is the first entry
// of a 256-element block; a "byte leader" the first entry of a mask byte
// (8 blocks, 2048 elements), which writes that whole byte.
template <bool VEC>
__device__ __forceinline__ void load_entries(const int32_t* __restrict__ idx, int64_t j0, int64_t k,
                                             int32_t (&v)[kPer], int32_t* prev) {
    if (VEC && j0 + kPer <= k) {
        const int4* p = reinterpret_cast<const int4*>(idx + j0);
#pragma unroll
        for (int q = 0; q < kPer / 4; ++q) {
            const int4 w = p[q];
            v[4 * q] = w.x;
            v[4 * q + 1] = w.y;
            v[4 * q + 2] = w.z;
            v[4 * q + 3] = w.w;
        }
    } else {
#pragma unroll
        for (int t = 0; t < kPer; ++t) v[t] = j0 + t < k ? idx[j0 + t] : -1;
    }
    *prev = j0 > 0 && j0 - 1 < k ? idx[j0 - 1] : -1;
}

__device__ __forceinline__ bool in_range(int64_t i, int64_t n) { return i >= 0 && i < n; }

// Runs of equal (entry >> shift) are walked backwards over the thread's
// entries; the run of its last entry may continue into the next thread's
// range, so that part is read from global memory first (at most `limit`
// entries).  An entry outside [0, n) ends a run.
__device__ __forceinline__ int64_t tail_run(const int32_t* __restrict__ idx, int64_t from, int64_t k, int64_t n,
                                            int64_t key, int shift, int64_t limit, uint32_t* bits) {
    int64_t len = 0;
    for (int64_t j = from; j < k && len < limit; ++j) {
        const int64_t ij = idx[j];
        if (!in_range(ij, n) || (ij >> shift) != key) break;
        ++len;
        if (bits) *bits |= 1u << ((ij >> 8) & 7);
    }
    return len;
}

template <bool VEC>
__global__ __launch_bounds__(kBlock) void k_be_count(const int32_t* __restrict__ idx, int64_t k, int64_t n,
                                                     int64_t nchunks, uint8_t* __restrict__ offs,
                                                     uint8_t* __restrict__ mask, uint32_t* __restrict__ cnt) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t j0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        int32_t v[kPer];
        int32_t prev;
        load_entries<VEC>(idx, j0, k, v, &prev);
        // mask byte of the run that ends this thread's entries, continued past them
        int64_t run_m = -1;
        uint32_t acc = 0;
        if (in_range(v[kPer - 1], n)) {
            run_m = v[kPer - 1] >> 11;
            tail_run(idx, j0 + kPer, k, n, run_m, 11, 2048, &acc);
        }
        uint32_t s = 0;
        uint32_t ob[kPer / 4] = {0, 0, 0, 0};
#pragma unroll
        for (int t = kPer - 1; t >= 0; --t) {
            const int64_t i = v[t];
            ob[t / 4] |= static_cast<uint32_t>(i & 255) << (8 * (t & 3));
            if (!in_range(i, n)) {
                run_m = -1;
                acc = 0;
                continue;
            }
            const int64_t m = i >> 11;
            if (m != run_m) {
                run_m = m;
                acc = 0;
            }
            acc |= 1u << ((i >> 8) & 7);
            const int64_t ip = t == 0 ? prev : v[t - 1];
            const bool ok_prev = in_range(ip, n);
            if (!ok_prev || (ip >> 8) != (i >> 8)) ++s;
            // the first entry of a mask byte writes the whole byte
            if (!ok_prev || (ip >> 11) != m) mask[m] = static_cast<uint8_t>(acc);
        }
        if (VEC && j0 + kPer <= k) {
            *reinterpret_cast<uint4*>(offs + j0) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
        } else {
            for (int t = 0; t < kPer && j0 + t < k; ++t) offs[j0 + t] = static_cast<uint8_t>(v[t] & 255);
        }
        uint32_t total;
        block_excl_scan<kBlock>(s, lds, &total);
        if (threadIdx.x == 0) cnt[c] = total;
    }
}

template <bool VEC>
__global__ __launch_bounds__(kBlock) void k_be_write(const int32_t* __restrict__ idx, int64_t k, int64_t n,
                                                     int64_t nchunks, const uint32_t* __restrict__ cnt,
                                                     uint8_t* __restrict__ counts_m1, int64_t cap) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t j0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        int32_t v[kPer];
        int32_t prev;
        load_entries<VEC>(idx, j0, k, v, &prev);
        // length of each entry's run of equal blocks from that entry on
        int64_t run_b = -1, run_len = 0;
        if (in_range(v[kPer - 1], n)) {
            run_b = v[kPer - 1] >> 8;
            run_len = tail_run(idx, j0 + kPer, k, n, run_b, 8, 256, nullptr);
        }
        uint32_t len_at[kPer];
        uint32_t lead = 0;
#pragma unroll
        for (int t = kPer - 1; t >= 0; --t) {
            const int64_t i = v[t];
            len_at[t] = 0;
            if (!in_range(i, n)) {
                run_b = -1;
                run_len = 0;
                continue;
            }
            const int64_t b = i >> 8;
            if (b != run_b) {
                run_b = b;
                run_len = 0;
            }
            ++run_len;
            len_at[t] = static_cast<uint32_t>(run_len < 256 ? run_len : 256);
            const int64_t ip = t == 0 ? prev : v[t - 1];
            if (!in_range(ip, n) || (ip >> 8) != b) lead |= 1u << t;
        }
        uint32_t total;
        int64_t ord = static_cast<int64_t>(cnt[c]) + block_excl_scan<kBlock>(__popc(lead), lds, &total);
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            if (!((lead >> t) & 1u)) continue;
            if (ord < cap) counts_m1[ord] = static_cast<uint8_t>(len_at[t] - 1);
            ++ord;
        }
    }
}

// Entries per non-empty block (count_m1 + 1) of the thread's kPer blocks from
// j0; 0 past the m blocks.  All loads are issued before any is used: a
// position past the end reads block m - 1 (none when m = 0).
__device__ __forceinline__ void load_counts(const uint8_t* counts_m1, int64_t m, int64_t j0, uint32_t (&cn)[kPer]) {
    if (m <= 0) {
#pragma unroll
        for (int t = 0; t < kPer; ++t) cn[t] = 0;
        return;
    }
#pragma unroll
    for (int t = 0; t < kPer; ++t) cn[t] = counts_m1[min(j0 + t, m - 1)] + 1u;
#pragma unroll
    for (int t = 0; t < kPer; ++t)
        if (j0 + t >= m) cn[t] = 0;
}

// per chunk of non-empty blocks: sum of (count_m1 + 1), limited to the device-side block count
__global__ __launch_bounds__(kBlock) void k_bd_count(const uint8_t* __restrict__ counts_m1,
                                                     const uint32_t* __restrict__ nblk, int64_t mcap,
                                                     int64_t nchunks, uint32_t* __restrict__ csum) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    const int64_t m = std::min<int64_t>(*nblk, mcap);
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t j0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        uint32_t cn[kPer];
        load_counts(counts_m1, m, j0, cn);
        uint32_t s = 0;
#pragma unroll
        for (int t = 0; t < kPer; ++t) s += cn[t];
        uint32_t total;
        block_excl_scan<kBlock>(s, lds, &total);
        if (threadIdx.x == 0) csum[c] = total;
    }
}

constexpr int kBdBatch = 8;  // outputs of a thread whose offsets are read at once
__global__ __launch_bounds__(kBlock) void k_bd_write(const uint8_t* __restrict__ counts_m1,
                                                     const uint8_t* __restrict__ offs,
                                                     const int32_t* __restrict__ blk,
                                                     const uint32_t* __restrict__ nblk, int64_t mcap,
                                                     int64_t nchunks, const uint32_t* __restrict__ csum, int64_t k,
                                                     int32_t* __restrict__ idx) {
    __shared__ uint32_t lds[kBlock / kWave + 1];
    const int64_t m = std::min<int64_t>(*nblk, mcap);
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t j0 = c * kChunk + static_cast<int64_t>(threadIdx.x) * kPer;
        uint32_t cn[kPer];
        load_counts(counts_m1, m, j0, cn);
        int32_t bl[kPer];
#pragma unroll
        for (int t = 0; t < kPer; ++t) bl[t] = m > 0 ? blk[min(j0 + t, m - 1)] : 0;
        uint32_t s = 0;
#pragma unroll
        for (int t = 0; t < kPer; ++t) s += cn[t];
        uint32_t total;
        const int64_t pos = static_cast<int64_t>(csum[c]) + block_excl_scan<kBlock>(s, lds, &total);
        // The thread's outputs [pos, pos + s) below k, kBdBatch at a time with
        // every offset load of a batch issued before any is used.  Output q
        // belongs to the last of the thread's blocks that starts at or before
        // it (blocks past m hold nothing and come last).
        uint32_t first[kPer];
        uint32_t run = 0;
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            first[t] = run;
            run += cn[t];
        }
        const int64_t lim = std::min<int64_t>(pos + s, k);
        for (int64_t p0 = pos; p0 < lim; p0 += kBdBatch) {
            uint32_t o[kBdBatch];
#pragma unroll
            for (int u = 0; u < kBdBatch; ++u) o[u] = offs[std::min<int64_t>(p0 + u, lim - 1)];
#pragma unroll
            for (int u = 0; u < kBdBatch; ++u) {
                if (p0 + u >= lim) break;
                const uint32_t q = static_cast<uint32_t>(p0 + u - pos);
                int32_t b = bl[0];
#pragma unroll
                for (int t = 1; t < kPer; ++t) b = first[t] <= q ? bl[t] : b;
                idx[p0 + u] = b * 256 + static_cast<int32_t>(o[u]);
            }
        }
    }
}

}  // namespace enc
}  // namespace efg

using namespace efg;
using namespace efg::enc;

extern "C" {

int encode_bitmap(const int32_t* idx, int64_t k, int64_t n, uint8_t* bits, void* stream) {
    if (n < 0 || n > kMaxElems || k < 0) return fail(EF_EINVAL, "encode_bitmap: bad sizes n=%lld k=%lld",
                                                     (long long)n, (long long)k);
    if (n > 0 && !bits) return fail(EF_EINVAL, "encode_bitmap: bits must not be NULL");
    if (k > 0 && !idx) return fail(EF_EINVAL, "encode_bitmap: idx must not be NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nbytes = (n + 7) / 8;
    if (nbytes == 0) return EF_OK;
    EF_TRY(launch("bitmap_clear", k_fill_bytes, dim3(grid_for(nbytes, kBlock * 16)), dim3(kBlock), s, bits, nbytes,
                  static_cast<uint8_t>(0)));
    if (k == 0) return EF_OK;
    return launch("bitmap_set", k_bitmap_set, dim3(grid_for(k, kBlock)), dim3(kBlock), s, idx, k, n, bits);
}

size_t decode_bitmap_workspace_bytes(int64_t n) {
    if (n < 0) return 0;
    const int64_t nchunks = std::max<int64_t>(1, cdiv((n + 7) / 8, kChunk));
    return round_up(static_cast<size_t>(nchunks + 1) * 4, 256);
}

static int bitmap_decode_into(const uint8_t* bits, int64_t nbits, int32_t* out, int64_t cap, int64_t* k_out,
                              uint32_t* k_out32, uint32_t* cnt, hipStream_t s) {
    const int64_t nbytes = (nbits + 7) / 8;
    const int64_t nchunks = std::max<int64_t>(1, cdiv(nbytes, kChunk));
    EF_TRY(launch("bitmap_count", k_bm_count, dim3(grid_for(nchunks, 1)), dim3(kBlock), s, bits, nbits, nchunks, cnt));
    EF_TRY(launch("bitmap_scan", k_excl_scan<uint32_t>, dim3(1), dim3(kScanThreads), s, cnt, nchunks, k_out32, k_out));
    return launch("bitmap_write", k_bm_write, dim3(grid_for(nchunks, 1)), dim3(kBlock), s, bits, nbits, nchunks,
                  static_cast<const uint32_t*>(cnt), out, cap);
}

int decode_bitmap(const uint8_t* bits, int64_t n, int32_t* idx, int64_t k_cap, int64_t* k_out, void* ws,
                  size_t ws_bytes, void* stream) {
    if (n < 0 || n > kMaxElems || k_cap < 0) return fail(EF_EINVAL, "decode_bitmap: bad sizes");
    if (!k_out) return fail(EF_EINVAL, "decode_bitmap: k_out must not be NULL");
    if (n > 0 && !bits) return fail(EF_EINVAL, "decode_bitmap: bits must not be NULL");
    if (k_cap > 0 && !idx) return fail(EF_EINVAL, "decode_bitmap: idx must not be NULL");
    const size_t need = decode_bitmap_workspace_bytes(n);
    if (!ws || ws_bytes < need) return fail(EF_EWS, "decode_bitmap: workspace %zu < %zu bytes", ws_bytes, need);
    return bitmap_decode_into(bits, n, idx, k_cap, k_out, nullptr, static_cast<uint32_t*>(ws),
                              static_cast<hipStream_t>(stream));
}

int64_t encode_delta_bound(int64_t k) { return k < 0 ? 0 : 5 * k; }

size_t delta_workspace_bytes(int64_t m) {
    if (m < 0) return 0;
    const int64_t nchunks = std::max<int64_t>(1, cdiv(m, kChunk));
    // uint32 counts, uint64 sums, two totals
    return round_up(static_cast<size_t>(nchunks + 1) * 4, 256) + round_up(static_cast<size_t>(nchunks + 1) * 8, 256) +
           256;
}

int encode_delta(const int32_t* idx, int64_t k, uint8_t* out, int64_t* nbytes_out, void* ws, size_t ws_bytes,
                 void* stream) {
    if (k < 0 || k > kMaxElems) return fail(EF_EINVAL, "encode_delta: bad k");
    if (!nbytes_out) return fail(EF_EINVAL, "encode_delta: nbytes_out must not be NULL");
    if (k > 0 && (!idx || !out)) return fail(EF_EINVAL, "encode_delta: idx and out must not be NULL");
    const size_t need = delta_workspace_bytes(k);
    if (!ws || ws_bytes < need) return fail(EF_EWS, "encode_delta: workspace %zu < %zu bytes", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t* cnt = static_cast<uint32_t*>(ws);
    const int64_t nchunks = std::max<int64_t>(1, cdiv(k, kChunk));
    EF_TRY(launch("delta_count", k_de_count, dim3(grid_for(nchunks, 1)), dim3(kBlock), s, idx, k, nchunks, cnt));
    EF_TRY(launch("delta_scan", k_excl_scan<uint32_t>, dim3(1), dim3(kScanThreads), s, cnt, nchunks,
                  static_cast<uint32_t*>(nullptr), nbytes_out));
    if (k == 0) return EF_OK;
    return launch("delta_write", k_de_write, dim3(grid_for(nchunks, 1)), dim3(kBlock), s, idx, k, nchunks,
                  static_cast<const uint32_t*>(cnt), out);
}

int decode_delta(const uint8_t* in, int64_t nbytes, int64_t k, int32_t* idx, uint32_t* status, void* ws,
                 size_t ws_bytes, void* stream) {
    if (k < 0 || k > kMaxElems || nbytes < 0) return fail(EF_EINVAL, "decode_delta: bad sizes");
    if (nbytes > 0 && !in) return fail(EF_EINVAL, "decode_delta: in must not be NULL");
    if (k > 0 && !idx) return fail(EF_EINVAL, "decode_delta: idx must not be NULL");
    const size_t need = delta_workspace_bytes(nbytes);
    if (!ws || ws_bytes < need) return fail(EF_EWS, "decode_delta: workspace %zu < %zu bytes", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nchunks = std::max<int64_t>(1, cdiv(nbytes, kChunk));
    uint8_t* W = static_cast<uint8_t*>(ws);
    uint32_t* tcnt = reinterpret_cast<uint32_t*>(W);
    uint64_t* dsum = reinterpret_cast<uint64_t*>(W + round_up(static_cast<size_t>(nchunks + 1) * 4, 256));
    if (status) EF_TRY(launch("delta_zero", k_zero_u32, dim3(1), dim3(1), s, status));
    EF_TRY(launch("delta_dcount", k_dd_count, dim3(grid_for(nchunks, 1)), dim3(kBlock), s, in, nbytes, nchunks, tcnt,
                  dsum, status));
    EF_TRY(launch("delta_dscan", k_dd_scan, dim3(1), dim3(kScanThreads), s, in, nbytes, k, nchunks, tcnt, dsum,
                  status));
    if (nbytes == 0) return EF_OK;
    return launch("delta_dwrite", k_dd_write, dim3(grid_for(nchunks, 1)), dim3(kBlock), s, in, nbytes, nchunks,
                  static_cast<const uint32_t*>(tcnt), static_cast<const uint64_t*>(dsum), k, idx, status);
}

// workspace: block flags (nb bytes), chunk counts, block list, block count
size_t blocks_workspace_bytes(int64_t k, int64_t n) {
    if (k < 0 || n < 0) return 0;
    const int64_t nb = cdiv(n, 256);
    const int64_t m = std::max<int64_t>(std::max<int64_t>(k, nb), 1);
    const int64_t nchunks = cdiv(m, kChunk) + cdiv((nb + 7) / 8 + 1, kChunk) + 1;
    return round_up(static_cast<size_t>(nb) + 16, 256) + round_up(static_cast<size_t>(nchunks + 1) * 4, 256) +
           round_up(static_cast<size_t>(nb + 1) * 4, 256) + 256;
}

int encode_blocks(const int32_t* idx, int64_t k, int64_t n, uint8_t* mask, uint8_t* counts_m1, uint8_t* offs,
                  int64_t* nblk_out, void* ws, size_t ws_bytes, void* stream) {
    if (n < 0 || n > kMaxElems || k < 0) return fail(EF_EINVAL, "encode_blocks: bad sizes");
    if (!nblk_out) return fail(EF_EINVAL, "encode_blocks: nblk_out must not be NULL");
    if (n > 0 && !mask) return fail(EF_EINVAL, "encode_blocks: mask must not be NULL");
    if (k > 0 && (!idx || !counts_m1 || !offs)) return fail(EF_EINVAL, "encode_blocks: NULL output");
    const size_t need = blocks_workspace_bytes(k, n);
    if (!ws || ws_bytes < need) return fail(EF_EWS, "encode_blocks: workspace %zu < %zu bytes", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nb = cdiv(n, 256);
    uint8_t* W = static_cast<uint8_t*>(ws);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(W + round_up(static_cast<size_t>(nb) + 16, 256));
    const int64_t nchunks = std::max<int64_t>(1, cdiv(k, kChunk));
    // mask bytes without any listed block stay zero; the others are written by their byte leader
    if (nb > 0)
        EF_TRY(launch("blocks_clear", k_fill_bytes, dim3(grid_for((nb + 7) / 8, kBlock * 16)), dim3(kBlock), s, mask,
                      (nb + 7) / 8, static_cast<uint8_t>(0)));
    const bool vec = aligned16(idx) && aligned16(offs);
    EF_TRY(launch("blocks_count", vec ? k_be_count<true> : k_be_count<false>, dim3(grid_for(nchunks, 1)),
                  dim3(kBlock), s, idx, k, n, nchunks, offs, mask, cnt));
    EF_TRY(launch("blocks_scan", k_excl_scan<uint32_t>, dim3(1), dim3(kScanThreads), s, cnt, nchunks,
                  static_cast<uint32_t*>(nullptr), nblk_out));
    if (k == 0) return EF_OK;
    return launch("blocks_write", vec ? k_be_write<true> : k_be_write<false>, dim3(grid_for(nchunks, 1)),
                  dim3(kBlock), s, idx, k, n, nchunks, static_cast<const uint32_t*>(cnt), counts_m1,
                  std::min(k, nb));
}

int decode_blocks(const uint8_t* mask, const uint8_t* counts_m1, const uint8_t* offs, int64_t n, int64_t k,
                  int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    if (n < 0 || n > kMaxElems || k < 0) return fail(EF_EINVAL, "decode_blocks: bad sizes");
    if (n > 0 && !mask) return fail(EF_EINVAL, "decode_blocks: mask must not be NULL");
    if (k > 0 && (!idx || !counts_m1 || !offs)) return fail(EF_EINVAL, "decode_blocks: NULL argument");
    const size_t need = blocks_workspace_bytes(k, n);
    if (!ws || ws_bytes < need) return fail(EF_EWS, "decode_blocks: workspace %zu < %zu bytes", ws_bytes, need);
    const int64_t nb = cdiv(n, 256);
    if (nb == 0 || k == 0) return EF_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* W = static_cast<uint8_t*>(ws);
    const int64_t m = std::max<int64_t>(std::max<int64_t>(k, nb), 1);
    const int64_t nchunks_all = cdiv(m, kChunk) + cdiv((nb + 7) / 8 + 1, kChunk) + 1;
    uint32_t* cnt = reinterpret_cast<uint32_t*>(W + round_up(static_cast<size_t>(nb) + 16, 256));
    int32_t* blk = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(cnt) +
                                              round_up(static_cast<size_t>(nchunks_all + 1) * 4, 256));
    uint32_t* nblk = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(blk) +
                                                 round_up(static_cast<size_t>(nb + 1) * 4, 256));
    // 1. list of non-empty blocks from the mask
    EF_TRY(bitmap_decode_into(mask, nb, blk, nb, nullptr, nblk, cnt, s));
    // 2. prefix of block counts, 3. indices
    const int64_t nchunks = std::max<int64_t>(1, cdiv(std::min(k, nb), kChunk));
    const int64_t mcap = std::min(k, nb);
    EF_TRY(launch("blocks_dcount", k_bd_count, dim3(grid_for(nchunks, 1)), dim3(kBlock), s, counts_m1,
                  static_cast<const uint32_t*>(nblk), mcap, nchunks, cnt));
    EF_TRY(launch("blocks_dscan", k_excl_scan<uint32_t>, dim3(1), dim3(kScanThreads), s, cnt, nchunks,
                  static_cast<uint32_t*>(nullptr), static_cast<int64_t*>(nullptr)));
    return launch("blocks_dwrite", k_bd_write, dim3(grid_for(nchunks, 1)), dim3(kBlock), s, counts_m1, offs,
                  static_cast<const int32_t*>(blk), static_cast<const uint32_t*>(nblk), mcap, nchunks,
                  static_cast<const uint32_t*>(cnt), k, idx);
}

}  // extern "C"
