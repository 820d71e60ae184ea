/*
 * CPU ORACLE for error-feedback gradient compression.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, single-threaded
 * statement of what the GPU library must compute.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the GPU library never
 * does, and this file includes nothing from it.
 *
 * Build:  gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * x86-64 scalar SSE float arithmetic is IEEE binary32, round to nearest even,
 * with subnormals kept (no FTZ/DAZ), so every float expression below rounds
 * exactly once per operation and no multiply is fused into an add.
 *
 * Sources ("pages"):
 *   [SPARSE] "梯度稀疏化：只传输重要的梯度元素" (gradient sparsification: send only
 *            the important gradient elements).
 *   [ONEBIT] "1bit Adam梯度压缩技术原理与分布式训练优化" (1-bit Adam gradient
 *            compression and distributed training).
 *
 * Readings taken where the pages leave a step open are marked READING.
 * Every function here has a pin in tests/ (brute force, closed forms,
 * invariants or an independent library routine); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENOMEM 2

static uint32_t f2u(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }

/* Magnitude key: the IEEE bit pattern without its sign bit.  For finite
 * values it orders exactly like |x| (+0 and -0 share key 0); +inf sits above
 * every finite value and NaN above +inf.
 * READING: the pages rank by absolute value and never say how to compare
 * +-0, inf or NaN; this key gives every value a fixed place. */
static uint32_t mag_key(float x) { return f2u(x) & 0x7fffffffu; }

static int is_nonfinite(float x) { return (f2u(x) & 0x7f800000u) == 0x7f800000u; }

typedef struct { uint32_t key; int64_t i; } ranked;

/* Ranking order of the selection: larger magnitude first; equal magnitudes
 * are ranked by lower index first.
 * READING: the pages do not say which of several equal magnitudes survives;
 * lower index first makes the kept set unique. */
static int rank_cmp(const void* pa, const void* pb) {
    const ranked* a = (const ranked*)pa;
    const ranked* b = (const ranked*)pb;
    if (a->key != b->key) return a->key > b->key ? -1 : 1;
    if (a->i != b->i) return a->i < b->i ? -1 : 1;
    return 0;
}

/*
 * Top-k sparsification with error feedback, one tensor.
 * [SPARSE] "详细算法流程：带误差补偿的Top-k稀疏化" (step-by-step algorithm),
 * steps 2-4, and "必不可少的误差补偿" (error compensation):
 *   x = g + e                        (add the carried residual back)
 *   keep the k entries of largest |x|, zero the others  ->  x~
 *   e' = x - x~                      (what was not sent this step)
 * [SPARSE] "梯度稀疏化的基本原理" step 3 and "Top-k 稀疏化": the message is the
 * k kept values plus their int32 positions.
 * READINGS: the sent value is x (residual included), not the raw g; indices
 * are written in ascending order; at a kept position e' is exactly +0.0
 * (x - x evaluated exactly); 0 <= k <= n.
 * Returns the count of non-finite x in *nonfinite (may be NULL).
 */
int orc_topk(const float* g, float* e, int64_t n, int64_t k,
             float* vals, int32_t* idx, uint32_t* nonfinite) {
    if (n < 0 || k < 0 || k > n || n > 0x7fffffffLL) return ORC_EINVAL;
    float* x = (float*)malloc((size_t)(n ? n : 1) * sizeof(float));
    ranked* order = (ranked*)malloc((size_t)(n ? n : 1) * sizeof(ranked));
    unsigned char* keep = (unsigned char*)calloc((size_t)(n ? n : 1), 1);
    if (!x || !order || !keep) { free(x); free(order); free(keep); return ORC_ENOMEM; }

    uint32_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        x[i] = g[i] + e[i];
        bad += (uint32_t)is_nonfinite(x[i]);
        order[i].key = mag_key(x[i]);
        order[i].i = i;
    }
    qsort(order, (size_t)n, sizeof(ranked), rank_cmp);
    for (int64_t j = 0; j < k; ++j) keep[order[j].i] = 1;

    int64_t out = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (keep[i]) {
            vals[out] = x[i];
            idx[out] = (int32_t)i;
            ++out;
            e[i] = 0.0f;
        } else {
            e[i] = x[i];
        }
    }
    if (nonfinite) *nonfinite = bad;
    free(x); free(order); free(keep);
    return ORC_OK;
}

/*
 * Layer-wise top-k: every tensor of a packed gradient is sparsified on its own
 * with its own k.  [SPARSE] "分层阈值与自适应稀疏率" and "分层自适应Top-k"
 * (per-layer top-k); [ONEBIT] "4.2 通信协议优化" item 1 (many tensors packed
 * into one contiguous buffer).
 * seg_off[nseg+1] are element offsets into the packed buffer, seg_k[nseg] the
 * per-tensor k.  Outputs are concatenated in tensor order.
 * READING: indices are positions in the packed buffer (tensor offset + local).
 */
int orc_topk_segmented(const float* g, float* e, int32_t nseg,
                       const int64_t* seg_off, const int64_t* seg_k,
                       float* vals, int32_t* idx, uint32_t* nonfinite) {
    if (nseg < 0) return ORC_EINVAL;
    int64_t out = 0;
    uint32_t bad_total = 0;
    for (int32_t s = 0; s < nseg; ++s) {
        int64_t off = seg_off[s], n = seg_off[s + 1] - seg_off[s], k = seg_k[s];
        uint32_t bad = 0;
        int rc = orc_topk(g + off, e + off, n, k, vals + out, idx + out, &bad);
        if (rc) return rc;
        for (int64_t j = 0; j < k; ++j) idx[out + j] += (int32_t)off;
        out += k;
        bad_total += bad;
    }
    if (nonfinite) *nonfinite = bad_total;
    return ORC_OK;
}

/*
 * 1-bit sign compression with an averaged error buffer and momentum.
 * [ONEBIT] "2.1 量化与误差补偿机制" (quantisation and error compensation):
 *   q     = sign(g + e)
 *   delta = (g + e) - q
 *   e'    = beta1 * e + (1 - beta1) * delta
 * [ONEBIT] "2.2 动量修正策略" (momentum correction):
 *   m'    = beta1 * m + (1 - beta1) * q
 * [ONEBIT] "3.2 核心算法实现细节" (implementation details): the gradient is
 * clipped to +-clip (5.0 by default) before quantisation, a NaN check follows
 * the error update, the quantised gradient is stored as int8; the error update
 * is written as (e * beta1) + (delta * (1 - beta1)).
 * [ONEBIT] "1. 梯度压缩技术背景": 32 bits become 1 bit per element.
 * READINGS: the clip applies to the raw gradient before e is added; sign(+-0)
 * and sign(NaN) are 0; each product and each sum is rounded to float32 on its
 * own (no fused multiply-add); (1 - beta1) is itself a float32 value; the
 * packed bit is 1 exactly when q = +1, least significant bit first, pad bits
 * zero; non-finite e' and m' are counted, not trapped.
 * sign_out and bits may be NULL.  m may be NULL: the momentum is then left to
 * the step that follows the exchange of the signs (orc_onebit_adam_update).
 */
int orc_sign(const float* g, float* e, float* m, int64_t n, float beta1, float clip,
             int8_t* sign_out, uint8_t* bits, uint32_t* nonfinite) {
    if (n < 0) return ORC_EINVAL;
    const float c = 1.0f - beta1;
    uint32_t bad = 0;
    if (bits) memset(bits, 0, (size_t)((n + 7) / 8));
    for (int64_t i = 0; i < n; ++i) {
        float gi = g[i];
        if (gi > clip) gi = clip;
        else if (gi < -clip) gi = -clip;
        float x = gi + e[i];
        int s = (x > 0.0f) - (x < 0.0f);
        float q = (float)s;
        float delta = x - q;
        float ea = beta1 * e[i];
        float eb = c * delta;
        float en = ea + eb;
        e[i] = en;
        bad += (uint32_t)is_nonfinite(en);
        if (m) {
            float ma = beta1 * m[i];
            float mb = c * q;
            float mn = ma + mb;
            m[i] = mn;
            bad += (uint32_t)is_nonfinite(mn);
        }
        if (sign_out) sign_out[i] = (int8_t)s;
        if (bits && s == 1) bits[i >> 3] |= (uint8_t)(1u << (i & 7));
    }
    if (nonfinite) *nonfinite = bad;
    return ORC_OK;
}

/*
 * Receiver-side aggregation: the values of all packets are added into the
 * dense buffer at their indices.  [SPARSE] "梯度稀疏化的基本原理" (sum the
 * values that share an index) and "详细算法流程" step 6.
 * Packet p occupies entries [pk_off[p], pk_off[p+1]) of vals/idx.
 * READINGS: G keeps its previous contents (the caller zeroes it); additions to
 * one index happen in packet order, one rounding each.
 */
int orc_decode(float* G, int64_t n, int32_t npk, const float* vals,
               const int32_t* idx, const int64_t* pk_off) {
    if (n < 0 || npk < 0) return ORC_EINVAL;
    for (int32_t p = 0; p < npk; ++p) {
        for (int64_t j = pk_off[p]; j < pk_off[p + 1]; ++j) {
            int64_t i = idx[j];
            if (i < 0 || i >= n) return ORC_EINVAL;
            G[i] = G[i] + vals[j];
        }
    }
    return ORC_OK;
}

/*
 * Parameter update with the aggregated gradient: w = w - lr * G.
 * [SPARSE] "详细算法流程" step 7.
 * READING: lr * G is rounded to float32, then subtracted (two roundings).
 */
int orc_sgd(float* w, const float* G, int64_t n, float lr) {
    if (n < 0) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        float step = lr * G[i];
        w[i] = w[i] - step;
    }
    return ORC_OK;
}

/*
 * Bitmap index encoding: one bit per element position.
 * [SPARSE] "索引编码压缩" (index encoding), the bitmap item.
 * READING: bit (i mod 8) of byte i/8, least significant bit first; ceil(n/8)
 * bytes; pad bits zero.
 */
int orc_bitmap_encode(const int32_t* idx, int64_t k, int64_t n, uint8_t* bits) {
    if (n < 0 || k < 0) return ORC_EINVAL;
    memset(bits, 0, (size_t)((n + 7) / 8));
    for (int64_t j = 0; j < k; ++j) {
        int64_t i = idx[j];
        if (i < 0 || i >= n) return ORC_EINVAL;
        bits[i >> 3] |= (uint8_t)(1u << (i & 7));
    }
    return ORC_OK;
}

/* Decode: every set bit, in ascending position.  Writes at most k_cap indices;
 * the number of set bits goes to *k_out. */
int orc_bitmap_decode(const uint8_t* bits, int64_t n, int32_t* idx, int64_t k_cap, int64_t* k_out) {
    if (n < 0 || k_cap < 0) return ORC_EINVAL;
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (bits[i >> 3] & (1u << (i & 7))) {
            if (k < k_cap) idx[k] = (int32_t)i;
            ++k;
        }
    }
    *k_out = k;
    return ORC_OK;
}

/*
 * Delta + variable-length index encoding.
 * [SPARSE] "索引编码压缩", the run-length / delta item: differences of
 * consecutive indices, each written with a variable number of bytes.
 * READINGS: the first difference is taken from 0; raw differences (no -1);
 * each difference is an unsigned LEB128 number (7 value bits per byte, low
 * group first, high bit set on every byte but the last), minimal length.
 * Requires strictly increasing indices >= 0.  *nbytes gets the stream length.
 */
int orc_delta_encode(const int32_t* idx, int64_t k, uint8_t* out, int64_t* nbytes) {
    if (k < 0) return ORC_EINVAL;
    int64_t pos = 0;
    int64_t prev = 0;
    for (int64_t j = 0; j < k; ++j) {
        int64_t cur = idx[j];
        if (cur < 0 || (j > 0 && cur <= prev)) return ORC_EINVAL;
        uint32_t d = (uint32_t)(cur - prev);
        for (;;) {
            uint8_t byte = (uint8_t)(d & 0x7fu);
            d >>= 7;
            if (d) { out[pos++] = (uint8_t)(byte | 0x80u); }
            else   { out[pos++] = byte; break; }
        }
        prev = cur;
    }
    *nbytes = pos;
    return ORC_OK;
}

/* Decode k differences and sum them back into indices. */
int orc_delta_decode(const uint8_t* in, int64_t nbytes, int64_t k, int32_t* idx) {
    if (k < 0 || nbytes < 0) return ORC_EINVAL;
    int64_t pos = 0;
    int64_t acc = 0;
    for (int64_t j = 0; j < k; ++j) {
        uint64_t d = 0;
        int shift = 0;
        for (;;) {
            if (pos >= nbytes || shift > 28) return ORC_EINVAL;
            uint8_t byte = in[pos++];
            d |= (uint64_t)(byte & 0x7fu) << shift;
            shift += 7;
            if (!(byte & 0x80u)) break;
        }
        acc += (int64_t)d;
        if (acc > 0x7fffffffLL) return ORC_EINVAL;
        idx[j] = (int32_t)acc;
    }
    return ORC_OK;
}

/*
 * Block-sparse index encoding with 256-element blocks.
 * [SPARSE] "索引编码压缩", the block item: one bit marks whether a block holds
 * any kept element; positions inside a block are sent only for blocks that
 * hold some.
 * READINGS: nb = ceil(n/256) blocks; mask bit b (least significant first,
 * ceil(nb/8) bytes) is set iff block b is non-empty; for each non-empty block
 * in ascending order one byte holds (count - 1); each kept index contributes
 * one byte (index - 256*block), in index order.  Values keep index order.
 * Requires strictly increasing indices in [0, n).  *nblk = non-empty blocks.
 */
int orc_blocks_encode(const int32_t* idx, int64_t k, int64_t n, uint8_t* mask,
                      uint8_t* counts_m1, uint8_t* offs, int64_t* nblk) {
    if (n < 0 || k < 0) return ORC_EINVAL;
    int64_t nb = (n + 255) / 256;
    memset(mask, 0, (size_t)((nb + 7) / 8));
    int64_t blocks = 0;
    int64_t j = 0;
    while (j < k) {
        int64_t i = idx[j];
        if (i < 0 || i >= n || (j > 0 && i <= idx[j - 1])) return ORC_EINVAL;
        int64_t b = i / 256;
        int64_t cnt = 0;
        while (j < k && idx[j] / 256 == b) {
            if (idx[j] >= n || (cnt > 0 && idx[j] <= idx[j - 1])) return ORC_EINVAL;
            offs[j] = (uint8_t)(idx[j] - 256 * b);
            ++cnt;
            ++j;
        }
        mask[b >> 3] |= (uint8_t)(1u << (b & 7));
        counts_m1[blocks++] = (uint8_t)(cnt - 1);
    }
    *nblk = blocks;
    return ORC_OK;
}

/* Inverse of orc_blocks_encode: rebuilds k ascending indices.  k_cap bounds the
 * output; *k_out gets the number of indices the stream describes. */
int orc_blocks_decode(const uint8_t* mask, const uint8_t* counts_m1, const uint8_t* offs,
                      int64_t n, int32_t* idx, int64_t k_cap, int64_t* k_out) {
    if (n < 0 || k_cap < 0) return ORC_EINVAL;
    int64_t nb = (n + 255) / 256;
    int64_t blocks = 0, k = 0;
    for (int64_t b = 0; b < nb; ++b) {
        if (!(mask[b >> 3] & (1u << (b & 7)))) continue;
        int64_t cnt = (int64_t)counts_m1[blocks++] + 1;
        for (int64_t t = 0; t < cnt; ++t, ++k) {
            if (k < k_cap) idx[k] = (int32_t)(256 * b + offs[k]);
        }
    }
    *k_out = k;
    return ORC_OK;
}

/*
 * 8-bit quantisation of a sent packet, with the quantisation error kept in the
 * residual.  [SPARSE] "与其他压缩技术的比较" (comparison with other compression):
 * systems combine top-k with 8-bit quantisation of the kept values.
 * READINGS: one symmetric scale per packet; amax = largest finite |v|;
 *   inv   = 127 / amax            (float32 division, correctly rounded)
 *   scale = amax / 127            (float32 division, correctly rounded)
 *   q     = rint(v * inv)         (float32 product, round half to even), clamped to [-127, 127]
 *   e[idx] = v - q * scale        (float32 product, then float32 difference)
 * A non-finite v, and every v when amax is 0 (all kept values are +-0) or when
 * no value is finite, gets q = 0 and keeps all of v in the residual.  A NaN
 * product (0 * inf, only when amax is below 127 / FLT_MAX) also gives q = 0.
 * *scale_out receives scale (0 when amax is 0 or absent).
 */
int orc_quantize_int8(const float* vals, const int32_t* idx, int64_t k, float* e, int8_t* q,
                      float* scale_out) {
    if (k < 0) return ORC_EINVAL;
    float amax = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        float a = fabsf(vals[j]);
        if (!is_nonfinite(vals[j]) && a > amax) amax = a;
    }
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    const float scale = amax > 0.0f ? amax / 127.0f : 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        float v = vals[j];
        int qi = 0;
        if (amax > 0.0f && !is_nonfinite(v)) {
            float t = v * inv;
            float r = rintf(t);
            if (r != r) r = 0.0f;  /* 0 * inf when amax is below 127 / FLT_MAX */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            qi = (int)r;
        }
        float deq = (float)qi * scale;
        q[j] = (int8_t)qi;
        e[idx[j]] = v - deq;
    }
    *scale_out = scale;
    return ORC_OK;
}

/*
 * Monitoring statistic: sum of squares of the finite entries of a float32
 * array, accumulated in float64 in index order.  [ONEBIT] "6.2" (a vanishing
 * L2 norm of the error buffer signals trouble) and "8" item 3 (watch the
 * error buffer's L2 norm).  Squares of float32 values are exact in float64;
 * only the summation rounds.
 */
double orc_sumsq(const float* a, int64_t n) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        if (!is_nonfinite(a[i])) s += (double)a[i] * (double)a[i];
    return s;
}

/*
 * Sum of |x_i| over the finite x_i, correctly rounded to float64.
 * READING: the pages normalise by the total magnitude without fixing how it
 * is summed; the exact sum rounded once is the one result that every
 * summation order can agree on.  Every finite float32 magnitude is an integer
 * multiple of 2^-149 below 2^128, so the exact sum of up to 2^31 of them is an
 * integer multiple of 2^-149 below 2^159: it is accumulated exactly in a
 * 320-bit fixed-point integer (ten 32-bit limbs, limb 0 holding 2^-149..2^-118)
 * and rounded to the nearest float64, ties to even, at the end.
 */
double orc_sum_abs_exact(const float* x, int64_t n) {
    uint64_t limb[11] = {0};
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = f2u(x[i]) & 0x7fffffffu;
        uint32_t ex = u >> 23;
        if (ex == 0xffu) continue;
        uint64_t mant = u & 0x7fffffu;
        int shift = 0;
        if (ex > 0) { mant |= 0x800000u; shift = (int)ex - 1; }
        /* |x| = mant * 2^(shift - 149) */
        int q = shift / 32, r = shift % 32;
        uint64_t v = mant << r; /* < 2^55 */
        limb[q] += v & 0xffffffffu;
        limb[q + 1] += v >> 32;
        for (int j = q; j < 10; ++j) { /* keep every limb below 2^32 */
            if (limb[j] >> 32) { limb[j + 1] += limb[j] >> 32; limb[j] &= 0xffffffffu; }
        }
    }
    /* Highest set bit of the 320-bit integer. */
    int top = -1;
    for (int j = 9; j >= 0 && top < 0; --j)
        if (limb[j]) for (int b = 31; b >= 0; --b) if ((limb[j] >> b) & 1u) { top = 32 * j + b; break; }
    if (top < 0) return 0.0;
    /* Take the 53 bits below and including 'top', then round on the rest. */
    uint64_t mant = 0;
    int sticky = 0, guard = 0;
    for (int b = top; b >= 0; --b) {
        int bit = (int)((limb[b / 32] >> (b % 32)) & 1u);
        if (b > top - 53) mant = (mant << 1) | (uint64_t)bit;
        else if (b == top - 53) guard = bit;
        else sticky |= bit;
    }
    int lsb_pos = top - 52; /* position of the last kept bit */
    if (lsb_pos < 0) lsb_pos = 0; /* 53 bits or fewer: mant holds every bit, exactly */
    if (guard && (sticky || (mant & 1u))) mant += 1; /* may carry to 2^53: ldexp still exact */
    return ldexp((double)mant, lsb_pos - 149);
}

/*
 * Philox4x32-10 counter-based generator, from its published definition
 * (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
 * 3", SC 2011): ten rounds of two 32x32->64 multiplications mixed with the
 * counter and a key bumped by two Weyl constants between rounds.
 */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* READING: the uniform draw u_i in [0, 1) for element i.  Philox is keyed by
 * the 64-bit seed (low word first) and run on the counter
 * {i div 4, 0, step low word, step high word}; element i takes output word
 * (i mod 4), keeps its top 24 bits and scales them by 2^-24, which is exact in
 * float32. */
float orc_uniform(uint64_t seed, uint64_t step, int64_t i) {
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    const uint32_t ctr[4] = {(uint32_t)(i / 4), 0u, (uint32_t)step, (uint32_t)(step >> 32)};
    uint32_t r[4];
    orc_philox4x32_10(ctr, key, r);
    return (float)(r[i % 4] >> 8) * 0x1p-24f;
}

/* READING: the keep probability of one element, in float32:
 * p = (float(k) * |x|) / S32, lowered to 1 when above it (IEEE comparisons, so
 * a NaN quotient is left alone and keeps nothing), and 0 for a non-finite x. */
float orc_keep_probability(float x, int64_t k, float S32) {
    if (is_nonfinite(x)) return 0.0f;
    float t = (float)k * fabsf(x);
    float p = t / S32;
    if (p > 1.0f) p = 1.0f;
    return p;
}

/*
 * Random sparsification with error feedback.  [SPARSE] "随机稀疏化" (random
 * sparsification): every element survives with a probability proportional to
 * its magnitude, scaled so that k elements survive on average; the error
 * compensation around it is the page's generic loop (add the residual, sparsify,
 * keep what was not sent).
 * READINGS:
 *   x_i = g_i + e_i (float32); S64 = orc_sum_abs_exact(x), S32 = float(S64);
 *   p_i = orc_keep_probability(x_i, k, S32); u_i = orc_uniform(seed, step, i);
 *   x_i is kept iff u_i < p_i (so p = 0 keeps nothing and p = 1 keeps always).
 *   Probabilities above 1 are clipped, so the expected count is k less what
 *   the clipped elements lose.  A kept element is sent as x_i, unscaled: the
 *   sparse tensor holds x on the kept positions and zero elsewhere, and its
 *   residual becomes +0; every other element keeps e' = x.  Kept elements are
 *   sent in index order; only the first cap of them are written, and kept
 *   elements beyond cap stay whole in the residual (they were not sent).
 * *count_out = number kept (may exceed cap); *sum_out = S32.
 */
int orc_random_sparsify(const float* g, float* e, int64_t n, int64_t k, uint64_t seed, uint64_t step,
                        int64_t cap, float* vals, int32_t* idx, int64_t* count_out, float* sum_out,
                        uint32_t* nonfinite) {
    if (n < 0 || k < 0 || cap < 0 || n > 0x7fffffffLL) return ORC_EINVAL;
    float* x = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!x) return ORC_ENOMEM;
    uint32_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        x[i] = g[i] + e[i];
        bad += (uint32_t)is_nonfinite(x[i]);
    }
    const float S32 = (float)orc_sum_abs_exact(x, n);
    int64_t count = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int keep = orc_uniform(seed, step, i) < orc_keep_probability(x[i], k, S32);
        if (keep && count < cap) {
            vals[count] = x[i];
            idx[count] = (int32_t)i;
            e[i] = 0.0f;
        } else {
            e[i] = x[i];
        }
        count += keep;
    }
    free(x);
    *count_out = count;
    *sum_out = S32;
    if (nonfinite) *nonfinite = bad;
    return ORC_OK;
}

/* The keep decision of orc_random_sparsify at chosen positions: keep[j] for
 * element pos[j], whose x = g + e is x[j], given S32.  Lets large inputs be
 * checked one sampled element at a time. */
int orc_random_keep_at(const float* x, const int64_t* pos, int64_t m, int64_t k, float S32, uint64_t seed,
                       uint64_t step, uint8_t* keep) {
    if (m < 0 || k < 0) return ORC_EINVAL;
    for (int64_t j = 0; j < m; ++j) {
        if (pos[j] < 0 || pos[j] > 0x7fffffffLL) return ORC_EINVAL;
        keep[j] = (uint8_t)(orc_uniform(seed, step, pos[j]) < orc_keep_probability(x[j], k, S32));
    }
    return ORC_OK;
}

/*
 * The parameter update shared by both Adam phases, per element:
 *   d = sqrt(v) / sqrt_bc2 + eps
 *   w' = w - step_size * (m / d)
 * READING: textbook Adam (Kingma and Ba, ICLR 2015, Algorithm 1: theta -=
 * alpha * mhat / (sqrt(vhat) + eps), mhat = m / (1 - beta1^t), vhat = v / (1 -
 * beta2^t)) with the two bias corrections folded into host scalars:
 * step_size = lr / (1 - beta1^t) and sqrt_bc2 = sqrt(1 - beta2^t_v), where t_v
 * is the step at which v was last updated.  Square root and divisions
 * correctly rounded float32, every operation rounded on its own.
 */
static float adam_param(float w, float m, float v, float step_size, float sqrt_bc2, float eps) {
    float r = sqrtf(v);
    float q = r / sqrt_bc2;
    float d = q + eps;
    float u = m / d;
    float s = step_size * u;
    return w - s;
}

/*
 * One full-precision Adam step (the warm-up phase).  [ONEBIT] "6.1 收敛不稳定问题"
 * trains its first steps at full precision before switching to 1-bit
 * compression; "3.1 关键数据结构设计" keeps momentum, variance, beta1, beta2,
 * eps and the step count.  READING: textbook Adam on the (averaged) gradient g:
 *   m' = beta1 * m + (1 - beta1) * g
 *   v' = beta2 * v + (1 - beta2) * (g * g)
 *   w' = adam_param(w, m', v', ...)
 * (1 - beta1) and (1 - beta2) are float32 values; no fused multiply-add.
 * Non-finite m', v', w' are counted.
 */
int orc_adam_step(const float* g, float* m, float* v, float* w, int64_t n, float beta1, float beta2,
                  float step_size, float sqrt_bc2, float eps, uint32_t* nonfinite) {
    if (n < 0) return ORC_EINVAL;
    const float c1 = 1.0f - beta1, c2 = 1.0f - beta2;
    uint32_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        float ma = beta1 * m[i];
        float mb = c1 * g[i];
        float mn = ma + mb;
        float g2 = g[i] * g[i];
        float va = beta2 * v[i];
        float vb = c2 * g2;
        float vn = va + vb;
        float wn = adam_param(w[i], mn, vn, step_size, sqrt_bc2, eps);
        m[i] = mn;
        v[i] = vn;
        w[i] = wn;
        bad += (uint32_t)is_nonfinite(mn) + (uint32_t)is_nonfinite(vn) + (uint32_t)is_nonfinite(wn);
    }
    if (nonfinite) *nonfinite = bad;
    return ORC_OK;
}

/*
 * One compression-phase step of 1-bit Adam after the signs were exchanged.
 * qsum[i] is the sum over the nworkers workers of their int8 signs q
 * (orc_sign with m = NULL), so the averaged compressed gradient is
 *   ghat = qsum / nworkers                      (float32 division)
 * [ONEBIT] "2.2 动量修正策略": m' = beta1 * m + (1 - beta1) * ghat.
 * READING: the pages list a variance in the state ("3.1 关键数据结构设计") but
 * give it no rule during compression.  This function keeps v frozen at its
 * value after warm-up (the choice of the published 1-bit Adam algorithm, made
 * outside these pages); v is read, never written.  w' = adam_param(w, m', v).
 * The other reading, v updated from ghat, is orc_adam_step fed ghat.
 * With one worker ghat = q and m' is exactly orc_sign's momentum.
 * 1 <= nworkers <= 127 (the sum fits int8).
 */
int orc_onebit_adam_update(const int8_t* qsum, int32_t nworkers, float* m, const float* v, float* w, int64_t n,
                           float beta1, float step_size, float sqrt_bc2, float eps, uint32_t* nonfinite) {
    if (n < 0 || nworkers < 1 || nworkers > 127) return ORC_EINVAL;
    const float c1 = 1.0f - beta1;
    const float nw = (float)nworkers;
    uint32_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        float ghat = (float)qsum[i] / nw;
        float ma = beta1 * m[i];
        float mb = c1 * ghat;
        float mn = ma + mb;
        float wn = adam_param(w[i], mn, v[i], step_size, sqrt_bc2, eps);
        m[i] = mn;
        w[i] = wn;
        bad += (uint32_t)is_nonfinite(mn) + (uint32_t)is_nonfinite(wn);
    }
    if (nonfinite) *nonfinite = bad;
    return ORC_OK;
}
