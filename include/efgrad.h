/*
 * efgrad — error-feedback gradient compression on one MI355X (gfx950).
 *
 * C ABI of libefgrad.so.  Every entry point takes plain pointers and sizes.
 *
 * Conventions shared by all calls
 * -------------------------------
 *  - Pointers are DEVICE pointers unless the comment says "host".  All device
 *    buffers belong to the caller; the library never allocates or frees them.
 *    Scratch memory comes from a caller-provided device workspace whose size
 *    the matching *_workspace_bytes() host query returns.  A workspace holds
 *    one call's scratch until that call's work on its stream has finished:
 *    calls in order on one stream may share a workspace; calls that can run
 *    at the same time (on different streams) need one each.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only ENQUEUES work on that stream and returns; results are
 *    valid once the caller synchronises the stream.  No call copies data
 *    device -> host, and none waits for the device, with one exception named
 *    at ef_topk_compress_segmented (its plan cache, beyond 16 table sets).
 *  - Sizes are int64_t.  Element indices are int32_t, so arrays that are
 *    indexed hold at most 2^31 - 1 elements.
 *  - float arrays read or written element-wise in bulk (g, e, m, w, G) must be
 *    16-byte aligned.  Outputs must not alias inputs unless stated.
 *  - Results are bit-identical from run to run and do not depend on launch
 *    configuration: no floating-point atomics are used anywhere.
 *  - Return value: EF_OK, or an error status with a message available from
 *    ef_last_error() (thread-local).  Argument checks happen on the host before
 *    anything is enqueued; on an error nothing is enqueued.
 *  - Floating-point data problems (Inf/NaN) are not call errors: the calls that
 *    can meet them count them into an optional device uint32 `nonfinite`
 *    (overwritten by each call).
 *  - HIP graph capture: every call only launches kernels (no memset, no host
 *    wait; ef_profile_enable records nothing on a stream under capture), so a
 *    captured call replays exactly like the eager one.
 *    ef_topk_compress_segmented with more than 11 tensors
 *    reads its cached plan from pinned host memory when called eagerly; under
 *    capture it passes the plan in kernel arguments instead (one small launch
 *    per 500 words, about 17 tensors), so a replay never depends on the cache.
 *
 * Sources cited below ("pages"):
 *   [SPARSE] "梯度稀疏化：只传输重要的梯度元素" — gradient sparsification.
 *   [ONEBIT] "1bit Adam梯度压缩技术原理与分布式训练优化" — 1-bit Adam.
 */
#ifndef EFGRAD_H
#define EFGRAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EF_OK 0
#define EF_EINVAL 1   /* bad argument (null pointer, size, alignment, k > n, ...) */
#define EF_EWS 2      /* workspace missing or smaller than the size query says   */
#define EF_EHIP 3     /* the HIP runtime rejected a launch                        */
#define EF_ENOTIMPL 4 /* reserved: an operation the library does not provide      */

/* Debug flag: take each call's exact fallback path even when its faster path
 * would have succeeded (top-k: the full-pass selection for every tensor;
 * random sparsification: see ef_random_sparsify).  Results do not change. */
#define EF_FLAG_FORCE_FALLBACK 1u

/* Message describing the last error returned on the calling thread. */
const char* ef_last_error(void);
/* Library version string. */
const char* ef_version(void);

/* ------------------------------------------------------------------------
 * Top-k sparsification with error feedback.
 * [SPARSE] section "详细算法流程：带误差补偿的Top-k稀疏化" (step-by-step
 * algorithm) steps 2-5, "必不可少的误差补偿" (error compensation),
 * "梯度稀疏化的基本原理" (basic principle) step 3, "Top-k 稀疏化".
 *
 * For i in [0, n):  x_i = g_i + e_i  (float32, round to nearest even).
 * The kept set S holds the k entries ranked first when entries are ordered by
 * larger |x| first (compared as the IEEE bit pattern without the sign bit, so
 * +0 == -0 and NaN > +Inf > every finite value) and, for equal |x|, by lower
 * index first.
 *   idx[0..k)  = S in ascending order                     (int32, output)
 *   vals[0..k) = x at those indices, bit for bit          (float32, output)
 *   e_i        = +0.0 for i in S, x_i otherwise           (in place)
 *   *nonfinite = number of i with x_i = +-Inf or NaN      (nullable)
 *   stats[0] = sum of vals^2, stats[1] = sum of new e^2   (device double[2],
 *              nullable; finite values only, float64; the monitoring signals of
 *              [ONEBIT] 6.2 and 8 item 3, computed in the same passes; the sums
 *              are reduced in a fixed order, so they repeat bit for bit)
 * g is read only.  0 <= k <= n <= 2^31 - 1.  vals/idx may be NULL when k = 0.
 * ws: device workspace of at least ef_topk_workspace_bytes(n, k) bytes, 256-byte
 * aligned; its contents on entry do not change the results.  A call leaves its
 * exact threshold in the workspace, and the next call on it uses that value
 * to sample the magnitudes around it at a finer resolution (error feedback
 * crowds values just below the threshold, and the finer sample keeps the
 * candidate set small there); any other contents only forgo that gain.  A
 * call that asks for stats does not use it, so its statistics depend on its
 * inputs alone.
 * flags: 0 or EF_FLAG_FORCE_FALLBACK.
 * ------------------------------------------------------------------------ */
size_t ef_topk_workspace_bytes(int64_t n, int64_t k);
int ef_topk_compress(const float* g, float* e, int64_t n, int64_t k, float* vals,
                     int32_t* idx, void* ws, size_t ws_bytes, uint32_t* nonfinite,
                     double* stats, uint32_t flags, void* stream);

/* Defensive count of the last top-k call on a workspace (ws; NULL = the
 * static scratch of ef_topk_compress_noalloc on the stream's device): the
 * number of indices that call found outside their tensor's range in its own
 * workspace entries and therefore did not write through.  0 unless something
 * else wrote to the workspace during the call.  *stray is a device uint32;
 * the copy is enqueued on `stream` after the calls before it. */
int ef_topk_workspace_status(const void* ws, uint32_t* stray, void* stream);

/* Which path each tensor of the last top-k call on a workspace took (ws of
 * ws_bytes bytes; NULL = the static scratch of ef_topk_compress_noalloc on the
 * stream's device, ws_bytes ignored), for monitoring how often the sample
 * misjudges the threshold.  nseg is the
 * number of tensors of that call (1 for ef_topk_compress).  out (device
 * uint32[2 * nseg]): out[2s] = 1 when tensor s took the exact full-pass
 * selection, else 0; out[2s + 1] = the candidates its streaming pass
 * collected (keys >= T_lo), 0 for a tensor with k = 0 or k = n.  The copy is
 * enqueued on `stream` after the calls before it; it reads what a call with
 * nseg tensors and at least one element left in the workspace.  EF_EWS when
 * ws_bytes is too small to hold the state of nseg tensors. */
int ef_topk_workspace_paths(const void* ws, size_t ws_bytes, int32_t nseg, uint32_t* out, void* stream);

/* ------------------------------------------------------------------------
 * Allocation-free top-k, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): ef_topk_compress without a workspace argument.
 *
 * Arguments and results are those of ef_topk_compress.  The scratch is one
 * static device array of EF_TOPK_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU the
 * library runs on, held until the process ends; the first call on a device
 * looks its address up (hipGetSymbolAddress).  A call whose scratch need,
 * ef_topk_workspace_bytes(n, k), exceeds the array returns EF_EWS before
 * enqueueing anything (n = 1e6, k = 1e4 needs 1.2 MB; n = 2^26, k = 2^16
 * 23 MB).  The call makes no hipMalloc, hipFree or other allocating call; a
 * one-tensor plan is built on the host stack.  Every call on one GPU uses
 * that GPU's array and leaves its contents behind (each call clears what it
 * needs cleared): calls that can overlap on one GPU (different streams) race
 * on the array and give wrong results, so serialise them.
 * ------------------------------------------------------------------------ */
#define EF_TOPK_NOALLOC_SCRATCH_BYTES (32u << 20)
int ef_topk_compress_noalloc(const float* g, float* e, int64_t n, int64_t k, float* vals,
                             int32_t* idx, uint32_t* nonfinite, double* stats, uint32_t flags,
                             void* stream);

/* ------------------------------------------------------------------------
 * Layer-wise top-k over many tensors packed in one buffer: the operation of
 * ef_topk_compress applied to every tensor on its own, all in one launch
 * sequence.  [SPARSE] "分层阈值与自适应稀疏率" and "分层自适应Top-k" (per-layer
 * top-k); [ONEBIT] "4.2 通信协议优化" item 1 (packing many tensors into one
 * contiguous buffer).
 *
 * seg_off (host, nseg+1 int64): tensor s occupies g/e[seg_off[s], seg_off[s+1]);
 *   non-decreasing, seg_off[nseg] <= 2^31 - 1.
 * seg_k (host, nseg int64): 0 <= seg_k[s] <= seg_off[s+1] - seg_off[s].
 * Output: tensor s's kept entries go to vals/idx[K_s, K_s + seg_k[s]) with
 *   K_s = seg_k[0] + ... + seg_k[s-1]; indices are positions in the packed
 *   buffer (seg_off[s] + local index), so idx is ascending overall.
 * *nonfinite counts over all tensors; stats (nullable) gets two doubles per
 * tensor, stats[2s] and stats[2s+1], as above.  The host tables are read during the
 * call only.  The per-tensor plan built from them is cached by the library
 * (16 distinct table sets, in pinned host memory it keeps for the life of the
 * process) and copied into the workspace by the call's first kernel, so
 * repeated calls with the same tables skip rebuilding it; the workspace
 * contents on entry still do not matter.  A call with a table set not in a
 * full cache reuses the least recently used entry and, if a queued call may
 * still read that entry, waits for that call's first kernel: the only case in
 * which a call waits for the device.
 * ------------------------------------------------------------------------ */
size_t ef_topk_segmented_workspace_bytes(int32_t nseg, const int64_t* seg_off,
                                         const int64_t* seg_k);
int ef_topk_compress_segmented(const float* g, float* e, int32_t nseg,
                               const int64_t* seg_off, const int64_t* seg_k,
                               float* vals, int32_t* idx, void* ws, size_t ws_bytes,
                               uint32_t* nonfinite, double* stats, uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * 1-bit sign compression with averaged error feedback and momentum.
 * [ONEBIT] "2.1 量化与误差补偿机制" (quantisation and error compensation),
 * "2.2 动量修正策略" (momentum correction), "3.2 核心算法实现细节"
 * (clip before quantisation, NaN check, int8 storage), section 1 (32 -> 1 bit).
 *
 * Per element, float32, each product and sum rounded on its own (no FMA):
 *   gc = min(max(g, -clip), clip)          NaN passes through; clip = +Inf: off
 *   x  = gc + e
 *   q  = sign(x) in {-1, 0, +1}            sign(+-0) = sign(NaN) = 0
 *   c  = 1 - beta1                         (a float32 value)
 *   e  = beta1*e + c*(x - q)               (in place)
 *   m  = beta1*m + c*q                     (in place; m may be NULL: compress
 *                                           only, for data-parallel 1-bit Adam
 *                                           where the momentum follows the
 *                                           exchange of the signs)
 *   sign_out[i] = q                        (int8, nullable)
 *   bits[i/8] bit (i%8) = (q == +1)        (uint8[ceil(n/8)], LSB first, pad 0, nullable)
 *   *nonfinite = count of non-finite new e plus non-finite new m (nullable)
 *                (stats: sum m'^2 is 0 when m is NULL)
 *   stats = {sum e'^2, sum m'^2, #(q = +1), #(q = -1)}  (device double[4],
 *           nullable; finite values only, float64, fixed-order sums; needs
 *           ws of ef_sign_workspace_bytes(n) bytes, 32-byte aligned; ws may be
 *           NULL when stats is NULL)
 * 0 <= n <= 2^31 - 1; 0 <= beta1 <= 1; clip > 0; sign_out 4-byte aligned.
 * ------------------------------------------------------------------------ */
size_t ef_sign_workspace_bytes(int64_t n);
int ef_sign_compress(const float* g, float* e, float* m, int64_t n, float beta1,
                     float clip, int8_t* sign_out, uint8_t* bits, uint32_t* nonfinite,
                     double* stats, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Adam around the 1-bit compression.  [ONEBIT] "3.1 关键数据结构设计" (the state
 * holds momentum, variance, beta1, beta2, eps and the step count), "2.2
 * 动量修正策略" (momentum on the compressed gradient) and "6.1 收敛不稳定问题" (full
 * precision for the first steps, then 1-bit compression).  The variance and
 * parameter rules are textbook Adam (Kingma and Ba, Algorithm 1), with the
 * bias corrections as host scalars:
 *   step_size = lr / (1 - beta1^t),   sqrt_bc2 = sqrt(1 - beta2^t_v)
 *   w = w - step_size * (m / (sqrt(v) / sqrt_bc2 + eps))
 * float32; square root and divisions correctly rounded, every other product
 * and sum rounded on its own; (1 - beta) is the float32 complement of beta.
 *
 * ef_adam_step: one full-precision (warm-up) step on the averaged gradient g:
 *   m = beta1*m + (1-beta1)*g;  v = beta2*v + (1-beta2)*(g*g);  w as above.
 * ef_onebit_adam_update: one compression-phase step once every worker's int8
 * signs (ef_sign_compress with m = NULL) were summed into qsum (exact integer
 * sum, 1 <= nworkers <= 127):
 *   ghat = qsum / nworkers;  m = beta1*m + (1-beta1)*ghat;  v unchanged
 *   (frozen at its value after warm-up, as the published 1-bit Adam does; the
 *   pages give v no rule here, and ef_onebit_adam_update_var is the other
 *   reading);  w as above.
 *   With nworkers = 1, m matches ef_sign_compress's fused momentum bit for bit.
 * *nonfinite (device uint32, nullable, overwritten) counts non-finite new m,
 * v (warm-up only) and w.  g, m, v, w 16-byte aligned; qsum 4-byte aligned;
 * 0 <= n <= 2^31 - 1; 0 <= beta <= 1; sqrt_bc2 > 0; eps >= 0.
 * ------------------------------------------------------------------------ */
/* The two host scalars of step t (1-based):
 *   *step_size = lr / (1 - beta1^t),  *sqrt_bc2 = sqrt(1 - beta2^t_v)
 * in float64 from the float32 betas (powers by pow, correctly rounded square
 * root), each rounded once to float32.  t_v = t while the variance is updated; once it is frozen, the last
 * warm-up step.  Host outputs.  0 <= beta < 1, t >= 1, t_v >= 1, lr finite. */
int ef_adam_scalars(double lr, float beta1, float beta2, int64_t t, int64_t t_v,
                    float* step_size, float* sqrt_bc2);
int ef_adam_step(const float* g, float* m, float* v, float* w, int64_t n, float beta1,
                 float beta2, float step_size, float sqrt_bc2, float eps, uint32_t* nonfinite,
                 void* stream);
int ef_onebit_adam_update(const int8_t* qsum, int32_t nworkers, float* m, const float* v,
                          float* w, int64_t n, float beta1, float step_size, float sqrt_bc2,
                          float eps, uint32_t* nonfinite, void* stream);
/* ef_onebit_adam_update_var: the compression-phase step with the variance
 * still updated, from the averaged compressed gradient (the pages list v in
 * the state but give no rule for it; this is textbook Adam fed ghat):
 *   ghat = qsum / nworkers;  m = beta1*m + (1-beta1)*ghat;
 *   v = beta2*v + (1-beta2)*(ghat*ghat);  w as above (t_v = t).
 * Every replica holds the same ghat, so v stays identical on all of them.
 * Same rounding, alignment and *nonfinite (m, v, w) rules as ef_adam_step. */
int ef_onebit_adam_update_var(const int8_t* qsum, int32_t nworkers, float* m, float* v,
                              float* w, int64_t n, float beta1, float beta2, float step_size,
                              float sqrt_bc2, float eps, uint32_t* nonfinite, void* stream);

/* ------------------------------------------------------------------------
 * 8-bit quantisation of a sent packet, the quantisation error kept in the
 * residual.  [SPARSE] "与其他压缩技术的比较" (comparison with other compression
 * techniques): top-k followed by 8-bit quantisation of the kept values.
 *
 * Applied after ef_topk_compress to its (vals, idx) and the residual e[n]:
 *   amax  = largest finite |vals[j]|           (0 if none)
 *   inv   = 127 / amax,  scale = amax / 127     (float32, correctly rounded)
 *   q[j]  = rint(vals[j] * inv) clamped to [-127, 127]   (round half to even;
 *           0 for a non-finite value, when amax = 0, or for a NaN product)
 *   e[idx[j]] = vals[j] - q[j] * scale         (float32; the receiver gets
 *           q[j] * scale, and q*scale + e' equals vals[j] exactly unless
 *           q*scale overflows: possible only when amax lies within 2^-24 of
 *           FLT_MAX, and then e' = -/+Inf at the entries coded +/-127)
 *   *scale_out = scale                          (device float)
 * Entries whose idx lies outside [0, n) update no residual.  ws: at least
 * ef_quantize_workspace_bytes(k) bytes, 4-byte aligned.
 * ------------------------------------------------------------------------ */
size_t ef_quantize_workspace_bytes(int64_t k);
int ef_quantize_int8(const float* vals, const int32_t* idx, int64_t k, float* e, int64_t n,
                     int8_t* q, float* scale_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Random magnitude-proportional sparsification with error feedback.
 * [SPARSE] "随机稀疏化" (random sparsification: each element survives with a
 * probability proportional to its magnitude, normalised so that about k
 * survive) inside the page's error-compensation loop ("误差补偿").
 *
 * Per element i, float32, each product and quotient rounded on its own:
 *   x  = g + e
 *   S  = sum of |x| over the finite x, exact, rounded to float64 and then to
 *        float32 (S32; *sum_out, device float, nullable)
 *   p  = min(1, (float(k) * |x|) / S32)      0 for a non-finite x; a NaN
 *        quotient (S32 = 0 or inf/inf) keeps nothing
 *   u  = word (i mod 4) of Philox4x32-10 on counter {i/4, 0, step low 32,
 *        step high 32} with key {seed low 32, seed high 32}, top 24 bits
 *        times 2^-24
 *   kept iff u < p
 * Kept elements are written in increasing index order: the first cap of them
 * as vals[j] = x, idx[j] = i, and their residual becomes +0.  Every other
 * element, a kept one beyond cap included, keeps e = x.
 *   *count_out = number kept (device int64, required; may exceed cap)
 *   *nonfinite = number of non-finite x (device uint32, nullable)
 * 0 <= n, k <= 2^31 - 1; cap >= 0 (vals/idx may be NULL when cap = 0);
 * g and e 16-byte aligned; ws: ef_random_sparsify_workspace_bytes(n) bytes,
 * 256-byte aligned (unused when n = 0).
 * flags: 0 or EF_FLAG_FORCE_FALLBACK (always take the exact integer sum
 * instead of the certified float64 one, and the second pass over x instead of
 * the candidates collected while summing; the result is the same).
 * ------------------------------------------------------------------------ */
size_t ef_random_sparsify_workspace_bytes(int64_t n);
int ef_random_sparsify(const float* g, float* e, int64_t n, int64_t k, uint64_t seed,
                       uint64_t step, float* vals, int32_t* idx, int64_t cap,
                       int64_t* count_out, float* sum_out, uint32_t* nonfinite, void* ws,
                       size_t ws_bytes, uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * Receiver-side aggregation of sparse packets.  [SPARSE] "梯度稀疏化的基本原理"
 * (values sharing an index are summed) and "详细算法流程" step 6.
 *
 * Packet p holds entries [pk_off[p], pk_off[p+1]) of vals/idx (device int64
 * table of npk+1 entries).  For p = 0 .. npk-1 in order, for each entry:
 *   G[idx] = G[idx] + val        (float32, one rounding per addition)
 * G keeps its incoming contents (zero it first for a plain sum).  Within one
 * packet indices must be strictly increasing and in [0, n) (the order top-k
 * emits).  An entry outside [0, n), or not above the entry before it in its
 * packet, is skipped and counted in *invalid (device uint32, nullable,
 * overwritten); with unordered packets other entries may be missed too, but no
 * write ever lands outside G.  pk_off must be non-decreasing with pk_off[0] >= 0
 * and pk_off[npk] at most the number of entries vals and idx hold (the library
 * cannot see their length and reads every entry the table names); it is read on
 * the device.
 * ------------------------------------------------------------------------ */
int sparse_decode_accumulate(float* G, int64_t n, int32_t npk, const float* vals,
                             const int32_t* idx, const int64_t* pk_off,
                             uint32_t* invalid, void* stream);

/* Parameter update, [SPARSE] "详细算法流程" step 7:
 *   w_i = w_i - (lr * G_i)     (product rounded to float32, then the subtraction) */
int sgd_apply(float* w, const float* G, int64_t n, float lr, void* stream);

/* The receiver's step in one pass, [SPARSE] "详细算法流程" steps 6-7: G starts
 * at +0 everywhere, the packets are added exactly as sparse_decode_accumulate
 * adds them, and w_i = w_i - (lr * G_i) as sgd_apply computes it.  Bit for bit
 * the same w (and G) as zeroing G, sparse_decode_accumulate, then sgd_apply,
 * reading w and writing G once; w is written back only where its bits change
 * (where the packets land), which gives the same memory contents.
 * G (nullable) receives the sum; w and G are n floats, 16-byte aligned, and
 * must not overlap.  Packets, pk_off and *invalid as for
 * sparse_decode_accumulate. */
int sparse_decode_sgd(float* w, float* G, int64_t n, int32_t npk, const float* vals,
                      const int32_t* idx, const int64_t* pk_off, float lr,
                      uint32_t* invalid, void* stream);

/* ------------------------------------------------------------------------
 * Index encodings, [SPARSE] "索引编码压缩" (index encoding).  Inputs are index
 * lists as top-k emits them: strictly increasing, in [0, n).
 * ------------------------------------------------------------------------ */

/* Bitmap: bits[i/8] bit (i%8) set iff i is listed; ceil(n/8) bytes, pad bits 0.
 * Indices outside [0, n) are ignored. */
int encode_bitmap(const int32_t* idx, int64_t k, int64_t n, uint8_t* bits, void* stream);

/* Every set bit of bits[ceil(n/8)] in ascending order.  Writes at most k_cap
 * indices; *k_out (device int64) = number of set bits. */
size_t decode_bitmap_workspace_bytes(int64_t n);
int decode_bitmap(const uint8_t* bits, int64_t n, int32_t* idx, int64_t k_cap,
                  int64_t* k_out, void* ws, size_t ws_bytes, void* stream);

/* Delta + varint: d_0 = idx_0, d_j = idx_j - idx_{j-1}; each d is written as a
 * minimal unsigned LEB128 number (7 bits per byte, low group first, high bit
 * set on all bytes but the last).  out needs encode_delta_bound(k) = 5k bytes;
 * *nbytes_out (device int64) = stream length. */
int64_t encode_delta_bound(int64_t k);
size_t delta_workspace_bytes(int64_t k_or_nbytes);
int encode_delta(const int32_t* idx, int64_t k, uint8_t* out, int64_t* nbytes_out,
                 void* ws, size_t ws_bytes, void* stream);
/* Parses exactly k varints from in[0, nbytes) and sums them back into idx[k].
 * *status (device uint32, nullable) = 0 if the stream held k well-formed
 * varints, else 1 (idx is then undefined where the stream was bad). */
int decode_delta(const uint8_t* in, int64_t nbytes, int64_t k, int32_t* idx,
                 uint32_t* status, void* ws, size_t ws_bytes, void* stream);

/* Block-sparse, 256-element blocks: nb = ceil(n/256).
 *   mask[ceil(nb/8)]: bit b (LSB first) set iff block b holds a listed index
 *   counts_m1[]     : for each non-empty block in ascending order, count - 1
 *                     (capacity min(k, nb))
 *   offs[k]         : idx_j - 256*(idx_j/256), in list order
 *   *nblk_out (device int64): number of non-empty blocks. */
size_t blocks_workspace_bytes(int64_t k, int64_t n);
int encode_blocks(const int32_t* idx, int64_t k, int64_t n, uint8_t* mask,
                  uint8_t* counts_m1, uint8_t* offs, int64_t* nblk_out, void* ws,
                  size_t ws_bytes, void* stream);
/* Inverse: rebuilds the k ascending indices described by mask/counts_m1/offs.
 * k is the number of indices the stream holds (the packet length). */
int decode_blocks(const uint8_t* mask, const uint8_t* counts_m1, const uint8_t* offs,
                  int64_t n, int64_t k, int32_t* idx, void* ws, size_t ws_bytes,
                  void* stream);

/* ------------------------------------------------------------------------
 * Kernel timing with HIP events on the stream each kernel is launched on.
 * ef_profile_enable(1, only) starts recording an event pair for every later
 * kernel launch of the process whose label contains `only` (host string; NULL
 * or "" = every launch), recorded by the dispatch itself (hipExtLaunchKernel),
 * so each pair spans the kernel's own run; launches on a stream under graph
 * capture are not recorded.  ef_profile_enable(0, NULL) stops and clears.
 * ef_profile_read() waits for the recorded events and returns the summed
 * duration (ms) and launch count of recorded kernels whose label contains
 * `name`.  Meant for benchmarks: a recorded launch takes longer to issue.
 * Labels are "topk_stream", "topk_sample_hist", ..., "sign_ef", "decode_scatter",
 * "sgd_apply", "bitmap_*", "delta_*", "blocks_*".
 * ------------------------------------------------------------------------ */
int ef_profile_enable(int on, const char* only);
int ef_profile_read(const char* name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* EFGRAD_H */
