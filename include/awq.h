/*
 * awq.h - C ABI of the MI355X (gfx950) W4A16 library: group-wise asymmetric
 * INT4 weight quantization, the fused dequantize-and-multiply linear layer
 * and AWQ's activation-aware per-input-channel scale search.
 *
 * Sources for the operations (cited by page title and section):
 *   "模型量化:GGUF/AWQ/GPTQ部署方案" (xxmr.cn), §1.2 量化映射: the affine map
 *       q = clamp(round(x / scale) + zero_point, 0, 2^bits - 1) and its
 *       inverse x_hat = (q - zero_point) * scale, the scale set by the range
 *       of the weights; §1.4 量化粒度: one scale per group of 128 weights.
 *   "模型量化实战：INT8/INT4、GPTQ、AWQ与精度-速度权衡" (aissn.com), sections
 *       量化粒度 (per-group, group_size=128) and 对称/非对称量化 (asymmetric,
 *       zero-point != 0).
 *   rskf.cn AWQ article: §2.1 (per-input-channel factor s: weights times s,
 *       activations divided by s, s searched to minimise the difference
 *       between the quantized and the original output), §2.3 / §4.1 (the
 *       factor is folded ahead of inference), §1.3 / §3.3 (INT4 -> FP16
 *       dequantization inside the matmul; a GEMV kernel for single-stream
 *       decode, a GEMM kernel for batches).
 *   "AWQ 模型量化技术：激活感知的权重量化革命", Per-channel Scaling 优化.
 *
 * Conventions shared by every call:
 *   - Matrices are row-major and densely packed. W[N, K]: row n is output
 *     channel n, column k is input channel k. Groups of G consecutive k share
 *     one scale and one zero-point (G = 32, 64, 128, 256 or 512).
 *   - qweight is uint32 [N, K/8]: the 4-bit code of column k = 8c + j sits in
 *     bits 4j..4j+3 of word c. scales and zeros are fp16 [N, K/G]; every zero
 *     is an integer 0..15.
 *   - Pointers marked "device" point to GPU memory of the current HIP device;
 *     they must be 16-byte aligned. The caller allocates and owns every
 *     buffer; the library allocates no device memory (the scale search takes
 *     a caller-provided workspace) and keeps no state between calls, except
 *     the static scratch array of awq_gemm_noalloc.
 *   - stream is a hipStream_t (NULL means the null stream). awq_quantize,
 *     awq_gemm and awq_activation_absmean only enqueue work on it and return.
 *   - Argument checks run on the host before anything is enqueued; a failed
 *     check launches nothing. No C++ exception crosses this interface.
 *   - Non-finite inputs give undefined (but memory-safe) results.
 */
#ifndef AWQ_MI355X_H
#define AWQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    AWQ_OK = 0,
    AWQ_ERR_NULL = 1,      /* a required pointer is NULL */
    AWQ_ERR_SHAPE = 2,     /* negative size, K not a multiple of G, ... */
    AWQ_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned */
    AWQ_ERR_CONFIG = 4,    /* unsupported group_size, path, mode, grid, ... */
    AWQ_ERR_WORKSPACE = 5, /* workspace smaller than the size query says */
    AWQ_ERR_HIP = 6        /* the HIP runtime reported an error */
} awq_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* awq_status_string(int status);

/* Interface version (major * 100 + minor). */
int awq_version(void);

/*
 * awq_quantize - group-wise asymmetric INT4 quantization of W.
 * (xxmr.cn §1.2 / §1.4; aissn.com 量化粒度, 对称/非对称量化)
 *
 * For every row n and group g, over w' = float32(w[n,k] * channel_scale[k])
 * (or w' = w when channel_scale is NULL), in IEEE float32:
 *   range = max(max(w') - min(w'), 1e-5)
 *   scale = fp16_rne(range / 15)            (stored in scales[n, g])
 *   zero  = clamp(rint(-min(w') / scale), 0, 15)   (stored in zeros[n, g])
 *   code  = clamp(rint(w' / scale) + zero, 0, 15)
 * where rint is round-half-to-even and the division is correctly rounded.
 *
 *   w_f16          device, fp16 [N, K]
 *   channel_scale  device, fp32 [K] or NULL (AWQ's W * diag(s), rskf.cn §2.1)
 *   N, K           N >= 0; K > 0, K % group_size == 0
 *   group_size     32, 64, 128, 256 or 512
 *   qweight        device, uint32 [N, K/8]            (output)
 *   scales_f16     device, fp16 [N, K/G]              (output)
 *   zeros_f16      device, fp16 [N, K/G]              (output)
 * N == 0 returns AWQ_OK without work. Results are bit-identical on every run.
 * Scales that overflow fp16 (range / 15 > 65504) are undefined.
 */
awq_status awq_quantize(const void* w_f16, const float* channel_scale,
                        int64_t N, int64_t K, int group_size,
                        uint32_t* qweight, void* scales_f16, void* zeros_f16,
                        void* stream);

/*
 * awq_quantize_ex - awq_quantize with a choice of map
 * (aissn.com 对称/非对称量化: asymmetric allows a zero-point != 0;
 * symmetric has zero-point 0, simple and hardware friendly).
 *
 *   mode AWQ_QUANT_ASYMMETRIC (0): as awq_quantize.
 *   mode AWQ_QUANT_SYMMETRIC (1): per row n and group g, in IEEE float32,
 *     a     = max(max |w'|, 1e-5)
 *     scale = fp16_rne(a / 7)                  (stored in scales[n, g])
 *     code  = clamp(rint(w' / scale) + 8, 0, 15),  zeros[n, g] = 8
 *   i.e. the signed code q = code - 8 = rint(w' / scale) lies in -7..7 and
 *   q(-w) = -q(w). The stored layout is the asymmetric one, so awq_gemm and
 *   the other linear-layer calls apply unchanged.
 *
 *   clip_fraction p in [0, 0.25): the clip step of xxmr.cn §1.5 (cut the
 *   extreme p of each group's values at both ends before the scale is
 *   taken; the page uses 1 %). The group's min and max above are replaced
 *   by the p and 1 - p quantiles, interpolated between its order statistics
 *   x(0) <= ... <= x(G-1): with h = (G - 1) p in double, i = floor(h),
 *   f = float(h - i), in float32 without fused multiply-adds,
 *     lo = x(i) + f (x(i+1) - x(i)),  hi = x(G-1-i) - f (x(G-1-i) - x(G-2-i))
 *   (asymmetric: range = hi - lo, zero from lo; symmetric: a = max(-lo,
 *   hi)). Values beyond the bounds take the clamped codes. p = 0 is the
 *   plain map, bit for bit.
 * Any other mode or clip_fraction returns AWQ_ERR_CONFIG. Arguments
 * otherwise as awq_quantize.
 */
enum { AWQ_QUANT_ASYMMETRIC = 0, AWQ_QUANT_SYMMETRIC = 1 };
awq_status awq_quantize_ex(const void* w_f16, const float* channel_scale,
                           int64_t N, int64_t K, int group_size, int mode,
                           double clip_fraction, uint32_t* qweight,
                           void* scales_f16, void* zeros_f16, void* stream);

/*
 * awq_gemm - the W4A16 linear layer y = x . dequant(Wq)^T.
 * (xxmr.cn §1.2 inverse map; rskf.cn §1.3 / §3.3 GEMV and GEMM kernels)
 *
 *   y[m, n] = sum_k x[m, k] * (code[n, k] - zeros[n, k/G]) * scales[n, k/G]
 * accumulated in fp32 and stored as fp16 (round-to-nearest-even).
 *
 *   x_f16        device, fp16 [M, K] (activations already divided by any
 *                AWQ factor s, which is folded upstream: rskf.cn §2.3)
 *   qweight, scales_f16, zeros_f16   device, as written by awq_quantize
 *   M, N, K      M, N >= 0; K > 0, K % group_size == 0
 *   group_size   32, 64, 128, 256 or 512
 *   y_f16        device, fp16 [M, N] (output; must not alias the inputs)
 * M == 0 or N == 0 returns AWQ_OK without work. Decode (M <= 2) runs a
 * bandwidth-bound GEMV; a batch of decode tokens (M <= 64) one of two MFMA
 * kernels that stream the packed weights straight into registers: column
 * tiles (one block per 16, 32, 48 or 64 output columns over all of K; M <= 32,
 * chosen from M = 3 up on layers of up to 48 Mi weights, or 96 Mi with
 * K <= 8192, and on every shape when no workspace is given) or the skinny
 * kernel (256 columns per block, K split across blocks with a workspace);
 * larger M the MFMA GEMM. Results do not depend on run-to-run scheduling.
 */
awq_status awq_gemm(const void* x_f16, const uint32_t* qweight,
                    const void* scales_f16, const void* zeros_f16,
                    int64_t M, int64_t N, int64_t K, int group_size,
                    void* y_f16, void* stream);

/*
 * awq_gemm_path - awq_gemm with the kernel chosen by the caller:
 * path 0 = automatic (as awq_gemm), 1 = GEMV (requires M <= 8),
 * 2 = MFMA GEMM, 3 = skinny MFMA kernel (requires M <= 64, G <= 256 and a
 * packed matrix under 4 GiB; without a workspace each block walks all of K,
 * staging it in LDS-sized phases), 4 = column-tile MFMA kernel (requires
 * M <= 32, G <= 256, M * K * 2 < 2^31 and the tile's (scale, zero) pairs in
 * LDS; no workspace).
 * Any other path, or a path whose requirement fails, returns AWQ_ERR_CONFIG.
 * The automatic choice takes the GEMV for M <= 2, and for M <= 4 on
 * layers of few rows of 4096 < K <= 16384 (all rows within one round of
 * its resident waves); the column tiles for 3 <= M <= 32 on layers of up
 * to 48 Mi weights, or up to 96 Mi with K <= 8192, and on any shape they
 * support when the call has no workspace; otherwise the GEMV for M <= 4
 * where it can run; the skinny kernel for M <= 64, except for M <= 8 where
 * it would have to stage K in phases and the GEMV can run (then the GEMV);
 * then the GEMM.
 */
awq_status awq_gemm_path(const void* x_f16, const uint32_t* qweight,
                         const void* scales_f16, const void* zeros_f16,
                         int64_t M, int64_t N, int64_t K, int group_size,
                         void* y_f16, int path, void* stream);

/*
 * awq_gemm_kernel - the kernel a linear-layer call of this shape runs:
 * 1 = GEMV, 2 = MFMA GEMM, 3 = skinny MFMA kernel, 4 = column tiles; -1
 * when the requested path cannot take it or an argument is invalid.
 * path as awq_gemm_path (0 = automatic); have_workspace != 0 for a call
 * with a workspace (awq_gemm_ex) or for awq_gemm_noalloc. No GPU work.
 */
int awq_gemm_kernel(int64_t M, int64_t N, int64_t K, int group_size, int path,
                    int have_workspace);

/*
 * awq_gemm_ex - awq_gemm_path with a caller-owned device workspace, which
 * lets the MFMA kernels split the K loop of output tiles across thread
 * blocks when the tile count would leave the GPU's resident blocks partly
 * idle: a stream-K decomposition for the GEMM (e.g. the M = 2048 prefill of
 * a 4096-wide layer, or only the tiles of a short last round behind whole
 * tiles), and fixed K splits for the skinny kernel (e.g. M = 16 on an
 * 8192 x 28672 layer). Same operation, arguments and
 * results as awq_gemm (rskf.cn §3.3 GEMM kernel), up to fp32 summation
 * order; the partial sums of a split tile are added in a fixed order, so
 * results do not depend on scheduling.
 *
 *   workspace        device memory of at least
 *                    awq_gemm_workspace_bytes(M, N, K) bytes, 256-byte
 *                    aligned, owned by the caller. It must be zero-filled
 *                    before its first use; every call leaves it ready for
 *                    the next one (the tile counters in it are back at zero
 *                    when the call's kernel ends), so later calls of any
 *                    size that fits reuse it without clearing it again.
 *                    Calls that may run concurrently must not share one
 *                    workspace. NULL = no split (as awq_gemm_path).
 *   workspace_bytes  its size; too small returns AWQ_ERR_WORKSPACE,
 *                    misaligned AWQ_ERR_ALIGN (both before any work).
 * The GEMV path (small M) never touches the workspace.
 */
size_t awq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
awq_status awq_gemm_ex(const void* x_f16, const uint32_t* qweight,
                       const void* scales_f16, const void* zeros_f16,
                       int64_t M, int64_t N, int64_t K, int group_size,
                       void* y_f16, int path, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * awq_gemm_noalloc - awq_gemm_ex for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. The same operation and arguments as awq_gemm_path;
 * the split scratch comes from a library-held device array instead of a
 * caller's workspace, and the call allocates nothing.
 *
 *   - The skinny kernel (4 < M <= 64, and M <= 4 where the GEMV's staged x
 *     does not fit) splits K as awq_gemm_ex does with a workspace, so the
 *     results are those of awq_gemm_ex bit for bit. Its partial tiles and
 *     tile counters live in a static device array of 49 MiB, one per device
 *     the library runs on, held until the process ends. A split plan that
 *     would need more (none on a 256-CU MI355X) returns AWQ_ERR_WORKSPACE
 *     before any work.
 *   - The MFMA GEMM (larger M) runs without stream-K splits, whose fp32
 *     partials would need up to 134 MB; the GEMV uses no scratch.
 *   - The first call on a device that runs the skinny kernel (after every
 *     argument check has passed) takes the array's device address and
 *     enqueues one small kernel on `stream`, ahead of its own, that clears
 *     the tile counters; every split kernel leaves them at zero when it
 *     ends.
 *   - All calls on one device share the array: calls that may run at the
 *     same time on one device (different streams, graphs replayed
 *     concurrently) race and give wrong results. Serialise them.
 * Returns AWQ_ERR_HIP if the array cannot be set up on the current device.
 */
awq_status awq_gemm_noalloc(const void* x_f16, const uint32_t* qweight,
                            const void* scales_f16, const void* zeros_f16,
                            int64_t M, int64_t N, int64_t K, int group_size,
                            void* y_f16, int path, void* stream);

/*
 * awq_gemm_grouped - several linear layers that read the same activations,
 * y_i = x . dequant(Wq_i)^T for i < n_layers: the independent projections of
 * a decoder layer (q / k / v, gate / up), which the pages' deployment fuses
 * (rskf.cn §3.4 fuse_layers), kept as separate tensors (rskf.cn §1.3 / §3.3
 * GEMV kernel). Where awq_gemm (without a workspace) would run the GEMV or
 * the column tiles on the layers' stacked rows, one launch computes all of
 * them, the rows of layer i after those of layers 0 .. i - 1; otherwise each
 * layer is an awq_gemm call, in order.
 *   - GEMV (M <= 2): each y_i equals that layer's awq_gemm result bit for
 *     bit (a row's arithmetic does not depend on the launch shape).
 *   - Column tiles (3 <= M <= 32): each layer on whole blocks of its own
 *     columns; the tile and wave counts follow the stacked rows, so the
 *     fp32 order of a layer's sums (and its last bits) may differ from its
 *     own awq_gemm call. Results are the same run to run.
 *   - Otherwise (one awq_gemm per layer): the same bits as those calls.
 *
 *   x_f16        device, fp16 [M, K], shared by every layer
 *   n_layers     1 .. 4
 *   qweight, scales_f16, zeros_f16, y_f16
 *                host arrays of n_layers device pointers, layer i's tensors
 *                as in awq_gemm ([N[i], K / 8], [N[i], K / G], [N[i], K / G],
 *                output [M, N[i]]); outputs must not alias any input or
 *                each other
 *   N            host array of n_layers row counts, each >= 0, summing to
 *                less than 2^31 - 256
 *   M, K, group_size  as in awq_gemm, common to every layer
 * n_layers outside 1 .. 4 returns AWQ_ERR_CONFIG; a NULL array or device
 * pointer AWQ_ERR_NULL; every layer is checked before anything is enqueued.
 */
awq_status awq_gemm_grouped(const void* x_f16, int n_layers, const uint32_t* const* qweight,
                            const void* const* scales_f16, const void* const* zeros_f16,
                            const int64_t* N, int64_t M, int64_t K, int group_size,
                            void* const* y_f16, void* stream);

/*
 * awq_activation_absmean - m[k] = max(mean_t |x[t, k]|, 1e-8), the
 * per-input-channel activation statistic AWQ's scale is built from
 * (rskf.cn §2.1-2.2; "AWQ 模型量化技术", Per-channel Scaling 优化).
 *
 *   x_f16    device, fp16 [T, K], T > 0, K > 0, K % 8 == 0
 *   m_f64    device, fp64 [K] (output)
 *   workspace, workspace_bytes  device scratch of at least
 *            awq_activation_absmean_workspace_bytes(T, K) bytes
 * Accumulation is in fp64 in a fixed order (bit-identical run to run).
 */
size_t awq_activation_absmean_workspace_bytes(int64_t T, int64_t K);
awq_status awq_activation_absmean(const void* x_f16, int64_t T, int64_t K,
                                  double* m_f64, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * awq_scale_search - AWQ's per-input-channel scale search over an alpha grid
 * (rskf.cn §2.1; "AWQ 模型量化技术", Per-channel Scaling 优化).
 *
 * With m = awq_activation_absmean(x) and, for every alpha_i,
 *   s_i[k] = float32(m[k] ^ alpha_i)   (pow in fp64, then rounded)
 *   loss_i = || Q(W . diag(s_i)) . (x / s_i)^T  -  W . x^T ||_F^2
 * where Q is awq_quantize with channel_scale = s_i and the product is the
 * W4A16 GEMM on fp16(x / s_i) (fp32 accumulation); the reference W . x^T is
 * computed once (fp16 MFMA, fp32 accumulation) and kept in the workspace.
 * The best index is the first minimum of the losses (ties go to the
 * smallest alpha).
 *
 *   w_f16         device, fp16 [N, K]
 *   x_f16         device, fp16 [T, K] (calibration activations)
 *   N, K, T       N > 0, T > 0, K > 0, K % group_size == 0
 *   group_size    32, 64, 128, 256 or 512
 *   alphas        host, float64 [n_alpha], every alpha finite (1 <= n_alpha <= 64);
 *                 NULL takes the grid alpha_i = i / n_alpha (n_alpha = 20:
 *                 0, 0.05, ..., 0.95)
 *   workspace     device, >= awq_scale_search_workspace_bytes(N, K, T, G, n_alpha)
 *   losses        host, float64 [n_alpha] (output)
 *   best_index    host, int (output)
 *   best_scales   device, fp32 [K] (output: s at the best alpha)
 * Synchronises the stream once, at the end, to read the losses back.
 */
size_t awq_scale_search_workspace_bytes(int64_t N, int64_t K, int64_t T,
                                        int group_size, int n_alpha);
awq_status awq_scale_search(const void* w_f16, const void* x_f16,
                            int64_t N, int64_t K, int64_t T, int group_size,
                            const double* alphas, int n_alpha,
                            void* workspace, size_t workspace_bytes,
                            double* losses, int* best_index,
                            float* best_scales, void* stream);

/*
 * awq_clip_search - the clip fraction of xxmr.cn §1.5, chosen by the scale
 * search's own objective (rskf.cn §2.1: the difference between the
 * quantized and the original output) over a caller-given grid.
 *
 * For every fraction p_i, with s = channel_scale (1 when NULL):
 *   loss_i = || Q_p(W . diag(s)) . (x / s)^T  -  W . x^T ||_F^2
 * where Q_p is awq_quantize_ex(mode, clip_fraction = p_i) with that channel
 * scale, and the products are the library's W4A16 GEMM and fp16 MFMA
 * reference (fp32 accumulation, fp64 loss sum). The best index is the first
 * minimum (ties go to the earlier fraction).
 *
 *   w_f16, x_f16   device, fp16 [N, K] and [T, K]
 *   channel_scale  device, fp32 [K] (e.g. awq_scale_search's best_scales)
 *                  or NULL
 *   N, K, T        N > 0, T > 0, K > 0, K % group_size == 0
 *   group_size     32, 64, 128, 256 or 512
 *   mode           AWQ_QUANT_ASYMMETRIC or AWQ_QUANT_SYMMETRIC
 *   fractions      host, double [n_fractions], each in [0, 0.25);
 *                  1 <= n_fractions <= 64
 *   workspace, workspace_bytes  device scratch of at least
 *                  awq_clip_search_workspace_bytes(N, K, T, group_size,
 *                  n_fractions, channel_scale != NULL) bytes, 16-byte aligned
 *   losses         host, double [n_fractions] (output)
 *   best_index     host (output)
 * Synchronises `stream` once, to read the losses back.
 */
size_t awq_clip_search_workspace_bytes(int64_t N, int64_t K, int64_t T,
                                        int group_size, int n_fractions,
                                        int scaled);
awq_status awq_clip_search(const void* w_f16, const void* x_f16,
                           const float* channel_scale, int64_t N, int64_t K,
                           int64_t T, int group_size, int mode,
                           const double* fractions, int n_fractions,
                           void* workspace, size_t workspace_bytes,
                           double* losses, int* best_index, void* stream);

/*
 * Mixed precision with fp16 salient weights ("AWQ 模型量化技术：激活感知的
 * 权重量化革命", 技术实现 1 and 混合精度设计: the important 1 % of the
 * weights, picked from the activation distribution, stay in fp16 and the
 * rest is quantized to 4 bits; xxmr.cn §2.2). The layer is
 *   y = x . dequant(Wq)^T + x[:, idx] . w_salient
 * where Wq is the usual group-wise INT4 matrix of all of W whose codes in
 * the salient input channels are set to the group's zero-point (so they
 * dequantize to exactly 0), and w_salient[j, n] = W[n, idx[j]] in fp16.
 */

/*
 * awq_select_salient - idx[0 .. n_salient) = the n_salient input channels
 * with the largest m[k] (awq_activation_absmean's mean |x|), by descending
 * m; equal m go by ascending channel index.
 *
 *   m_f64      device, double [K], 8-byte aligned; finite values
 *   K          1 <= K <= 131072
 *   n_salient  0 <= n_salient <= K (0 does nothing)
 *   idx        device, int32 [n_salient] (output), 4-byte aligned
 * Asynchronous on `stream`.
 */
awq_status awq_select_salient(const double* m_f64, int64_t K, int n_salient,
                              int* idx, void* stream);

/*
 * awq_quantize_salient - the stored mixed-precision form: awq_quantize_ex
 * (mode, no clip) of all of W, then the codes of the channels idx[j] set to
 * their group's zero-point and w_salient[j, n] = W[n, idx[j]].
 *
 *   w_f16          device, fp16 [N, K], 16-byte aligned
 *   N, K, group_size, mode   as awq_quantize_ex
 *   idx            device, int32 [n_salient]: distinct channels in [0, K)
 *                  (an index outside it is skipped and its w_salient row is
 *                  0; a repeated index would be counted twice by
 *                  awq_salient_apply)
 *   n_salient      0 <= n_salient <= K
 *   qweight, scales_f16, zeros_f16   outputs, as awq_quantize
 *   w_salient_f16  device, fp16 [n_salient, N] (output)
 * Asynchronous on `stream`.
 */
awq_status awq_quantize_salient(const void* w_f16, int64_t N, int64_t K,
                                int group_size, int mode, const int* idx,
                                int n_salient, uint32_t* qweight,
                                void* scales_f16, void* zeros_f16,
                                void* w_salient_f16, void* stream);

/*
 * awq_salient_apply - the fp16 side product of the mixed layer, added in
 * place: y[m, n] = fp16(y[m, n] + sum_j x[m, idx[j]] * w_salient[j, n]),
 * the sum in fp32. Run it after awq_gemm on the same stream to get the
 * mixed layer's output.
 *
 *   x_f16          device, fp16 [M, K]
 *   idx            device, int32 [n_salient] (as awq_quantize_salient)
 *   w_salient_f16  device, fp16 [n_salient, N]
 *   y_f16          device, fp16 [M, N] (input and output)
 * M == 0, N == 0 or n_salient == 0 return AWQ_OK without work.
 * Asynchronous on `stream`.
 */
awq_status awq_salient_apply(const void* x_f16, const int* idx,
                             const void* w_salient_f16, int64_t M, int64_t N,
                             int64_t K, int n_salient, void* y_f16,
                             void* stream);

/*
 * awq_salient_loss - the ablation of the mixed form against the plain
 * quantizer, by the scale search's objective (rskf.cn §2.1):
 *   loss_rtn     = || Q(W) . x^T - W . x^T ||_F^2
 *   loss_salient = || W_mixed . x^T - W . x^T ||_F^2
 * with the salient channels chosen by awq_select_salient from x's mean |x|
 * and Q the quantizer of `mode` (no channel scale). The products are the
 * library's W4A16 GEMM, the fp16 MFMA reference and the side product
 * (fp32), the sums in fp64.
 *
 *   w_f16, x_f16   device, fp16 [N, K] and [T, K], 16-byte aligned
 *   N, K, T        N > 0, 0 < T <= 2^24, K % 8 == 0, K <= 131072,
 *                  K % group_size == 0
 *   group_size     32, 64, 128, 256 or 512
 *   mode           AWQ_QUANT_ASYMMETRIC or AWQ_QUANT_SYMMETRIC
 *   n_salient      0 <= n_salient <= K, or negative for the pages' 1 %:
 *                  awq_salient_count(K) channels
 *   workspace, workspace_bytes  device scratch of at least
 *                  awq_salient_loss_workspace_bytes(N, K, T, group_size,
 *                  n_salient) bytes (the same negative n_salient allowed),
 *                  16-byte aligned
 *   loss_rtn, loss_salient  host, double (outputs)
 *   idx_out        device, int32 [n_salient] (output: the chosen channels)
 *                  or NULL
 * Synchronises `stream` once, to read the losses back.
 */
/*
 * awq_salient_count - the number of salient input channels the pages keep,
 * about 1 % ("AWQ 模型量化技术", 技术实现 1): round(K / 100), ties to even
 * (41 of 4096). K <= 0 gives 0.
 */
int64_t awq_salient_count(int64_t K);

size_t awq_salient_loss_workspace_bytes(int64_t N, int64_t K, int64_t T,
                                         int group_size, int n_salient);
awq_status awq_salient_loss(const void* w_f16, const void* x_f16, int64_t N,
                            int64_t K, int64_t T, int group_size, int mode,
                            int n_salient, void* workspace,
                            size_t workspace_bytes, double* loss_rtn,
                            double* loss_salient, int* idx_out, void* stream);

/*
 * W8A16: 8-bit weights with fp16 activations (aissn.com "INT8 vs INT4" and
 * "INT8 实战": the steadier choice, weight INT8 with activations kept in
 * fp16). The map of xxmr.cn §1.2 with 2^8 levels, group-wise as the INT4
 * form: asymmetric scale = range / 255, zero-point in [0, 255]; symmetric
 * scale = max|w| / 127, code = q + 128, zero-point 128. Four codes per
 * uint32 along K, the code of column k = 4c + j in bits 8j..8j+7 of word c.
 */

/*
 * awq_quantize_w8 - group-wise 8-bit quantization of W[N, K].
 *
 *   w_f16          device, fp16 [N, K], 16-byte aligned
 *   channel_scale  device, fp32 [K] (quantize W . diag(s)) or NULL
 *   N, K           N >= 0, K > 0, K % group_size == 0
 *   group_size     64, 128, 256 or 512
 *   mode           AWQ_QUANT_ASYMMETRIC or AWQ_QUANT_SYMMETRIC
 *   qweight        device, uint32 [N, K/4] (output), 16-byte aligned
 *   scales_f16, zeros_f16   device, fp16 [N, K/group_size] (outputs)
 * Asynchronous on `stream`.
 */
awq_status awq_quantize_w8(const void* w_f16, const float* channel_scale,
                           int64_t N, int64_t K, int group_size, int mode,
                           uint32_t* qweight, void* scales_f16,
                           void* zeros_f16, void* stream);

/*
 * awq_gemm_w8 - the W8A16 linear layer y = x . dequant(Wq)^T (fp32
 * accumulation, fp16 output), Wq from awq_quantize_w8.
 *
 *   x_f16        device, fp16 [M, K], 16-byte aligned
 *   qweight      device, uint32 [N, K/4], 16-byte aligned
 *   scales_f16, zeros_f16   device, fp16 [N, K/group_size]
 *   group_size   64, 128, 256 or 512
 *   y_f16        device, fp16 [M, N] (output)
 *   path         0 = automatic (the GEMV for M <= 8, else the MFMA GEMM),
 *                1 = GEMV (M <= 8), 2 = MFMA GEMM (K * 512 < 2^31)
 *   workspace    as awq_gemm_ex (stream-K splits of the GEMM) or NULL
 * M == 0 or N == 0 returns AWQ_OK without work. Asynchronous on `stream`.
 */
awq_status awq_gemm_w8(const void* x_f16, const uint32_t* qweight,
                       const void* scales_f16, const void* zeros_f16,
                       int64_t M, int64_t N, int64_t K, int group_size,
                       void* y_f16, int path, void* workspace,
                       size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_H */
