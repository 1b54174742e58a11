// C ABI of the library (declared in include/awq.h): argument checks on the
// host, then kernels enqueued on the caller's stream.
#include <algorithm>
#include <cmath>
#include <vector>

#include "awq_internal.h"

using namespace awq;

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;      // any single extent
constexpr int64_t kMaxElems = int64_t(1) << 40;    // any product of extents

bool valid_group(int g) { return g == 32 || g == 64 || g == 128 || g == 256; }

awq_status check_dims(int64_t N, int64_t K, int group_size) {
    if (!valid_group(group_size)) return AWQ_ERR_CONFIG;
    if (N < 0 || K <= 0 || N > kMaxDim || K > kMaxDim) return AWQ_ERR_SHAPE;
    if (K % group_size != 0) return AWQ_ERR_SHAPE;
    return AWQ_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

struct Carve {
    char* base;
    size_t used = 0;
    explicit Carve(void* p) : base(static_cast<char*>(p)) {}
    template <class T>
    T* take(size_t count) {
        T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
        used = round_up(used + count * sizeof(T), 256);
        return p;
    }
};

// Lays out the scale-search workspace; with base == nullptr it only sizes it.
struct SearchLayout {
    double* m = nullptr;
    double* abs_partials = nullptr;
    float* s = nullptr;
    uint32_t* qweight = nullptr;
    half_t* scales = nullptr;
    half_t* zeros = nullptr;
    half_t* xs = nullptr;
    float* yref = nullptr;
    double* tile_partials = nullptr;
    double* losses = nullptr;
    size_t bytes = 0;

    SearchLayout(void* base, int64_t N, int64_t K, int64_t T, int G, int n_alpha) {
        Carve c(base);
        m = c.take<double>(K);
        abs_partials = c.take<double>(absmean_workspace_bytes(T, K) / sizeof(double));
        s = c.take<float>(K);
        qweight = c.take<uint32_t>(static_cast<size_t>(N) * (K / 8));
        scales = c.take<half_t>(static_cast<size_t>(N) * (K / G));
        zeros = c.take<half_t>(static_cast<size_t>(N) * (K / G));
        xs = c.take<half_t>(static_cast<size_t>(T) * K);
        yref = c.take<float>(static_cast<size_t>(T) * N);
        tile_partials = c.take<double>(gemm_tile_count(T, N));
        losses = c.take<double>(n_alpha);
        bytes = c.used;
    }
};

}  // namespace

extern "C" {

const char* awq_status_string(int status) {
    switch (status) {
        case AWQ_OK: return "AWQ_OK";
        case AWQ_ERR_NULL: return "AWQ_ERR_NULL: a required pointer is NULL";
        case AWQ_ERR_SHAPE: return "AWQ_ERR_SHAPE: invalid matrix sizes";
        case AWQ_ERR_ALIGN: return "AWQ_ERR_ALIGN: a device pointer is not 16-byte aligned";
        case AWQ_ERR_CONFIG: return "AWQ_ERR_CONFIG: unsupported configuration";
        case AWQ_ERR_WORKSPACE: return "AWQ_ERR_WORKSPACE: workspace too small";
        case AWQ_ERR_HIP: return "AWQ_ERR_HIP: HIP runtime error";
        default: return "unknown awq_status";
    }
}

int awq_version(void) { return 100; }

awq_status awq_quantize_ex(const void* w_f16, const float* channel_scale, int64_t N, int64_t K,
                           int group_size, int mode, uint32_t* qweight, void* scales_f16, void* zeros_f16,
                           void* stream) {
    if (mode != AWQ_QUANT_ASYMMETRIC && mode != AWQ_QUANT_SYMMETRIC) return AWQ_ERR_CONFIG;
    awq_status st = check_dims(N, K, group_size);
    if (st != AWQ_OK) return st;
    if (N * K > kMaxElems) return AWQ_ERR_SHAPE;
    if (N == 0) return AWQ_OK;
    if (!w_f16 || !qweight || !scales_f16 || !zeros_f16) return AWQ_ERR_NULL;
    if (!aligned16(w_f16) || !aligned16(qweight) || (channel_scale && !aligned16(channel_scale)))
        return AWQ_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(scales_f16) & 1) || (reinterpret_cast<uintptr_t>(zeros_f16) & 1))
        return AWQ_ERR_ALIGN;
    return launch_quantize(static_cast<const half_t*>(w_f16), channel_scale, N, K, group_size,
                           mode == AWQ_QUANT_SYMMETRIC, qweight, static_cast<half_t*>(scales_f16),
                           static_cast<half_t*>(zeros_f16), as_stream(stream));
}

awq_status awq_quantize(const void* w_f16, const float* channel_scale, int64_t N, int64_t K,
                        int group_size, uint32_t* qweight, void* scales_f16, void* zeros_f16,
                        void* stream) {
    return awq_quantize_ex(w_f16, channel_scale, N, K, group_size, AWQ_QUANT_ASYMMETRIC, qweight, scales_f16,
                           zeros_f16, stream);
}

size_t awq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
    return std::max(gemm_workspace_bytes(M, N), skinny_workspace_bytes(M, N, K));
}

awq_status awq_gemm_ex(const void* x_f16, const uint32_t* qweight, const void* scales_f16,
                       const void* zeros_f16, int64_t M, int64_t N, int64_t K, int group_size,
                       void* y_f16, int path, void* workspace, size_t workspace_bytes, void* stream) {
    awq_status st = check_dims(N, K, group_size);
    if (st != AWQ_OK) return st;
    if (path < 0 || path > 3) return AWQ_ERR_CONFIG;
    if (M < 0 || M > kMaxDim) return AWQ_ERR_SHAPE;
    // The MFMA kernel indexes with 32-bit row/column numbers and 64-bit offsets.
    if (M > (int64_t(1) << 31) - 256 || N > (int64_t(1) << 31) - 256) return AWQ_ERR_SHAPE;
    if (M == 0 || N == 0) return AWQ_OK;
    if (!x_f16 || !qweight || !scales_f16 || !zeros_f16 || !y_f16) return AWQ_ERR_NULL;
    if (!aligned16(x_f16) || !aligned16(qweight) || (reinterpret_cast<uintptr_t>(scales_f16) & 1) ||
        (reinterpret_cast<uintptr_t>(zeros_f16) & 1) || (reinterpret_cast<uintptr_t>(y_f16) & 1))
        return AWQ_ERR_ALIGN;
    const half_t* x = static_cast<const half_t*>(x_f16);
    const half_t* sc = static_cast<const half_t*>(scales_f16);
    const half_t* zr = static_cast<const half_t*>(zeros_f16);
    half_t* y = static_cast<half_t*>(y_f16);
    const bool gemv_ok = gemv_supported(M, K);
    const bool skinny_ok = skinny_supported(M, N, K, group_size, workspace != nullptr);
    if (path == 1 && !gemv_ok) return AWQ_ERR_CONFIG;
    if (path == 3 && !skinny_ok) return AWQ_ERR_CONFIG;
    // automatic: the GEMV up to 4 rows, the skinny kernel up to 64 where it
    // applies, else the GEMV up to 8 rows, else the GEMM
    const bool use_skinny = path == 3 || (path == 0 && M > 4 && skinny_ok);
    const bool use_gemv = path == 1 || (path == 0 && gemv_ok && !use_skinny);
    if (use_gemv) return launch_gemv(x, qweight, sc, zr, M, N, K, group_size, y, as_stream(stream));
    if (workspace != nullptr) {
        if (reinterpret_cast<uintptr_t>(workspace) & 255) return AWQ_ERR_ALIGN;
        const size_t need = use_skinny ? skinny_workspace_bytes(M, N, K) : gemm_workspace_bytes(M, N);
        if (workspace_bytes < need) return AWQ_ERR_WORKSPACE;
    }
    if (use_skinny)
        return launch_skinny(x, qweight, sc, zr, M, N, K, group_size, y, workspace, as_stream(stream));
    GemmArgs a;
    a.a = x;
    a.qweight = qweight;
    a.scales = sc;
    a.zeros = zr;
    a.group_size = group_size;
    a.M = M;
    a.N = N;
    a.K = K;
    a.y16 = y;
    return launch_gemm(a, GemmB::kInt4, GemmOut::kF16, as_stream(stream), workspace);
}

awq_status awq_gemm_path(const void* x_f16, const uint32_t* qweight, const void* scales_f16,
                         const void* zeros_f16, int64_t M, int64_t N, int64_t K, int group_size,
                         void* y_f16, int path, void* stream) {
    return awq_gemm_ex(x_f16, qweight, scales_f16, zeros_f16, M, N, K, group_size, y_f16, path, nullptr, 0,
                       stream);
}

awq_status awq_gemm(const void* x_f16, const uint32_t* qweight, const void* scales_f16,
                    const void* zeros_f16, int64_t M, int64_t N, int64_t K, int group_size,
                    void* y_f16, void* stream) {
    return awq_gemm_path(x_f16, qweight, scales_f16, zeros_f16, M, N, K, group_size, y_f16, 0, stream);
}

size_t awq_activation_absmean_workspace_bytes(int64_t T, int64_t K) {
    if (T <= 0 || K <= 0) return 0;
    return absmean_workspace_bytes(T, K);
}

awq_status awq_activation_absmean(const void* x_f16, int64_t T, int64_t K, double* m_f64,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (T <= 0 || K <= 0 || K % 8 != 0 || K > kMaxDim || T > (int64_t(1) << 24)) return AWQ_ERR_SHAPE;
    if (!x_f16 || !m_f64 || !workspace) return AWQ_ERR_NULL;
    if (!aligned16(x_f16) || (reinterpret_cast<uintptr_t>(m_f64) & 7) ||
        (reinterpret_cast<uintptr_t>(workspace) & 7))
        return AWQ_ERR_ALIGN;
    if (workspace_bytes < absmean_workspace_bytes(T, K)) return AWQ_ERR_WORKSPACE;
    return launch_absmean(static_cast<const half_t*>(x_f16), T, K, m_f64, static_cast<double*>(workspace),
                          as_stream(stream));
}

size_t awq_scale_search_workspace_bytes(int64_t N, int64_t K, int64_t T, int group_size, int n_alpha) {
    if (check_dims(N, K, group_size) != AWQ_OK || N <= 0 || T <= 0 || n_alpha < 1) return 0;
    return SearchLayout(nullptr, N, K, T, group_size, n_alpha).bytes;
}

awq_status awq_scale_search(const void* w_f16, const void* x_f16, int64_t N, int64_t K, int64_t T,
                            int group_size, const double* alphas, int n_alpha, void* workspace,
                            size_t workspace_bytes, double* losses, int* best_index, float* best_scales,
                            void* stream) {
    awq_status st = check_dims(N, K, group_size);
    if (st != AWQ_OK) return st;
    if (N <= 0 || T <= 0 || T > (int64_t(1) << 24)) return AWQ_ERR_SHAPE;
    if (T > (int64_t(1) << 31) - 256 || N > (int64_t(1) << 31) - 256) return AWQ_ERR_SHAPE;
    if (n_alpha < 1 || n_alpha > 64) return AWQ_ERR_CONFIG;
    if (!w_f16 || !x_f16 || !alphas || !workspace || !losses || !best_index || !best_scales)
        return AWQ_ERR_NULL;
    for (int i = 0; i < n_alpha; ++i)
        if (!std::isfinite(alphas[i])) return AWQ_ERR_CONFIG;
    if (!aligned16(w_f16) || !aligned16(x_f16) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(best_scales) & 3))
        return AWQ_ERR_ALIGN;
    SearchLayout L(workspace, N, K, T, group_size, n_alpha);
    if (workspace_bytes < L.bytes) return AWQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    const half_t* w = static_cast<const half_t*>(w_f16);
    const half_t* x = static_cast<const half_t*>(x_f16);

    // m = mean |x| per input channel
    if ((st = launch_absmean(x, T, K, L.m, L.abs_partials, s)) != AWQ_OK) return st;
    // reference output W . x^T, once, in fp32
    GemmArgs ref;
    ref.a = x;
    ref.w = w;
    ref.group_size = group_size;
    ref.M = T;
    ref.N = N;
    ref.K = K;
    ref.y32 = L.yref;
    if ((st = launch_gemm(ref, GemmB::kF16, GemmOut::kF32, s)) != AWQ_OK) return st;

    const int64_t tiles = gemm_tile_count(T, N);
    for (int i = 0; i < n_alpha; ++i) {
        if ((st = launch_pow_scales(L.m, K, alphas[i], L.s, s)) != AWQ_OK) return st;
        if ((st = launch_quantize(w, L.s, N, K, group_size, false, L.qweight, L.scales, L.zeros, s)) != AWQ_OK)
            return st;
        if ((st = launch_divide_columns(x, L.s, T, K, L.xs, s)) != AWQ_OK) return st;
        GemmArgs q;
        q.a = L.xs;
        q.qweight = L.qweight;
        q.scales = L.scales;
        q.zeros = L.zeros;
        q.group_size = group_size;
        q.M = T;
        q.N = N;
        q.K = K;
        q.yref = L.yref;
        q.partials = L.tile_partials;
        if ((st = launch_gemm(q, GemmB::kInt4, GemmOut::kLoss, s)) != AWQ_OK) return st;
        if ((st = launch_sum_partials(L.tile_partials, tiles, L.losses + i, s)) != AWQ_OK) return st;
    }
    if (hipMemcpyAsync(losses, L.losses, sizeof(double) * n_alpha, hipMemcpyDeviceToHost, s) != hipSuccess)
        return AWQ_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return AWQ_ERR_HIP;
    int best = 0;
    for (int i = 1; i < n_alpha; ++i)
        if (losses[i] < losses[best]) best = i;   // strict: ties keep the smaller alpha
    *best_index = best;
    if ((st = launch_pow_scales(L.m, K, alphas[best], best_scales, s)) != AWQ_OK) return st;
    return AWQ_OK;
}

}  // extern "C"
