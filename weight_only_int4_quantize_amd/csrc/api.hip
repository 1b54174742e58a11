// C ABI of the library (declared in include/awq.h): argument checks on the
// host, then kernels enqueued on the caller's stream.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "awq_internal.h"

using namespace awq;

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;      // any single extent
constexpr int64_t kMaxElems = int64_t(1) << 40;    // any product of extents

bool valid_group(int g) { return g == 32 || g == 64 || g == 128 || g == 256 || g == 512; }

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

// Halves of the reference's tiled copy of W: whole 64-k steps take it, other
// K none (the reference then reads W in place).
size_t reference_tiled_halves(int64_t N, int64_t K) { return gemm_ref_tiled_ok(K) ? tiled_fp16_halves(N, K) : 0; }

// Lays out the scale-search workspace; with base == nullptr it only sizes it.
struct SearchLayout {
    double* m = nullptr;
    double* abs_partials = nullptr;
    float* s = nullptr;
    uint32_t* qweight = nullptr;
    half_t* scales = nullptr;
    half_t* zeros = nullptr;
    half_t* xs = nullptr;
    half_t* wt = nullptr;   // W in the reference's tiled order (whole 64-k steps only)
    float* yref = nullptr;
    double* tile_partials = nullptr;
    double* losses = nullptr;
    size_t bytes = 0;

    SearchLayout(void* base, int64_t N, int64_t K, int64_t T, int G, int n_alpha) {
        Carve c(base);
        m = c.take<double>(K);
        abs_partials = c.take<double>(absmean_workspace_bytes(T, K) / sizeof(double));
        s = c.take<float>(K);
        qweight = c.take<uint32_t>(tiled_qweight_words(N, K));   // tiled order or row-major
        scales = c.take<half_t>(static_cast<size_t>(N) * (K / G));
        zeros = c.take<half_t>(static_cast<size_t>(N) * (K / G));
        xs = c.take<half_t>(static_cast<size_t>(T) * K);
        wt = c.take<half_t>(reference_tiled_halves(N, K));
        yref = c.take<float>(static_cast<size_t>(ref_tiled_floats(T, N)));
        tile_partials = c.take<double>(gemm_tile_count(T, N) + kLossSumBlocks);
        losses = c.take<double>(n_alpha);
        bytes = c.used;
    }
};

// Lays out the salient-loss workspace; with base == nullptr it only sizes it.
struct SalientLayout {
    double* m = nullptr;
    double* abs_partials = nullptr;
    int* idx = nullptr;
    uint32_t* qweight = nullptr;
    half_t* scales = nullptr;
    half_t* zeros = nullptr;
    half_t* w_sal = nullptr;
    half_t* wt = nullptr;   // W in the reference's tiled order (whole 64-k steps only)
    float* yref = nullptr;
    double* tile_partials = nullptr;
    double* losses = nullptr;
    size_t bytes = 0;

    SalientLayout(void* base, int64_t N, int64_t K, int64_t T, int G, int n_sal) {
        Carve c(base);
        m = c.take<double>(K);
        abs_partials = c.take<double>(absmean_workspace_bytes(T, K) / sizeof(double));
        idx = c.take<int>(std::max(n_sal, 1));
        qweight = c.take<uint32_t>(static_cast<size_t>(N) * (K / 8));
        scales = c.take<half_t>(static_cast<size_t>(N) * (K / G));
        zeros = c.take<half_t>(static_cast<size_t>(N) * (K / G));
        w_sal = c.take<half_t>(static_cast<size_t>(std::max(n_sal, 1)) * N);
        wt = c.take<half_t>(reference_tiled_halves(N, K));
        yref = c.take<float>(static_cast<size_t>(ref_tiled_floats(T, N)));
        tile_partials = c.take<double>(gemm_tile_count(T, N) + kLossSumBlocks);
        losses = c.take<double>(2);
        bytes = c.used;
    }
};

// Channels the K^2 selection accepts (a few milliseconds at the largest).
constexpr int64_t kMaxSelectK = int64_t(1) << 17;

// Lays out the clip-search workspace; with base == nullptr it only sizes it.
struct ClipLayout {
    uint32_t* qweight = nullptr;
    half_t* scales = nullptr;
    half_t* zeros = nullptr;
    half_t* xs = nullptr;           // x / s, only with channel scales
    half_t* wt = nullptr;           // W in the reference's tiled order (whole 64-k steps only)
    float* yref = nullptr;
    double* tile_partials = nullptr;
    double* losses = nullptr;
    size_t bytes = 0;

    ClipLayout(void* base, int64_t N, int64_t K, int64_t T, int G, int n, bool scaled) {
        Carve c(base);
        qweight = c.take<uint32_t>(tiled_qweight_words(N, K));   // tiled order or row-major
        scales = c.take<half_t>(static_cast<size_t>(N) * (K / G));
        zeros = c.take<half_t>(static_cast<size_t>(N) * (K / G));
        if (scaled) xs = c.take<half_t>(static_cast<size_t>(T) * K);
        wt = c.take<half_t>(reference_tiled_halves(N, K));
        yref = c.take<float>(static_cast<size_t>(ref_tiled_floats(T, N)));
        tile_partials = c.take<double>(gemm_tile_count(T, N) + kLossSumBlocks);
        losses = c.take<double>(n);
        bytes = c.used;
    }
};

// Y = x . W^T in fp32 (fp16 MFMA, fp32 accumulation), the unquantized
// reference of the searches, written in the tiled layout of ref_offset. With
// K whole 64-k steps W is first copied into wt in the GEMM's tiled B order
// (each wave's B of a step one contiguous piece); the products are the same.
awq_status reference_output(const half_t* x, const half_t* w, int64_t T, int64_t N, int64_t K, int G, float* y,
                            half_t* wt, hipStream_t s) {
    GemmArgs ref;
    ref.a = x;
    ref.w = w;
    ref.group_size = G;
    ref.M = T;
    ref.N = N;
    ref.K = K;
    ref.y32 = y;
    if (reference_tiled_halves(N, K) != 0 && T != 0 && N != 0) {
        const awq_status st = launch_tile_fp16_b(w, N, K, wt, s);
        if (st != AWQ_OK) return st;
        ref.w = wt;
        ref.b_tiled = true;
    }
    return launch_gemm(ref, GemmB::kF16, GemmOut::kF32, s);
}

// loss_out = || x' . dequant(Wq)^T - yref ||_F^2 (fused epilogue + fixed-order sum)
// tiled: qw holds the words in the tiled order (GemmArgs::b_tiled)
awq_status output_loss(const half_t* xa, const uint32_t* qw, const half_t* sc, const half_t* zr, int64_t T,
                       int64_t N, int64_t K, int G, const float* yref, double* partials, double* loss_out,
                       hipStream_t s, bool tiled = false) {
    GemmArgs q;
    q.a = xa;
    q.qweight = qw;
    q.scales = sc;
    q.zeros = zr;
    q.group_size = G;
    q.M = T;
    q.N = N;
    q.K = K;
    q.yref = yref;
    q.partials = partials;
    q.b_tiled = tiled;
    awq_status st = launch_gemm(q, GemmB::kInt4, GemmOut::kLoss, s);
    if (st != AWQ_OK) return st;
    return launch_sum_partials(partials, gemm_tile_count(T, N), loss_out, s);
}

// ---- the library-held scratch of awq_gemm_noalloc ----
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops) get the skinny kernel's K-split partial tiles and
// tile counters from this array instead of a workspace. 49 MiB holds the
// split plan of every M <= 64 on a 256-CU device (4 KiB of counters + 768
// partial tiles of up to 64 KiB). Each device the library runs on holds its
// own copy until the process ends.
constexpr size_t kNoAllocScratchBytes = size_t(49) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;         // the device address of `scratch` on this device
    awq_status status = AWQ_OK;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's copy of `scratch` (its device address, taken once per
// device with that device current). The first call on a device also clears
// the tile counters (a fill kernel on `stream`, ahead of the call's own
// work); every split kernel leaves them at zero when it ends.
awq_status device_scratch(void** out, hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AWQ_ERR_HIP;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            slot.status = AWQ_ERR_HIP;
            return;
        }
        const int64_t words = static_cast<int64_t>(split_counter_bytes() / sizeof(uint32_t));
        hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>(ceil_div(words, 256))), dim3(256), 0, stream,
                           static_cast<uint32_t*>(p), words);
        slot.status = last_launch_status();
        if (slot.status == AWQ_OK) slot.ptr = p;
    });
    if (slot.status != AWQ_OK) return slot.status;
    *out = slot.ptr;
    return AWQ_OK;
}

// The kernel a linear-layer call runs (1 GEMV, 2 GEMM, 3 skinny, 4 column
// tiles), or -1 when the requested path cannot take the shape. Automatic
// (path 0): the column tiles where they measured fastest; otherwise the GEMV
// up to 4 rows; the skinny kernel up to 64 rows (and below 5 rows where the
// GEMV's staged x does not fit the LDS), but below 9 rows only where it runs
// without K phases if the GEMV can run (the phased form, one block per
// column tile, is 2-3x slower than the GEMV there and 2-3x faster than the
// GEMM tile everywhere); else the GEMM.
int choose_path(int64_t M, int64_t N, int64_t K, int group_size, int path, bool have_workspace) {
    const bool gemv_ok = gemv_supported(M, K);
    bool skinny_phased = false;
    const bool skinny_ok = skinny_supported(M, N, K, group_size, have_workspace, &skinny_phased);
    switch (path) {
        case 1: return gemv_ok ? 1 : -1;
        case 2: return 2;
        case 3: return skinny_ok ? 3 : -1;
        case 4: return coltile_supported(M, N, K, group_size) ? 4 : -1;
        default: break;
    }
    // few-row layers with long rows: the GEMV's one-shot form beats the
    // column tiles up to 4 rows of x (512 x 11008 at M = 4: 7.9 against
    // 8.7 us; 1024 x 8192: 5.7 against 7.2 us)
    if (M >= 3 && gemv_ok && gemv_few_rows(M, N, K)) return 1;
    if (coltile_preferred(M, N, K, group_size, have_workspace)) return 4;
    if (skinny_ok && (M > 4 || !gemv_ok) && !(skinny_phased && gemv_ok)) return 3;
    return gemv_ok ? 1 : 2;
}

// The linear layer behind awq_gemm_ex and awq_gemm_noalloc: checks, then
// the kernel choice. workspace (may be NULL) feeds the skinny kernel's K
// splits and, when split_gemm is set, the GEMM's stream-K partials. With
// library_scratch the skinny kernel's splits take the device's `scratch`
// instead (set up only once every check has passed); the GEMM then runs
// unsplit.
awq_status gemm_dispatch(const void* x_f16, const uint32_t* qweight, const void* scales_f16, const void* zeros_f16,
                         int64_t M, int64_t N, int64_t K, int group_size, void* y_f16, int path, void* workspace,
                         size_t workspace_bytes, bool split_gemm, bool library_scratch, hipStream_t stream) {
    awq_status st = check_dims(N, K, group_size);
    if (st != AWQ_OK) return st;
    if (path < 0 || path > 4) return AWQ_ERR_CONFIG;
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
    const int chosen = choose_path(M, N, K, group_size, path, workspace != nullptr || library_scratch);
    if (chosen < 0) return AWQ_ERR_CONFIG;
    const bool use_skinny = chosen == 3;
    if (chosen == 4) return launch_coltile(x, qweight, sc, zr, M, N, K, group_size, y, stream);
    if (chosen == 1) return launch_gemv(x, qweight, sc, zr, M, N, K, group_size, y, stream);
    if (!use_skinny && !split_gemm) workspace = nullptr;
    if (use_skinny && library_scratch) {
        if (skinny_workspace_bytes(M, N, K) > kNoAllocScratchBytes) return AWQ_ERR_WORKSPACE;
        if ((st = device_scratch(&workspace, stream)) != AWQ_OK) return st;
        workspace_bytes = kNoAllocScratchBytes;
    }
    if (workspace != nullptr) {
        if (reinterpret_cast<uintptr_t>(workspace) & 255) return AWQ_ERR_ALIGN;
        const size_t need = use_skinny ? skinny_workspace_bytes(M, N, K) : gemm_workspace_bytes(M, N);
        if (workspace_bytes < need) return AWQ_ERR_WORKSPACE;
    }
    if (use_skinny) return launch_skinny(x, qweight, sc, zr, M, N, K, group_size, y, workspace, stream);
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
    return launch_gemm(a, GemmB::kInt4, GemmOut::kF16, stream, workspace);
}

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
                           int group_size, int mode, double clip_fraction, uint32_t* qweight, void* scales_f16,
                           void* zeros_f16, void* stream) {
    if (mode != AWQ_QUANT_ASYMMETRIC && mode != AWQ_QUANT_SYMMETRIC) return AWQ_ERR_CONFIG;
    if (!clip_fraction_ok(clip_fraction)) return AWQ_ERR_CONFIG;
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
                           mode == AWQ_QUANT_SYMMETRIC, clip_fraction, qweight, static_cast<half_t*>(scales_f16),
                           static_cast<half_t*>(zeros_f16), as_stream(stream));
}

awq_status awq_quantize(const void* w_f16, const float* channel_scale, int64_t N, int64_t K,
                        int group_size, uint32_t* qweight, void* scales_f16, void* zeros_f16,
                        void* stream) {
    return awq_quantize_ex(w_f16, channel_scale, N, K, group_size, AWQ_QUANT_ASYMMETRIC, 0.0, qweight,
                           scales_f16, zeros_f16, stream);
}

size_t awq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
    return std::max(gemm_workspace_bytes(M, N), skinny_workspace_bytes(M, N, K));
}

awq_status awq_gemm_ex(const void* x_f16, const uint32_t* qweight, const void* scales_f16,
                       const void* zeros_f16, int64_t M, int64_t N, int64_t K, int group_size,
                       void* y_f16, int path, void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_dispatch(x_f16, qweight, scales_f16, zeros_f16, M, N, K, group_size, y_f16, path, workspace,
                         workspace_bytes, true, false, as_stream(stream));
}

awq_status awq_gemm_path(const void* x_f16, const uint32_t* qweight, const void* scales_f16,
                         const void* zeros_f16, int64_t M, int64_t N, int64_t K, int group_size,
                         void* y_f16, int path, void* stream) {
    return awq_gemm_ex(x_f16, qweight, scales_f16, zeros_f16, M, N, K, group_size, y_f16, path, nullptr, 0,
                       stream);
}

int awq_gemm_kernel(int64_t M, int64_t N, int64_t K, int group_size, int path, int have_workspace) {
    if (check_dims(N, K, group_size) != AWQ_OK || path < 0 || path > 4) return -1;
    if (M < 1 || N < 1 || M > (int64_t(1) << 31) - 256 || N > (int64_t(1) << 31) - 256) return -1;
    return choose_path(M, N, K, group_size, path, have_workspace != 0);
}

awq_status awq_gemm_grouped(const void* x_f16, int n_layers, const uint32_t* const* qweight,
                            const void* const* scales_f16, const void* const* zeros_f16, const int64_t* N,
                            int64_t M, int64_t K, int group_size, void* const* y_f16, void* stream) {
    if (n_layers < 1 || n_layers > kGemvMaxLayers) return AWQ_ERR_CONFIG;
    if (!qweight || !scales_f16 || !zeros_f16 || !N || !y_f16) return AWQ_ERR_NULL;
    if (M < 0 || M > kMaxDim) return AWQ_ERR_SHAPE;
    int64_t total = 0;
    for (int i = 0; i < n_layers; ++i) {
        const awq_status st = check_dims(N[i], K, group_size);
        if (st != AWQ_OK) return st;
        total += N[i];
        if (M > 0 && N[i] > 0) {
            if (!x_f16 || !qweight[i] || !scales_f16[i] || !zeros_f16[i] || !y_f16[i]) return AWQ_ERR_NULL;
            if (!aligned16(x_f16) || !aligned16(qweight[i]) || (reinterpret_cast<uintptr_t>(scales_f16[i]) & 1) ||
                (reinterpret_cast<uintptr_t>(zeros_f16[i]) & 1) || (reinterpret_cast<uintptr_t>(y_f16[i]) & 1))
                return AWQ_ERR_ALIGN;
        }
    }
    if (total > (int64_t(1) << 31) - 256) return AWQ_ERR_SHAPE;
    if (M == 0 || total == 0) return AWQ_OK;
    const hipStream_t s = as_stream(stream);
    const int chosen = choose_path(M, total, K, group_size, 0, false);
    GemvLayers L{};
    int r = 0;
    for (int i = 0; i < n_layers; ++i) {
        if (N[i] == 0) continue;
        L.qweight[L.n] = qweight[i];
        L.scales[L.n] = static_cast<const half_t*>(scales_f16[i]);
        L.zeros[L.n] = static_cast<const half_t*>(zeros_f16[i]);
        L.y[L.n] = static_cast<half_t*>(y_f16[i]);
        L.row0[L.n] = r;
        r += static_cast<int>(N[i]);
        ++L.n;
    }
    L.row0[L.n] = r;
    for (int i = L.n + 1; i <= kGemvMaxLayers; ++i) L.row0[i] = INT32_MAX;
    const half_t* x = static_cast<const half_t*>(x_f16);
    if (chosen == 1 && M <= kGemvGroupedMaxM) return launch_gemv_grouped(x, L, M, K, group_size, s);
    // column tiles over the stacked layers where awq_gemm takes them, and at
    // 3-4 rows of x on few-row layers (which awq_gemm gives the GEMV one at a
    // time); the layers' own block counts must fit the launch
    if ((chosen == 4 || (chosen == 1 && M > kGemvGroupedMaxM)) && coltile_grouped_supported(M, L, K, group_size))
        return launch_coltile_grouped(x, L, M, K, group_size, s);
    for (int i = 0; i < n_layers; ++i) {
        const awq_status st = gemm_dispatch(x_f16, qweight[i], scales_f16[i], zeros_f16[i], M, N[i], K, group_size,
                                            y_f16[i], 0, nullptr, 0, false, false, s);
        if (st != AWQ_OK) return st;
    }
    return AWQ_OK;
}

awq_status awq_gemm_noalloc(const void* x_f16, const uint32_t* qweight, const void* scales_f16,
                            const void* zeros_f16, int64_t M, int64_t N, int64_t K, int group_size, void* y_f16,
                            int path, void* stream) {
    return gemm_dispatch(x_f16, qweight, scales_f16, zeros_f16, M, N, K, group_size, y_f16, path, nullptr, 0,
                         false, true, as_stream(stream));
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
    if (!w_f16 || !x_f16 || !workspace || !losses || !best_index || !best_scales) return AWQ_ERR_NULL;
    // no grid given: alpha_i = i / n_alpha (n_alpha = 20: 0, 0.05, ..., 0.95)
    std::vector<double> grid(n_alpha);
    for (int i = 0; i < n_alpha; ++i) {
        grid[i] = alphas ? alphas[i] : static_cast<double>(i) / static_cast<double>(n_alpha);
        if (!std::isfinite(grid[i])) return AWQ_ERR_CONFIG;
    }
    if (!aligned16(w_f16) || !aligned16(x_f16) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(best_scales) & 3))
        return AWQ_ERR_ALIGN;
    SearchLayout L(workspace, N, K, T, group_size, n_alpha);
    if (workspace_bytes < L.bytes) return AWQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    const half_t* w = static_cast<const half_t*>(w_f16);
    const half_t* x = static_cast<const half_t*>(x_f16);

    // the loss GEMM reads the quantized words in the tiled order where its
    // direct form runs (one contiguous 1 KB piece per wave and K step)
    const bool tiled = gemm_tiled_ok(K, group_size);
    // m = mean |x| per input channel
    if ((st = launch_absmean(x, T, K, L.m, L.abs_partials, s)) != AWQ_OK) return st;
    // reference output W . x^T, once, in fp32
    if ((st = reference_output(x, w, T, N, K, group_size, L.yref, L.wt, s)) != AWQ_OK) return st;
    for (int i = 0; i < n_alpha; ++i) {
        if ((st = launch_pow_scales(L.m, K, grid[i], L.s, s)) != AWQ_OK) return st;
        if ((st = launch_quantize(w, L.s, N, K, group_size, false, 0.0, L.qweight, L.scales, L.zeros, s, 4,
                                  tiled)) != AWQ_OK)
            return st;
        // s = 1 exactly at alpha = 0, where x / s is x itself, bit for bit
        const bool identity = grid[i] == 0.0;
        if (!identity && (st = launch_divide_columns(x, L.s, T, K, L.xs, s)) != AWQ_OK) return st;
        if ((st = output_loss(identity ? x : L.xs, L.qweight, L.scales, L.zeros, T, N, K, group_size, L.yref,
                              L.tile_partials, L.losses + i, s, tiled)) != AWQ_OK)
            return st;
    }
    if (hipMemcpyAsync(losses, L.losses, sizeof(double) * n_alpha, hipMemcpyDeviceToHost, s) != hipSuccess)
        return AWQ_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return AWQ_ERR_HIP;
    int best = 0;
    for (int i = 1; i < n_alpha; ++i)
        if (losses[i] < losses[best]) best = i;   // strict: ties keep the smaller alpha
    *best_index = best;
    if ((st = launch_pow_scales(L.m, K, grid[best], best_scales, s)) != AWQ_OK) return st;
    return AWQ_OK;
}

size_t awq_clip_search_workspace_bytes(int64_t N, int64_t K, int64_t T, int group_size, int n_fractions,
                                        int scaled) {
    if (check_dims(N, K, group_size) != AWQ_OK || N <= 0 || T <= 0 || n_fractions < 1) return 0;
    return ClipLayout(nullptr, N, K, T, group_size, n_fractions, scaled != 0).bytes;
}

awq_status awq_clip_search(const void* w_f16, const void* x_f16, const float* channel_scale, int64_t N, int64_t K,
                           int64_t T, int group_size, int mode, const double* fractions, int n_fractions,
                           void* workspace, size_t workspace_bytes, double* losses, int* best_index,
                           void* stream) {
    awq_status st = check_dims(N, K, group_size);
    if (st != AWQ_OK) return st;
    if (N <= 0 || T <= 0 || T > (int64_t(1) << 24)) return AWQ_ERR_SHAPE;
    if (T > (int64_t(1) << 31) - 256 || N > (int64_t(1) << 31) - 256) return AWQ_ERR_SHAPE;
    if (mode != AWQ_QUANT_ASYMMETRIC && mode != AWQ_QUANT_SYMMETRIC) return AWQ_ERR_CONFIG;
    if (n_fractions < 1 || n_fractions > 64) return AWQ_ERR_CONFIG;
    if (!w_f16 || !x_f16 || !fractions || !workspace || !losses || !best_index) return AWQ_ERR_NULL;
    for (int i = 0; i < n_fractions; ++i)
        if (!clip_fraction_ok(fractions[i])) return AWQ_ERR_CONFIG;
    if (!aligned16(w_f16) || !aligned16(x_f16) || !aligned16(workspace) ||
        (channel_scale && !aligned16(channel_scale)))
        return AWQ_ERR_ALIGN;
    ClipLayout L(workspace, N, K, T, group_size, n_fractions, channel_scale != nullptr);
    if (workspace_bytes < L.bytes) return AWQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    const half_t* w = static_cast<const half_t*>(w_f16);
    const half_t* x = static_cast<const half_t*>(x_f16);

    if ((st = reference_output(x, w, T, N, K, group_size, L.yref, L.wt, s)) != AWQ_OK) return st;
    const half_t* xa = x;
    if (channel_scale != nullptr) {
        if ((st = launch_divide_columns(x, channel_scale, T, K, L.xs, s)) != AWQ_OK) return st;
        xa = L.xs;
    }
    const bool tiled = gemm_tiled_ok(K, group_size);   // as in the scale search
    for (int i = 0; i < n_fractions; ++i) {
        if ((st = launch_quantize(w, channel_scale, N, K, group_size, mode == AWQ_QUANT_SYMMETRIC, fractions[i],
                                  L.qweight, L.scales, L.zeros, s, 4, tiled)) != AWQ_OK)
            return st;
        if ((st = output_loss(xa, L.qweight, L.scales, L.zeros, T, N, K, group_size, L.yref, L.tile_partials,
                              L.losses + i, s, tiled)) != AWQ_OK)
            return st;
    }
    if (hipMemcpyAsync(losses, L.losses, sizeof(double) * n_fractions, hipMemcpyDeviceToHost, s) != hipSuccess)
        return AWQ_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return AWQ_ERR_HIP;
    int best = 0;
    for (int i = 1; i < n_fractions; ++i)
        if (losses[i] < losses[best]) best = i;   // strict: ties keep the earlier fraction
    *best_index = best;
    return AWQ_OK;
}

awq_status awq_select_salient(const double* m_f64, int64_t K, int n_salient, int* idx, void* stream) {
    if (K <= 0 || K > kMaxSelectK || n_salient < 0 || n_salient > K) return AWQ_ERR_SHAPE;
    if (n_salient == 0) return AWQ_OK;
    if (!m_f64 || !idx) return AWQ_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(m_f64) & 7) || (reinterpret_cast<uintptr_t>(idx) & 3)) return AWQ_ERR_ALIGN;
    return launch_select_salient(m_f64, K, n_salient, idx, as_stream(stream));
}

awq_status awq_quantize_salient(const void* w_f16, int64_t N, int64_t K, int group_size, int mode, const int* idx,
                                int n_salient, uint32_t* qweight, void* scales_f16, void* zeros_f16,
                                void* w_salient_f16, void* stream) {
    awq_status st = check_dims(N, K, group_size);
    if (st != AWQ_OK) return st;
    if (N * K > kMaxElems || n_salient < 0 || n_salient > K) return AWQ_ERR_SHAPE;
    if (mode != AWQ_QUANT_ASYMMETRIC && mode != AWQ_QUANT_SYMMETRIC) return AWQ_ERR_CONFIG;
    if (N == 0) return AWQ_OK;
    if (!w_f16 || !qweight || !scales_f16 || !zeros_f16 || (n_salient > 0 && (!idx || !w_salient_f16)))
        return AWQ_ERR_NULL;
    if (!aligned16(w_f16) || !aligned16(qweight) || (reinterpret_cast<uintptr_t>(scales_f16) & 1) ||
        (reinterpret_cast<uintptr_t>(zeros_f16) & 1) || (reinterpret_cast<uintptr_t>(idx) & 3) ||
        (reinterpret_cast<uintptr_t>(w_salient_f16) & 1))
        return AWQ_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    const half_t* w = static_cast<const half_t*>(w_f16);
    if ((st = launch_quantize(w, nullptr, N, K, group_size, mode == AWQ_QUANT_SYMMETRIC, 0.0, qweight,
                              static_cast<half_t*>(scales_f16), static_cast<half_t*>(zeros_f16), s)) != AWQ_OK)
        return st;
    return launch_salient_fix(w, N, K, group_size, idx, n_salient, qweight, static_cast<const half_t*>(zeros_f16),
                              static_cast<half_t*>(w_salient_f16), s);
}

awq_status awq_salient_apply(const void* x_f16, const int* idx, const void* w_salient_f16, int64_t M, int64_t N,
                             int64_t K, int n_salient, void* y_f16, void* stream) {
    if (M < 0 || N < 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || n_salient < 0 || n_salient > K)
        return AWQ_ERR_SHAPE;
    if (M == 0 || N == 0 || n_salient == 0) return AWQ_OK;
    if (!x_f16 || !idx || !w_salient_f16 || !y_f16) return AWQ_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(x_f16) & 1) || (reinterpret_cast<uintptr_t>(idx) & 3) ||
        (reinterpret_cast<uintptr_t>(w_salient_f16) & 1) || (reinterpret_cast<uintptr_t>(y_f16) & 1))
        return AWQ_ERR_ALIGN;
    return launch_salient_apply(static_cast<const half_t*>(x_f16), idx, static_cast<const half_t*>(w_salient_f16), M,
                                N, K, n_salient, static_cast<half_t*>(y_f16), as_stream(stream));
}

int64_t awq_salient_count(int64_t K) {
    if (K <= 0) return 0;
    // round(K / 100), ties to even (the default rounding mode)
    return static_cast<int64_t>(std::nearbyint(0.01 * static_cast<double>(K)));
}

size_t awq_salient_loss_workspace_bytes(int64_t N, int64_t K, int64_t T, int group_size, int n_salient) {
    if (n_salient < 0) n_salient = static_cast<int>(awq_salient_count(K));
    if (check_dims(N, K, group_size) != AWQ_OK || N <= 0 || T <= 0 || n_salient > K) return 0;
    return SalientLayout(nullptr, N, K, T, group_size, n_salient).bytes;
}

awq_status awq_salient_loss(const void* w_f16, const void* x_f16, int64_t N, int64_t K, int64_t T, int group_size,
                            int mode, int n_salient, void* workspace, size_t workspace_bytes, double* loss_rtn,
                            double* loss_salient, int* idx_out, void* stream) {
    awq_status st = check_dims(N, K, group_size);
    if (st != AWQ_OK) return st;
    if (N <= 0 || T <= 0 || T > (int64_t(1) << 24) || K % 8 != 0) return AWQ_ERR_SHAPE;
    if (T > (int64_t(1) << 31) - 256 || N > (int64_t(1) << 31) - 256) return AWQ_ERR_SHAPE;
    if (n_salient < 0 && K <= kMaxSelectK) n_salient = static_cast<int>(awq_salient_count(K));
    if (K > kMaxSelectK || n_salient < 0 || n_salient > K) return AWQ_ERR_SHAPE;
    if (mode != AWQ_QUANT_ASYMMETRIC && mode != AWQ_QUANT_SYMMETRIC) return AWQ_ERR_CONFIG;
    if (!w_f16 || !x_f16 || !workspace || !loss_rtn || !loss_salient) return AWQ_ERR_NULL;
    if (!aligned16(w_f16) || !aligned16(x_f16) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(idx_out) & 3))
        return AWQ_ERR_ALIGN;
    SalientLayout L(workspace, N, K, T, group_size, n_salient);
    if (workspace_bytes < L.bytes) return AWQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    const half_t* w = static_cast<const half_t*>(w_f16);
    const half_t* x = static_cast<const half_t*>(x_f16);
    const bool sym = mode == AWQ_QUANT_SYMMETRIC;

    // salient channels from m = mean |x|
    if ((st = launch_absmean(x, T, K, L.m, L.abs_partials, s)) != AWQ_OK) return st;
    if ((st = launch_select_salient(L.m, K, n_salient, L.idx, s)) != AWQ_OK) return st;
    // reference W . x^T; the plain quantizer's loss
    if ((st = reference_output(x, w, T, N, K, group_size, L.yref, L.wt, s)) != AWQ_OK) return st;
    if ((st = launch_quantize(w, nullptr, N, K, group_size, sym, 0.0, L.qweight, L.scales, L.zeros, s)) != AWQ_OK)
        return st;
    if ((st = output_loss(x, L.qweight, L.scales, L.zeros, T, N, K, group_size, L.yref, L.tile_partials, L.losses,
                          s)) != AWQ_OK)
        return st;
    // mixed layer: INT4 part with the salient codes at the zero-point, fp16
    // side part moved to the reference: || x Q0^T - (W x^T - x_S W_S^T) ||^2
    if ((st = launch_salient_fix(w, N, K, group_size, L.idx, n_salient, L.qweight, L.zeros, L.w_sal, s)) != AWQ_OK)
        return st;
    if ((st = launch_salient_subtract(x, L.idx, L.w_sal, T, N, K, n_salient, L.yref, s)) != AWQ_OK) return st;
    if ((st = output_loss(x, L.qweight, L.scales, L.zeros, T, N, K, group_size, L.yref, L.tile_partials,
                          L.losses + 1, s)) != AWQ_OK)
        return st;
    if (idx_out && n_salient > 0 &&
        hipMemcpyAsync(idx_out, L.idx, sizeof(int) * n_salient, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return AWQ_ERR_HIP;
    double host[2];
    if (hipMemcpyAsync(host, L.losses, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess) return AWQ_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return AWQ_ERR_HIP;
    *loss_rtn = host[0];
    *loss_salient = host[1];
    return AWQ_OK;
}

awq_status awq_quantize_w8(const void* w_f16, const float* channel_scale, int64_t N, int64_t K, int group_size,
                           int mode, uint32_t* qweight, void* scales_f16, void* zeros_f16, void* stream) {
    awq_status st = check_dims(N, K, group_size);
    if (st != AWQ_OK) return st;
    if (group_size < 64) return AWQ_ERR_CONFIG;
    if (N * K > kMaxElems) return AWQ_ERR_SHAPE;
    if (mode != AWQ_QUANT_ASYMMETRIC && mode != AWQ_QUANT_SYMMETRIC) return AWQ_ERR_CONFIG;
    if (N == 0) return AWQ_OK;
    if (!w_f16 || !qweight || !scales_f16 || !zeros_f16) return AWQ_ERR_NULL;
    if (!aligned16(w_f16) || !aligned16(qweight) || (channel_scale && !aligned16(channel_scale)) ||
        (reinterpret_cast<uintptr_t>(scales_f16) & 1) || (reinterpret_cast<uintptr_t>(zeros_f16) & 1))
        return AWQ_ERR_ALIGN;
    return launch_quantize(static_cast<const half_t*>(w_f16), channel_scale, N, K, group_size,
                           mode == AWQ_QUANT_SYMMETRIC, 0.0, qweight, static_cast<half_t*>(scales_f16),
                           static_cast<half_t*>(zeros_f16), as_stream(stream), 8);
}

awq_status awq_gemm_w8(const void* x_f16, const uint32_t* qweight, const void* scales_f16, const void* zeros_f16,
                       int64_t M, int64_t N, int64_t K, int group_size, void* y_f16, int path, void* workspace,
                       size_t workspace_bytes, void* stream) {
    awq_status st = check_dims(N, K, group_size);
    if (st != AWQ_OK) return st;
    if (group_size < 64) return AWQ_ERR_CONFIG;
    if (path < 0 || path > 2) return AWQ_ERR_CONFIG;
    if (M < 0 || M > kMaxDim) return AWQ_ERR_SHAPE;
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
    const bool gemv_ok = gemv_supported(M, K, 8);
    if (path == 1 && !gemv_ok) return AWQ_ERR_CONFIG;
    // the MFMA form needs 32-bit byte offsets within a 256-row tile of x
    if (path == 2 && K * 256 * 2 >= (int64_t(1) << 31)) return AWQ_ERR_CONFIG;
    if (path == 1 || (path == 0 && gemv_ok))
        return launch_gemv(x, qweight, sc, zr, M, N, K, group_size, y, as_stream(stream), 8);
    if (K * 256 * 2 >= (int64_t(1) << 31)) return AWQ_ERR_SHAPE;
    if (workspace != nullptr) {
        if (reinterpret_cast<uintptr_t>(workspace) & 255) return AWQ_ERR_ALIGN;
        if (workspace_bytes < gemm_workspace_bytes(M, N)) return AWQ_ERR_WORKSPACE;
    }
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
    return launch_gemm(a, GemmB::kInt8, GemmOut::kF16, as_stream(stream), workspace);
}

}  // extern "C"
