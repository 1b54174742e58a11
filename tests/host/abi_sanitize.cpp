// Host-side sanitizer run of the C ABI's argument checks: built against a
// copy of the library whose host code carries AddressSanitizer and
// UndefinedBehaviorSanitizer (device code unchanged), this calls every entry
// point with arguments that its checks must refuse before any GPU work
// (null, misaligned and out-of-range pointers and sizes, short workspaces,
// bad configurations, extreme sizes that would overflow a naive size
// product), and the size queries with extreme sizes. The sanitizers abort
// on any out-of-bounds access, overflow or undefined operation in that host
// code; a wrong status code is reported here. Prints "ok" and exits 0, or
// names the first failure and exits 1. No GPU is needed or touched.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/awq.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
    if (got != want) {
        std::printf("%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

}  // namespace

int main() {
    void* const F = fake(0x10000);       // aligned, never dereferenced
    void* const ODD = fake(0x10008);     // 8- but not 16-byte aligned
    void* const WS = fake(0x100000);     // 256-byte aligned
    const int64_t big = int64_t(1) << 40;
    const int64_t huge = INT64_MAX;

    // status strings: every code and out-of-range codes
    for (int c = -3; c < 10; ++c)
        if (awq_status_string(c) == nullptr || std::strlen(awq_status_string(c)) == 0) {
            std::printf("status string %d empty\n", c);
            ++failures;
        }

    // quantize
    expect("quantize null w", awq_quantize(nullptr, nullptr, 4, 128, 128, (uint32_t*)F, F, F, nullptr), AWQ_ERR_NULL);
    expect("quantize K % G", awq_quantize(F, nullptr, 4, 100, 64, (uint32_t*)F, F, F, nullptr), AWQ_ERR_SHAPE);
    expect("quantize G", awq_quantize(F, nullptr, 4, 128, 96, (uint32_t*)F, F, F, nullptr), AWQ_ERR_CONFIG);
    expect("quantize N < 0", awq_quantize(F, nullptr, -1, 128, 128, (uint32_t*)F, F, F, nullptr), AWQ_ERR_SHAPE);
    expect("quantize huge N", awq_quantize(F, nullptr, huge, 128, 128, (uint32_t*)F, F, F, nullptr), AWQ_ERR_SHAPE);
    expect("quantize huge K", awq_quantize(F, nullptr, 4, huge - 127, 128, (uint32_t*)F, F, F, nullptr),
           AWQ_ERR_SHAPE);
    expect("quantize N*K", awq_quantize(F, nullptr, big, big, 128, (uint32_t*)F, F, F, nullptr), AWQ_ERR_SHAPE);
    expect("quantize align", awq_quantize(ODD, nullptr, 4, 128, 128, (uint32_t*)F, F, F, nullptr), AWQ_ERR_ALIGN);
    expect("quantize_ex mode", awq_quantize_ex(F, nullptr, 4, 128, 128, 7, 0.0, (uint32_t*)F, F, F, nullptr),
           AWQ_ERR_CONFIG);
    expect("quantize_ex clip", awq_quantize_ex(F, nullptr, 4, 128, 128, 0, 0.3, (uint32_t*)F, F, F, nullptr),
           AWQ_ERR_CONFIG);
    expect("quantize_ex nan clip",
           awq_quantize_ex(F, nullptr, 4, 128, 128, 0, __builtin_nan(""), (uint32_t*)F, F, F,
                           nullptr),
           AWQ_ERR_CONFIG);
    expect("quantize empty", awq_quantize(nullptr, nullptr, 0, 128, 128, nullptr, nullptr, nullptr, nullptr),
           AWQ_OK);

    // linear layer (every path and both workspace forms)
    for (int path = 0; path < 6; ++path) {
        expect("gemm null x", awq_gemm_path(nullptr, (uint32_t*)F, F, F, 16, 64, 128, 128, F, path, nullptr),
               path == 5 ? AWQ_ERR_CONFIG : AWQ_ERR_NULL);
        expect("gemm huge M", awq_gemm_path(F, (uint32_t*)F, F, F, huge, 64, 128, 128, F, path, nullptr),
               path == 5 ? AWQ_ERR_CONFIG : AWQ_ERR_SHAPE);
        expect("gemm huge N", awq_gemm_path(F, (uint32_t*)F, F, F, 4, huge, 128, 128, F, path, nullptr),
               AWQ_ERR_SHAPE);
        expect("noalloc null y", awq_gemm_noalloc(F, (uint32_t*)F, F, F, 16, 64, 128, 128, nullptr, path, nullptr),
               path == 5 ? AWQ_ERR_CONFIG : AWQ_ERR_NULL);
    }
    expect("gemm align x", awq_gemm(ODD, (uint32_t*)F, F, F, 4, 64, 128, 128, F, nullptr), AWQ_ERR_ALIGN);
    expect("gemm align y", awq_gemm(F, (uint32_t*)F, F, F, 4, 64, 128, 128, fake(0x10001), nullptr),
           AWQ_ERR_ALIGN);
    expect("gemm M < 0", awq_gemm(F, (uint32_t*)F, F, F, -5, 64, 128, 128, F, nullptr), AWQ_ERR_SHAPE);
    expect("gemm empty", awq_gemm(nullptr, nullptr, nullptr, nullptr, 0, 64, 128, 128, nullptr, nullptr), AWQ_OK);
    const size_t need = awq_gemm_workspace_bytes(2048, 4096, 4096);
    expect("gemm_ex short ws",
           awq_gemm_ex(F, (uint32_t*)F, F, F, 2048, 4096, 4096, 128, F, 2, WS, need - 1, nullptr), AWQ_ERR_WORKSPACE);
    expect("gemm_ex misaligned ws",
           awq_gemm_ex(F, (uint32_t*)F, F, F, 2048, 4096, 4096, 128, F, 2, fake(0x100010), need, nullptr),
           AWQ_ERR_ALIGN);
    if (awq_gemm_workspace_bytes(huge, 4096, 4096) != 0 || awq_gemm_workspace_bytes(16, -1, 4096) != 0) {
        std::printf("gemm workspace query accepted bad sizes\n");
        ++failures;
    }
    expect("gemm_w8 G", awq_gemm_w8(F, (uint32_t*)F, F, F, 4, 64, 128, 32, F, 0, nullptr, 0, nullptr),
           AWQ_ERR_CONFIG);
    expect("gemm_w8 path", awq_gemm_w8(F, (uint32_t*)F, F, F, 4, 64, 128, 128, F, 3, nullptr, 0, nullptr),
           AWQ_ERR_CONFIG);
    expect("quantize_w8 null", awq_quantize_w8(F, nullptr, 4, 128, 128, 0, nullptr, F, F, nullptr), AWQ_ERR_NULL);

    // activation statistic and the searches
    expect("absmean K % 8", awq_activation_absmean(F, 10, 12, (double*)F, F, 1 << 20, nullptr), AWQ_ERR_SHAPE);
    expect("absmean huge T", awq_activation_absmean(F, huge, 512, (double*)F, F, 1 << 20, nullptr), AWQ_ERR_SHAPE);
    expect("absmean short ws", awq_activation_absmean(F, 1000, 512, (double*)F, F, 8, nullptr), AWQ_ERR_WORKSPACE);
    double losses[64];
    int best = -1;
    const double alphas[2] = {0.0, __builtin_nan("")};
    const size_t ns = awq_scale_search_workspace_bytes(256, 512, 1024, 128, 20);
    expect("search short ws",
           awq_scale_search(F, F, 256, 512, 1024, 128, nullptr, 20, F, ns - 256, losses, &best, (float*)F, nullptr),
           AWQ_ERR_WORKSPACE);
    expect("search nan alpha",
           awq_scale_search(F, F, 256, 512, 1024, 128, alphas, 2, F, ns, losses, &best, (float*)F, nullptr),
           AWQ_ERR_CONFIG);
    expect("search n_alpha", awq_scale_search(F, F, 256, 512, 1024, 128, nullptr, 65, F, ns, losses, &best,
                                              (float*)F, nullptr),
           AWQ_ERR_CONFIG);
    expect("search huge T", awq_scale_search(F, F, 256, 512, huge, 128, nullptr, 20, F, ns, losses, &best,
                                             (float*)F, nullptr),
           AWQ_ERR_SHAPE);
    if (awq_scale_search_workspace_bytes(256, 500, 1024, 128, 20) != 0) {
        std::printf("search workspace query accepted K %% G != 0\n");
        ++failures;
    }
    const double fr[2] = {0.0, 0.5};
    const size_t nc = awq_clip_search_workspace_bytes(256, 512, 1024, 128, 2, 0);
    expect("clip bad fraction",
           awq_clip_search(F, F, nullptr, 256, 512, 1024, 128, 0, fr, 2, F, nc, losses, &best, nullptr),
           AWQ_ERR_CONFIG);
    expect("clip mode", awq_clip_search(F, F, nullptr, 256, 512, 1024, 128, 3, fr, 1, F, nc, losses, &best, nullptr),
           AWQ_ERR_CONFIG);

    // fp16 salient channels
    expect("select K", awq_select_salient((double*)F, (int64_t(1) << 17) + 1, 4, (int*)F, nullptr), AWQ_ERR_SHAPE);
    expect("select n > K", awq_select_salient((double*)F, 16, 17, (int*)F, nullptr), AWQ_ERR_SHAPE);
    expect("select empty", awq_select_salient(nullptr, 16, 0, nullptr, nullptr), AWQ_OK);
    expect("salient quantize n", awq_quantize_salient(F, 4, 128, 128, 0, (int*)F, 129, (uint32_t*)F, F, F, F,
                                                      nullptr),
           AWQ_ERR_SHAPE);
    expect("salient apply null", awq_salient_apply(F, nullptr, F, 4, 64, 128, 2, F, nullptr), AWQ_ERR_NULL);
    double lr = 0, ls = 0;
    const size_t nl = awq_salient_loss_workspace_bytes(256, 1024, 512, 128, -1);
    expect("salient loss short ws",
           awq_salient_loss(F, F, 256, 1024, 512, 128, 0, -1, F, nl - 16, &lr, &ls, nullptr, nullptr),
           AWQ_ERR_WORKSPACE);
    if (awq_salient_count(4096) != 41 || awq_salient_count(-7) != 0 || awq_salient_count(huge) <= 0) {
        std::printf("salient count\n");
        ++failures;
    }

    if (failures) return 1;
    std::printf("ok\n");
    return 0;
}
