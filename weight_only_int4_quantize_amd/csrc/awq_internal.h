// Internal declarations shared by the HIP translation units of the library.
// Only gfx950 (CDNA4) is targeted: 64-lane wavefronts, fp16 MFMA, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/awq.h"

namespace awq {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kQMax = 15;          // 2^4 - 1
constexpr float kRangeFloor = 1e-5f;
constexpr double kMeanFloor = 1e-8;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

inline awq_status hip_status(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP; }

// Compute units of the current device (queried once; 256 on MI355X).
inline int cu_count() {
    static int cached = -1;
    if (cached < 0) {
        int dev = 0, v = 256;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            v = 256;
        cached = v;
    }
    return cached;
}
inline awq_status last_launch_status() { return hip_status(hipGetLastError()); }

// ---- launchers (each returns after enqueueing on `stream`) ----

// Group-wise INT4 quantization of W[N, K] (optionally times channel_scale[K]),
// asymmetric (the group's [min, max]) or symmetric (max |w| -> +-7, zero 8),
// after an optional percentile clip of each group (clip_fraction in [0, 0.25)).
bool clip_fraction_ok(double p);
// bits = 8 gives the W8A16 form (4 codes per word, 255 levels). tiled (INT4,
// K a multiple of 64): the packed words in the searches' loss-GEMM order
// (kTiledB below) instead of row-major [N, K/8].
awq_status launch_quantize(const half_t* w, const float* channel_scale, int64_t N, int64_t K,
                           int group_size, bool symmetric, double clip_fraction, uint32_t* qweight,
                           half_t* scales, half_t* zeros, hipStream_t stream, int bits = 4, bool tiled = false);

// Decode GEMV y[M, N] = x[M, K] . dequant(Wq)^T for M <= kGemvMaxM.
constexpr int kGemvMaxM = 8;
// bits = 8: the W8A16 form (qweight [N, K/4], four byte codes per word).
bool gemv_supported(int64_t M, int64_t K, int bits = 4);
// Layers of few rows and long rows that the GEMV takes one-shot (every item
// of a row in flight); the automatic choice prefers it there up to M = 4.
bool gemv_few_rows(int64_t M, int64_t N, int64_t K, int bits = 4);
awq_status launch_gemv(const half_t* x, const uint32_t* qweight, const half_t* scales,
                       const half_t* zeros, int64_t M, int64_t N, int64_t K, int group_size,
                       half_t* y, hipStream_t stream, int bits = 4);
// Several INT4 layers that share x (and K, G) in one GEMV launch: their rows
// stacked in order, layer i < n owning rows [row0[i], row0[i + 1]), each row
// read from and written to its own layer's tensors; row0[n] is the total and
// the entries past it are INT_MAX. M <= kGemvGroupedMaxM.
constexpr int kGemvMaxLayers = 4;
constexpr int kGemvGroupedMaxM = 2;
struct GemvLayers {
    const uint32_t* qweight[kGemvMaxLayers];
    const half_t* scales[kGemvMaxLayers];
    const half_t* zeros[kGemvMaxLayers];
    half_t* y[kGemvMaxLayers];
    int row0[kGemvMaxLayers + 1];
    int n;
};
awq_status launch_gemv_grouped(const half_t* x, const GemvLayers& layers, int64_t M, int64_t K, int group_size,
                               hipStream_t stream);

// MFMA GEMM. The B operand is INT4 or W8 (qweight/scales/zeros) or fp16 W[N, K].
enum class GemmB { kInt4, kF16, kInt8 };
enum class GemmOut { kF16, kF32, kLoss };
// The searches' fp32 reference output (kF32 results, kLoss references) is
// kept in the accumulator order of v_mfma_f32_32x32x16: 256 x 128 tiles
// (row-major over ceil(N / 128) tile columns), each of 32 sub-tiles of
// 32 x 32 ordered by (column block of 32, row block of 32), each sub-tile
// 64 lanes x 16 floats, lane L and element e holding row
// 8 (e / 4) + 4 (L / 32) + e % 4 and column L % 32 of the sub-tile. A lane
// thus reads or writes its 16 values of a sub-tile as four 16-byte
// accesses. The buffer holds whole tiles (rows padded to 256, columns to
// 128); padding positions hold nothing meaningful.
constexpr int kRefTileM = 256;
constexpr int kRefTileN = 128;
__host__ __device__ inline int64_t ref_tiled_floats(int64_t M, int64_t N) {
    return (M + kRefTileM - 1) / kRefTileM * kRefTileM * ((N + kRefTileN - 1) / kRefTileN * kRefTileN);
}
// first float of the 32 x 32 sub-tile starting at (m0, n0), both multiples of 32
__host__ __device__ inline int64_t ref_subtile_base(int64_t m0, int64_t n0, int64_t tiles_n) {
    const int64_t tile = (m0 / kRefTileM) * tiles_n + n0 / kRefTileN;
    return (tile * 32 + ((n0 % kRefTileN) / 32) * 8 + (m0 % kRefTileM) / 32) * 1024;
}
__host__ __device__ inline int64_t ref_offset(int64_t m, int64_t n, int64_t tiles_n) {
    const int64_t lane = n % 32 + 32 * ((m % 8) / 4);
    const int64_t e = ((m % 32) / 8) * 4 + m % 4;
    return ref_subtile_base(m / 32 * 32, n / 32 * 32, tiles_n) + lane * 16 + e;
}

struct GemmArgs {
    const half_t* a = nullptr;        // [M, K]
    const uint32_t* qweight = nullptr;
    const half_t* scales = nullptr;
    const half_t* zeros = nullptr;
    const half_t* w = nullptr;        // fp16 B, [N, K]
    int group_size = 128;
    int64_t M = 0, N = 0, K = 0;
    half_t* y16 = nullptr;            // kF16 output [M, N]
    float* y32 = nullptr;             // kF32 output [M, N], tiled (ref_offset)
    const float* yref = nullptr;      // kLoss reference [M, N], tiled (ref_offset)
    double* partials = nullptr;       // kLoss: one double per tile
    // kLoss with INT4 B: qweight in the tiled order (word c of row n at
    // ((n / 32 * K / 64 + c / 8) * 64 + (c / 4 % 2) * 32 + n % 32) * 4 + c % 4,
    // ceil(N / 32) * 32 rows), so a wave's packed words of one 64-k step
    // are one contiguous 1 KB piece. kF32 with fp16 B: w in the tiled order
    // of launch_tile_fp16_b.
    bool b_tiled = false;
};
// fp16 W[N, K] (K a multiple of 64) into the fp16-B reference's tiled order:
// 16-byte piece (lane, v) of 32-row group g and 64-k step t, at piece index
// ((g * K / 64 + t) * 4 + v) * 64 + lane, holds W[32 g + lane % 32]
// [64 t + 32 (lane / 32) + 8 v .. + 7]; rows past N are zero. wt holds
// tiled_fp16_halves(N, K) halves.
inline size_t tiled_fp16_halves(int64_t N, int64_t K) {
    return static_cast<size_t>((N + 31) / 32 * 32) * static_cast<size_t>(K);
}
awq_status launch_tile_fp16_b(const half_t* w, int64_t N, int64_t K, half_t* wt, hipStream_t stream);
// whether the fp16-B reference takes tiled B at this K
bool gemm_ref_tiled_ok(int64_t K);
// whether the loss form takes tiled B at this K and group size
bool gemm_tiled_ok(int64_t K, int group_size);
// words of a tiled packed-weight buffer of N rows
inline size_t tiled_qweight_words(int64_t N, int64_t K) {
    return static_cast<size_t>((N + 31) / 32 * 32) * static_cast<size_t>(K / 8);
}
// Workspaces of the split kernels (GEMM stream-K, skinny K splits) start
// with one shared region of tile counters: the counters of any call sit at
// offset 0 and are back at zero when its kernel ends, so one workspace
// serves calls of every shape and both kernels. Splits are only used for at
// most split_counter_slots() output tiles.
inline int split_counter_slots() { return 4 * cu_count(); }
inline size_t split_counter_bytes() { return round_up(static_cast<size_t>(split_counter_slots()) * sizeof(int), 256); }

// Output tiles of the loss-form GEMM launch (one loss partial each).
int64_t gemm_tile_count(int64_t M, int64_t N);
// Workspace of the stream-K launch (fp32 partial tiles + per-tile counters);
// with workspace == nullptr launch_gemm runs one tile per block.
size_t gemm_workspace_bytes(int64_t M, int64_t N);
awq_status launch_gemm(const GemmArgs& args, GemmB b, GemmOut out, hipStream_t stream,
                       void* workspace = nullptr);

// Skinny MFMA GEMM for 4 < M <= 64 (decode batches): 16x16x32 MFMAs whose B
// operand is one packed word per lane, K optionally split across blocks
// (workspace != nullptr) with a fixed-order in-kernel fixup. Without K
// splits a block walks all of K, in LDS-sized phases if need be.
constexpr int kSkinnyMaxM = 64;
// phased (optional): set when the call would walk K in LDS-sized phases on
// one block per column tile (no K splits), the slow form.
bool skinny_supported(int64_t M, int64_t N, int64_t K, int group_size, bool have_workspace,
                      bool* phased = nullptr);
size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K);
awq_status launch_skinny(const half_t* x, const uint32_t* qweight, const half_t* scales,
                         const half_t* zeros, int64_t M, int64_t N, int64_t K, int group_size,
                         half_t* y, void* workspace, hipStream_t stream);

// Column-tile MFMA kernel for small batches (M <= kColTileMaxM): one block
// per 16 output columns over all of K, x read straight into the MFMA A
// operand, the waves' K ranges added in LDS; no workspace.
constexpr int kColTileMaxM = 32;
bool coltile_supported(int64_t M, int64_t N, int64_t K, int group_size);
// whether the automatic choice takes it (by measured times against the GEMV
// and the skinny kernel, which has K splits only with a workspace)
bool coltile_preferred(int64_t M, int64_t N, int64_t K, int group_size, bool have_workspace);
awq_status launch_coltile(const half_t* x, const uint32_t* qweight, const half_t* scales,
                          const half_t* zeros, int64_t M, int64_t N, int64_t K, int group_size,
                          half_t* y, hipStream_t stream);
// The layers of `layers` (as for launch_gemv_grouped), sharing x, in one
// column-tile launch: each layer on whole blocks of its own columns, the
// tile and wave counts those of their total rows.
awq_status launch_coltile_grouped(const half_t* x, const GemvLayers& layers, int64_t M, int64_t K,
                                  int group_size, hipStream_t stream);
// whether that launch can run (its tile and wave counts from the layers' own
// blocks, and their LDS)
bool coltile_grouped_supported(int64_t M, const GemvLayers& layers, int64_t K, int group_size);

// Mixed precision with fp16 salient channels.
awq_status launch_select_salient(const double* m, int64_t K, int n, int* idx, hipStream_t stream);
awq_status launch_salient_fix(const half_t* w, int64_t N, int64_t K, int group_size, const int* idx, int n_sal,
                              uint32_t* qweight, const half_t* zeros, half_t* w_sal, hipStream_t stream);
awq_status launch_salient_apply(const half_t* x, const int* idx, const half_t* w_sal, int64_t M, int64_t N,
                                int64_t K, int n_sal, half_t* y, hipStream_t stream);
awq_status launch_salient_subtract(const half_t* x, const int* idx, const half_t* w_sal, int64_t M, int64_t N,
                                   int64_t K, int n_sal, float* y32, hipStream_t stream);

// Scale-search helpers.
size_t absmean_workspace_bytes(int64_t T, int64_t K);
awq_status launch_absmean(const half_t* x, int64_t T, int64_t K, double* m, double* partials,
                          hipStream_t stream);
awq_status launch_pow_scales(const double* m, int64_t K, double alpha, float* s, hipStream_t stream);
awq_status launch_divide_columns(const half_t* x, const float* s, int64_t T, int64_t K, half_t* xs,
                                 hipStream_t stream);
// Sum of n per-tile loss partials into *out, in a fixed order. The buffer
// holds kLossSumBlocks doubles of scratch behind the n partials.
constexpr int kLossSumBlocks = 256;
awq_status launch_sum_partials(double* partials, int64_t n, double* out, hipStream_t stream);

}  // namespace awq
