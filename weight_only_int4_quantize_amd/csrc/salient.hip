// Mixed precision with the salient weights kept in fp16
// ("AWQ 模型量化技术：激活感知的权重量化革命", 技术实现 1 and 混合精度设计:
// the important 1 % of the weights, identified from the activation
// distribution, stay in fp16 while the rest is quantized to 4 bits;
// xxmr.cn §2.2).
//
// Stored form: the usual INT4 matrix of all of W (each group's range over
// all its weights), with the codes of the salient input channels set to
// their group's zero-point so that they dequantize to exactly 0, plus the
// salient weights w_salient[j, n] = W[n, idx[j]] in fp16. The layer is then
// the W4A16 product plus a small side product x[:, idx] . w_salient.
//
//  * select: idx = the n channels of largest m[k] (mean |x|), by descending
//    m, equal m by ascending k. Each thread ranks its channel against all K
//    (count of larger, plus equal with a smaller index) and writes itself to
//    slot rank when rank < n: K^2 compares, no sort, deterministic.
//  * fix: one thread per output row rewrites the salient nibbles of its row
//    (sequentially, so nibbles sharing a word never race) and gathers the
//    row's salient weights into w_salient (coalesced across rows).
//  * apply: y[m, n] += sum_j x[m, idx[j]] * w_salient[j, n] in fp32. A block
//    covers 32 rows x 256 columns: the gathered x of its rows goes through
//    LDS in chunks of 32 channels, each thread keeps 32 row accumulators for
//    its column and reads w_salient coalesced. The fp16 form rounds
//    fp32(y) + sum once; the fp32 form subtracts the sum from a reference
//    output kept in the tiled layout of ref_offset (the loss of the mixed
//    layer against W x^T). Decode batches
//    (M <= 8) take a narrower form with more blocks (see apply_small_kernel).
#include "awq_internal.h"

namespace awq {
namespace {

constexpr int kSelThreads = 256;

__global__ __launch_bounds__(kSelThreads) void select_kernel(const double* __restrict__ m, int K, int n,
                                                             int* __restrict__ idx) {
    __shared__ double tile[kSelThreads];
    const int k = blockIdx.x * kSelThreads + threadIdx.x;
    const double mk = k < K ? m[k] : 0.0;
    int rank = 0;
    for (int j0 = 0; j0 < K; j0 += kSelThreads) {
        const int j = j0 + threadIdx.x;
        tile[threadIdx.x] = j < K ? m[j] : 0.0;
        __syncthreads();
        const int cnt = min(kSelThreads, K - j0);
        for (int t = 0; t < cnt; ++t) {
            const double mj = tile[t];
            rank += (mj > mk) || (mj == mk && j0 + t < k);
        }
        __syncthreads();
    }
    if (k < K && rank < n) idx[rank] = k;
}

// Indices outside [0, K) are skipped (their w_salient entries become 0).
__global__ __launch_bounds__(256) void fix_kernel(const half_t* __restrict__ w, int64_t N, int64_t K, int G,
                                                  const int* __restrict__ idx, int n_sal,
                                                  uint32_t* __restrict__ qweight, const half_t* __restrict__ zeros,
                                                  half_t* __restrict__ w_sal) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (row >= N) return;
    const int64_t ngroups = K / G;
    uint32_t* qrow = qweight + row * (K / 8);
    for (int j = 0; j < n_sal; ++j) {
        const int k = idx[j];
        half_t v = static_cast<half_t>(0.0f);
        if (k >= 0 && k < K) {
            const uint32_t z = static_cast<uint32_t>(static_cast<float>(zeros[row * ngroups + k / G]));
            const int sh = 4 * (k % 8);
            qrow[k / 8] = (qrow[k / 8] & ~(0xFu << sh)) | ((z & 0xFu) << sh);
            v = w[row * K + k];
        }
        w_sal[static_cast<int64_t>(j) * N + row] = v;
    }
}

constexpr int kApRows = 32;
constexpr int kApCols = 256;
constexpr int kApChunk = 32;

template <bool F32_SUB>
__global__ __launch_bounds__(kApCols) void apply_kernel(const half_t* __restrict__ x, const int* __restrict__ idx,
                                                        const half_t* __restrict__ w_sal, int64_t M, int64_t N,
                                                        int64_t K, int n_sal, int64_t tiles_n,
                                                        half_t* __restrict__ y16, float* __restrict__ y32) {
    __shared__ float xs[kApRows][kApChunk + 1];
    const int64_t tile = blockIdx.x;
    const int64_t m0 = (tile / tiles_n) * kApRows;
    const int64_t n = (tile % tiles_n) * kApCols + threadIdx.x;
    float acc[kApRows];
#pragma unroll
    for (int r = 0; r < kApRows; ++r) acc[r] = 0.f;
    for (int j0 = 0; j0 < n_sal; j0 += kApChunk) {
        for (int e = threadIdx.x; e < kApRows * kApChunk; e += kApCols) {
            const int r = e / kApChunk, jj = e % kApChunk;
            const int64_t mm = m0 + r;
            float v = 0.f;
            if (mm < M && j0 + jj < n_sal) {
                const int k = idx[j0 + jj];
                if (k >= 0 && k < K) v = static_cast<float>(x[mm * K + k]);
            }
            xs[r][jj] = v;
        }
        __syncthreads();
        const int cnt = min(kApChunk, n_sal - j0);
        if (n < N) {
            for (int jj = 0; jj < cnt; ++jj) {
                const float wv = static_cast<float>(w_sal[static_cast<int64_t>(j0 + jj) * N + n]);
#pragma unroll
                for (int r = 0; r < kApRows; ++r) acc[r] += xs[r][jj] * wv;
            }
        }
        __syncthreads();
    }
    if (n >= N) return;
    if constexpr (F32_SUB) {
        // the tiled reference layout (ref_offset): the 32 rows are one
        // sub-tile's; its lane n % 32 holds rows 8q + 0..3 as 16 contiguous
        // floats, lane n % 32 + 32 rows 8q + 4..7. Rows past M are padding.
        float4_t* p = reinterpret_cast<float4_t*>(
            y32 + ref_subtile_base(m0, n / 32 * 32, (N + kRefTileN - 1) / kRefTileN) + (n % 32) * 16);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4_t v = p[h * 32 * 4 + q];
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] -= acc[q * 8 + h * 4 + k];
                p[h * 32 * 4 + q] = v;
            }
    } else {
#pragma unroll
        for (int r = 0; r < kApRows; ++r) {
            const int64_t mm = m0 + r;
            if (mm < M) {
                const float v = static_cast<float>(y16[mm * N + n]) + acc[r];
                y16[mm * N + n] = static_cast<half_t>(v);
            }
        }
    }
}

// Decode form (M <= kSmallRows): a block covers 64 columns; its 4 waves
// take interleaved quarters of the salient channels (lane = column, so
// w_salient reads stay coalesced), the gathered x of all rows goes through
// LDS 256 channels at a time, and the 4 partial sums are added in wave
// order through LDS, so the result does not depend on scheduling.
constexpr int kSmallRows = 8;
constexpr int kSmallCols = 64;
constexpr int kSmallChunk = 256;

template <int MR, bool F32_SUB>
__global__ __launch_bounds__(256) void apply_small_kernel(const half_t* __restrict__ x, const int* __restrict__ idx,
                                                          const half_t* __restrict__ w_sal, int M, int64_t N,
                                                          int64_t K, int n_sal, half_t* __restrict__ y16,
                                                          float* __restrict__ y32) {
    __shared__ float xs[MR][kSmallChunk];
    __shared__ float red[4][MR][kSmallCols];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n = static_cast<int64_t>(blockIdx.x) * kSmallCols + lane;
    float acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0.f;
    for (int j0 = 0; j0 < n_sal; j0 += kSmallChunk) {
        const int cnt = min(kSmallChunk, n_sal - j0);
        {
            const int jj = threadIdx.x;
            int k = -1;
            if (jj < cnt) k = idx[j0 + jj];
#pragma unroll
            for (int r = 0; r < MR; ++r)
                xs[r][jj] = (r < M && k >= 0 && k < K) ? static_cast<float>(x[static_cast<int64_t>(r) * K + k]) : 0.f;
        }
        __syncthreads();
        if (n < N) {
            for (int jj = wave; jj < cnt; jj += 4) {
                const float wv = static_cast<float>(w_sal[static_cast<int64_t>(j0 + jj) * N + n]);
#pragma unroll
                for (int r = 0; r < MR; ++r) acc[r] += xs[r][jj] * wv;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (wave != 0 || n >= N) return;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        if (r < M) {
            const float v = ((red[0][r][lane] + red[1][r][lane]) + red[2][r][lane]) + red[3][r][lane];
            if constexpr (F32_SUB) {
                y32[ref_offset(r, n, (N + kRefTileN - 1) / kRefTileN)] -= v;
            } else {
                y16[static_cast<int64_t>(r) * N + n] = static_cast<half_t>(static_cast<float>(
                                                           y16[static_cast<int64_t>(r) * N + n]) + v);
            }
        }
    }
}

template <bool F32_SUB>
awq_status launch_apply_t(const half_t* x, const int* idx, const half_t* w_sal, int64_t M, int64_t N, int64_t K,
                          int n_sal, half_t* y16, float* y32, hipStream_t stream) {
    if (M == 0 || N == 0 || n_sal == 0) return AWQ_OK;
    if (M <= kSmallRows) {
        const int64_t blocks = ceil_div(N, kSmallCols);
        if (blocks >= (int64_t{1} << 31)) return AWQ_ERR_SHAPE;
        hipLaunchKernelGGL((apply_small_kernel<kSmallRows, F32_SUB>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                           0, stream, x, idx, w_sal, static_cast<int>(M), N, K, n_sal, y16, y32);
        return last_launch_status();
    }
    const int64_t tiles_n = ceil_div(N, kApCols);
    const int64_t tiles = ceil_div(M, kApRows) * tiles_n;
    if (tiles >= (int64_t{1} << 31)) return AWQ_ERR_SHAPE;
    hipLaunchKernelGGL((apply_kernel<F32_SUB>), dim3(static_cast<unsigned>(tiles)), dim3(kApCols), 0, stream, x,
                       idx, w_sal, M, N, K, n_sal, tiles_n, y16, y32);
    return last_launch_status();
}

}  // namespace

awq_status launch_select_salient(const double* m, int64_t K, int n, int* idx, hipStream_t stream) {
    if (n == 0) return AWQ_OK;
    const int64_t blocks = ceil_div(K, kSelThreads);
    hipLaunchKernelGGL(select_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kSelThreads), 0, stream, m,
                       static_cast<int>(K), n, idx);
    return last_launch_status();
}

awq_status launch_salient_fix(const half_t* w, int64_t N, int64_t K, int group_size, const int* idx, int n_sal,
                              uint32_t* qweight, const half_t* zeros, half_t* w_sal, hipStream_t stream) {
    if (N == 0 || n_sal == 0) return AWQ_OK;
    hipLaunchKernelGGL(fix_kernel, dim3(static_cast<unsigned>(ceil_div(N, 256))), dim3(256), 0, stream, w, N, K,
                       group_size, idx, n_sal, qweight, zeros, w_sal);
    return last_launch_status();
}

awq_status launch_salient_apply(const half_t* x, const int* idx, const half_t* w_sal, int64_t M, int64_t N,
                                int64_t K, int n_sal, half_t* y, hipStream_t stream) {
    return launch_apply_t<false>(x, idx, w_sal, M, N, K, n_sal, y, nullptr, stream);
}

awq_status launch_salient_subtract(const half_t* x, const int* idx, const half_t* w_sal, int64_t M, int64_t N,
                                   int64_t K, int n_sal, float* y32, hipStream_t stream) {
    return launch_apply_t<true>(x, idx, w_sal, M, N, K, n_sal, nullptr, y32, stream);
}

}  // namespace awq
