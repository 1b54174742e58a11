// Kernels of AWQ's activation-aware scale search (rskf.cn AWQ article §2.1:
// per-input-channel s, weights times s, activations divided by s, s chosen to
// minimise the difference between the quantized and the original output;
// "AWQ 模型量化技术：激活感知的权重量化革命", Per-channel Scaling 优化: the
// search is driven by the activation distribution).
//
//  * absmean: m[k] = mean_t |x[t, k]|, a column reduction of the calibration
//    activations. A block covers 256 columns (32 lanes x 8 halves, one
//    16-byte load each) and a slice of rows; 8 row-lanes per column group
//    accumulate in fp64 and combine through LDS, then one pass adds the
//    slices in a fixed order. fp64 makes the statistic exact to the last bits
//    of an fp64 sum and independent of scheduling.
//  * pow_scales: s[k] = float32(m[k] ^ alpha) with fp64 pow.
//  * divide_columns: x'[t, k] = fp16(x[t, k] / s[k]) (IEEE fp32 divide).
//  * sum_partials: deterministic fixed-order sum of per-tile loss partials,
//    over many blocks when they are many.
#include "awq_internal.h"

namespace awq {
namespace {

#pragma clang fp contract(off)

constexpr int kAbsRowsPerSlice = 256;

__global__ __launch_bounds__(256) void absmean_partial_kernel(const half_t* __restrict__ x, int64_t T,
                                                              int64_t K, double* __restrict__ partials) {
    __shared__ double red[8][32][8 + 1];
    const int col_lane = threadIdx.x & 31;   // which 8-column word
    const int row_lane = threadIdx.x >> 5;   // 0..7
    const int64_t k0 = (static_cast<int64_t>(blockIdx.x) * 32 + col_lane) * 8;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kAbsRowsPerSlice;
    const int64_t t1 = min(T, t0 + kAbsRowsPerSlice);
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (k0 < K) {
        for (int64_t t = t0 + row_lane; t < t1; t += 8) {
            const uint4 r = *reinterpret_cast<const uint4*>(x + t * K + k0);
            const uint32_t p[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half_t lo = __builtin_bit_cast(half_t, static_cast<uint16_t>(p[i] & 0xFFFFu));
                const half_t hi = __builtin_bit_cast(half_t, static_cast<uint16_t>(p[i] >> 16));
                acc[2 * i] += fabs(static_cast<double>(lo));
                acc[2 * i + 1] += fabs(static_cast<double>(hi));
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[row_lane][col_lane][j] = acc[j];
    __syncthreads();
    if (row_lane == 0 && k0 < K) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            double s = 0.0;
            for (int r = 0; r < 8; ++r) s += red[r][col_lane][j];
            partials[static_cast<int64_t>(blockIdx.y) * K + k0 + j] = s;
        }
    }
}

__global__ __launch_bounds__(256) void absmean_final_kernel(const double* __restrict__ partials,
                                                            int64_t slices, int64_t T, int64_t K,
                                                            double* __restrict__ m) {
    const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (k >= K) return;
    double s = 0.0;
    for (int64_t i = 0; i < slices; ++i) s += partials[i * K + k];
    const double mean = s / static_cast<double>(T);
    m[k] = mean > kMeanFloor ? mean : kMeanFloor;
}

__global__ __launch_bounds__(256) void pow_scales_kernel(const double* __restrict__ m, int64_t K,
                                                         double alpha, float* __restrict__ s) {
    const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (k >= K) return;
    // alpha = 0 gives exactly 1 (the identity the search relies on to
    // skip x / s there)
    s[k] = alpha == 0.0 ? 1.0f : static_cast<float>(pow(m[k], alpha));
}

__global__ __launch_bounds__(256) void divide_columns_kernel(const half_t* __restrict__ x,
                                                             const float* __restrict__ s, int64_t n_words,
                                                             int64_t words_per_row, half_t* __restrict__ xs) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= n_words) return;
    const int64_t k0 = (t % words_per_row) * 8;
    const uint4 r = reinterpret_cast<const uint4*>(x)[t];
    const float4 c0 = *reinterpret_cast<const float4*>(s + k0);
    const float4 c1 = *reinterpret_cast<const float4*>(s + k0 + 4);
    const float sc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const uint32_t p[4] = {r.x, r.y, r.z, r.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(p[i] & 0xFFFFu)));
        const float hi = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(p[i] >> 16)));
        const half_t qlo = static_cast<half_t>(lo / sc[2 * i]);
        const half_t qhi = static_cast<half_t>(hi / sc[2 * i + 1]);
        o[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, qlo)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, qhi)) << 16);
    }
    reinterpret_cast<uint4*>(xs)[t] = make_uint4(o[0], o[1], o[2], o[3]);
}

// Fixed-order sum of n doubles: block b adds the slice [b n / B, (b + 1) n / B)
// (each thread a strided part, then a tree over the block) into out[b]; with
// one block the slice is the whole range. Run as B blocks, then one block
// over the B block sums, the result depends on n and B only.
__global__ __launch_bounds__(256) void sum_partials_kernel(const double* __restrict__ partials, int64_t n,
                                                           double* __restrict__ out) {
    __shared__ double red[256];
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * n / gridDim.x;
    const int64_t i1 = static_cast<int64_t>(blockIdx.x + 1) * n / gridDim.x;
    double s = 0.0;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += 256) s += partials[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace

size_t absmean_workspace_bytes(int64_t T, int64_t K) {
    const int64_t slices = ceil_div(T, kAbsRowsPerSlice);
    return static_cast<size_t>(slices) * static_cast<size_t>(K) * sizeof(double);
}

awq_status launch_absmean(const half_t* x, int64_t T, int64_t K, double* m, double* partials,
                          hipStream_t stream) {
    const int64_t slices = ceil_div(T, kAbsRowsPerSlice);
    const int64_t col_blocks = ceil_div(K / 8, 32);
    hipLaunchKernelGGL(absmean_partial_kernel, dim3(static_cast<unsigned>(col_blocks), static_cast<unsigned>(slices)),
                       dim3(256), 0, stream, x, T, K, partials);
    awq_status st = last_launch_status();
    if (st != AWQ_OK) return st;
    hipLaunchKernelGGL(absmean_final_kernel, dim3(static_cast<unsigned>(ceil_div(K, 256))), dim3(256), 0, stream,
                       partials, slices, T, K, m);
    return last_launch_status();
}

awq_status launch_pow_scales(const double* m, int64_t K, double alpha, float* s, hipStream_t stream) {
    hipLaunchKernelGGL(pow_scales_kernel, dim3(static_cast<unsigned>(ceil_div(K, 256))), dim3(256), 0, stream, m, K,
                       alpha, s);
    return last_launch_status();
}

awq_status launch_divide_columns(const half_t* x, const float* s, int64_t T, int64_t K, half_t* xs,
                                 hipStream_t stream) {
    const int64_t n_words = T * (K / 8);
    if (n_words == 0) return AWQ_OK;
    hipLaunchKernelGGL(divide_columns_kernel, dim3(static_cast<unsigned>(ceil_div(n_words, 256))), dim3(256), 0,
                       stream, x, s, n_words, K / 8, xs);
    return last_launch_status();
}

awq_status launch_sum_partials(double* partials, int64_t n, double* out, hipStream_t stream) {
    // large counts: kLossSumBlocks blocks into the scratch behind the
    // partials, then one block over those
    if (n >= 64 * 256) {
        hipLaunchKernelGGL(sum_partials_kernel, dim3(kLossSumBlocks), dim3(256), 0, stream, partials, n, partials + n);
        const awq_status st = last_launch_status();
        if (st != AWQ_OK) return st;
        hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(256), 0, stream, partials + n,
                           static_cast<int64_t>(kLossSumBlocks), out);
        return last_launch_status();
    }
    hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(256), 0, stream, partials, n, out);
    return last_launch_status();
}

}  // namespace awq
