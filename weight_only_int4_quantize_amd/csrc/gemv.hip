// Decode GEMV of the W4A16 linear layer, y[M, N] = x[M, K] . dequant(Wq)^T
// for small M (single-stream decode: the "GEMV" kernel choice of the rskf.cn
// AWQ article, §3.3; the dequantize-in-the-matmul step of §1.3). Decode is
// bound by streaming the packed weights from HBM, so the kernel is built
// around 16-byte coalesced loads of qweight with everything else kept on chip.
//
// Work split:
//  * a block (4 wavefronts) owns 4 * RPW consecutive output rows; each
//    wavefront owns RPW rows and walks K with its 64 lanes: lane l handles the
//    32-weight chunks c = l, l + 64, ... (one uint4 of qweight per row), so a
//    wave-wide load is 1 KB of contiguous packed weights per row;
//  * x is staged once per block in LDS, rearranged into the fp16 pairs that
//    match the nibble unpack below, together with two per-chunk sums;
//  * the partial dot products are reduced across the wavefront with xor
//    shuffles at the end (no atomics: results are deterministic).
//
// Nibble unpack (8 codes of one word, code j in bits 4j..4j+3): OR-ing a
// nibble into the mantissa of an fp16 constant gives an exact fp16 integer:
//   (w & 0x000F000F) | 0x64006400 = (1024 + q0, 1024 + q4)
//   (w & 0x00F000F0) | 0x54005400 = (  64 + q1,   64 + q5)
// and the same on w >> 8 for (q2, q6) and (q3, q7). v_dot2_f32_f16 multiplies
// these with the matching x pairs; the constant offsets and the zero-point
// are removed per chunk with the precomputed sums
//   off = 1024 * sum_{j even} x_j + 64 * sum_{j odd} x_j,   xs = sum_j x_j,
// so sum_k x_k (q_k - z) = dot - off - z * xs, scaled by the group's scale.
#include "awq_internal.h"

namespace awq {
namespace {

__device__ inline half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ inline float h_lo(uint32_t u) {
    return static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(u & 0xFFFFu)));
}
__device__ inline float h_hi(uint32_t u) {
    return static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(u >> 16)));
}

// dot of one packed word (8 codes, offset-encoded) with its 4 x pairs
__device__ inline float word_dot(uint32_t wq, const uint4& p, float acc) {
    const uint32_t w8 = wq >> 8;
    const uint32_t a = (wq & 0x000F000Fu) | 0x64006400u;
    const uint32_t b = (wq & 0x00F000F0u) | 0x54005400u;
    const uint32_t c = (w8 & 0x000F000Fu) | 0x64006400u;
    const uint32_t d = (w8 & 0x00F000F0u) | 0x54005400u;
    acc = __builtin_amdgcn_fdot2(as_h2(a), as_h2(p.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(b), as_h2(p.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(c), as_h2(p.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(d), as_h2(p.w), acc, false);
    return acc;
}

template <int MT, int RPW>
__global__ __launch_bounds__(256) void gemv_kernel(const half_t* __restrict__ x,
                                                   const uint32_t* __restrict__ qweight,
                                                   const half_t* __restrict__ scales,
                                                   const half_t* __restrict__ zeros,
                                                   half_t* __restrict__ y, int N, int K,
                                                   int log2g) {
    extern __shared__ uint4 smem[];
    const int nchunk = K >> 5;                      // 32 weights per chunk
    uint4* xp = smem;                               // [MT][nchunk][4] x pairs
    float2* xo = reinterpret_cast<float2*>(smem + MT * nchunk * 4);  // [MT][nchunk] (off, xs)

    for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4* src = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(m) * K) + c * 4;
            float even = 0.f, odd = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 r = src[j];  // halves (0,1) (2,3) (4,5) (6,7)
                uint4 p;
                p.x = (r.x & 0xFFFFu) | (r.z << 16);            // (x0, x4)
                p.y = (r.x >> 16) | (r.z & 0xFFFF0000u);        // (x1, x5)
                p.z = (r.y & 0xFFFFu) | (r.w << 16);            // (x2, x6)
                p.w = (r.y >> 16) | (r.w & 0xFFFF0000u);        // (x3, x7)
                xp[(m * nchunk + c) * 4 + j] = p;
                even += (h_lo(r.x) + h_lo(r.y)) + (h_lo(r.z) + h_lo(r.w));
                odd += (h_hi(r.x) + h_hi(r.y)) + (h_hi(r.z) + h_hi(r.w));
            }
            xo[m * nchunk + c] = make_float2(1024.0f * even + 64.0f * odd, even + odd);
        }
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int row0 = (blockIdx.x * 4 + wave) * RPW;
    if (row0 >= N) return;
    const int ngroups = K >> log2g;
    const uint4* q4 = reinterpret_cast<const uint4*>(qweight);

    int rows[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) rows[i] = min(row0 + i, N - 1);

    float acc[RPW][MT];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[i][m] = 0.f;

    for (int c = lane; c < nchunk; c += kWave) {
        uint4 wv[RPW];
        float s[RPW], z[RPW];
        const int g = (c << 5) >> log2g;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            wv[i] = q4[static_cast<int64_t>(rows[i]) * nchunk + c];
            s[i] = static_cast<float>(scales[static_cast<int64_t>(rows[i]) * ngroups + g]);
            z[i] = static_cast<float>(zeros[static_cast<int64_t>(rows[i]) * ngroups + g]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4* pp = xp + (m * nchunk + c) * 4;
            const uint4 p0 = pp[0], p1 = pp[1], p2 = pp[2], p3 = pp[3];
            const float2 o = xo[m * nchunk + c];
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                float d = 0.f;
                d = word_dot(wv[i].x, p0, d);
                d = word_dot(wv[i].y, p1, d);
                d = word_dot(wv[i].z, p2, d);
                d = word_dot(wv[i].w, p3, d);
                acc[i][m] += s[i] * (d - (o.x + z[i] * o.y));
            }
        }
    }

#pragma unroll
    for (int i = 0; i < RPW; ++i) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float v = acc[i][m];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
            acc[i][m] = v;
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if (row0 + i < N) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    y[static_cast<int64_t>(m) * N + row0 + i] = static_cast<half_t>(acc[i][m]);
            }
        }
    }
}

int max_shared_bytes() {
    static int cached = -1;
    if (cached < 0) {
        int dev = 0, v = 65536;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess) {
            cached = v;
        } else {
            cached = 65536;
        }
    }
    return cached;
}

size_t gemv_lds_bytes(int64_t M, int64_t K) { return static_cast<size_t>(M) * static_cast<size_t>(K / 32) * 72; }

template <int MT, int RPW>
awq_status launch_t(const half_t* x, const uint32_t* qweight, const half_t* scales,
                    const half_t* zeros, int64_t N, int64_t K, int log2g, half_t* y,
                    hipStream_t stream) {
    const size_t lds = gemv_lds_bytes(MT, K);
    static bool attr_set = false;
    if (!attr_set && lds > 65536) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<MT, RPW>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, max_shared_bytes()) != hipSuccess)
            return AWQ_ERR_HIP;
        attr_set = true;
    }
    const int64_t rows_per_block = 4 * RPW;
    const int64_t blocks = ceil_div(N, rows_per_block);
    hipLaunchKernelGGL((gemv_kernel<MT, RPW>), dim3(static_cast<unsigned>(blocks)), dim3(256), lds,
                       stream, x, qweight, scales, zeros, y, static_cast<int>(N), static_cast<int>(K),
                       log2g);
    return last_launch_status();
}

template <int MT>
awq_status launch_m(const half_t* x, const uint32_t* qweight, const half_t* scales,
                    const half_t* zeros, int64_t N, int64_t K, int log2g, half_t* y,
                    hipStream_t stream) {
    // Small N: fewer rows per wave keeps more blocks in flight.
    if (N >= 8192) return launch_t<MT, 4>(x, qweight, scales, zeros, N, K, log2g, y, stream);
    return launch_t<MT, 2>(x, qweight, scales, zeros, N, K, log2g, y, stream);
}

}  // namespace

bool gemv_supported(int64_t M, int64_t K) {
    if (M < 1 || M > kGemvMaxM) return false;
    if (K % 32 != 0 || K > (int64_t(1) << 30)) return false;
    return gemv_lds_bytes(M, K) <= static_cast<size_t>(max_shared_bytes());
}

awq_status launch_gemv(const half_t* x, const uint32_t* qweight, const half_t* scales,
                       const half_t* zeros, int64_t M, int64_t N, int64_t K, int group_size,
                       half_t* y, hipStream_t stream) {
    const int log2g = group_size == 128 ? 7 : 6;
    switch (M) {
        case 1: return launch_m<1>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 2: return launch_m<2>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 3: return launch_m<3>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 4: return launch_m<4>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 5: return launch_m<5>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 6: return launch_m<6>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 7: return launch_m<7>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 8: return launch_m<8>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        default: return AWQ_ERR_SHAPE;
    }
}

}  // namespace awq
