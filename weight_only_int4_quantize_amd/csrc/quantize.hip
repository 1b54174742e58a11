// Group-wise INT4 quantization (range -> scale/zero -> codes -> pack).
//
// The map is the one of "模型量化:GGUF/AWQ/GPTQ部署方案" §1.2 (q = clamp(round(x /
// scale) + zero_point, 0, 15), scale from the weight range) with one scale and
// zero-point per group of G consecutive input channels (§1.4; aissn.com
// "量化粒度"). Asymmetric by default (aissn.com "对称/非对称量化": zero-point
// != 0, the group's own [min, max]); the symmetric form of that section
// (zero-point 0) maps the group's largest magnitude to +-7, s = max|w| / 7,
// q = clamp(round(w / s), -8, 7), and stores q + 8 with zero-point 8, so the
// same dequantization (q - z) * s serves both. The W8A16 form (aissn.com
// "INT8 实战": 8-bit weights, fp16 activations) is the same map with 255
// levels (symmetric at +-127, stored as q + 128), four codes per word.
//
// Layout: one thread per 8 consecutive k of one row (one packed INT4 word, or
// two W8 words), read as one 16-byte load. The G/8 threads of a group are adjacent lanes of one
// wavefront, so a wave streams 64 * 16 B = 1 KB of contiguous weights and the
// group min/max is a 3- or 4-step butterfly over lanes. Every arithmetic step
// is IEEE fp32 (correctly rounded divide, round-half-to-even rint) so the
// codes, scales and zeros are bit-identical to a plain fp32 evaluation.
#include <cmath>

#include "awq_internal.h"

namespace awq {
namespace {

#pragma clang fp contract(off)

constexpr float kTieBand = 1e-3f;   // |frac(v / s) - 1/2| below which the exact divide decides

// Clip step (xxmr.cn §1.5: cut the extreme p of the values at both ends
// before the scale is taken). The bounds are the p and 1 - p quantiles of the
// group, interpolated between order statistics x(0) <= ... <= x(G-1):
//   lo = x(i) + f * (x(i+1) - x(i)),  hi = x(G-1-i) - f * (x(G-1-i) - x(G-2-i))
// with (i, f) = (floor(h), h - floor(h)), h = (G - 1) * p, taken on the host.
// The four order statistics are found by selection from both ends (see the
// kernel), in O((i + 2) log G) group reductions rather than a sort.
struct Clip {
    int i = 0;          // lower order-statistic position
    float f = 0.f;      // interpolation fraction
};

// BITS = 4 (INT4: 8 codes per word) or 8 (W8A16: 4 codes per word, the
// same map with 255 levels; symmetric at +-127 stored as code + 128).
template <int G, bool SYM, bool CLIP, int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const half_t* __restrict__ w,
                                                       const float* __restrict__ channel_scale,
                                                       int64_t n_words, int64_t words_per_row,
                                                       uint32_t* __restrict__ qweight,
                                                       half_t* __restrict__ scales,
                                                       half_t* __restrict__ zeros, Clip clip) {
    constexpr int kLanes = G / 8;  // threads per group: 4 .. 64 (G = 32 .. 512)
    constexpr float kQ = static_cast<float>((1 << BITS) - 1);            // 15 or 255
    constexpr float kSymQ = static_cast<float>((1 << (BITS - 1)) - 1);   // 7 or 127
    constexpr float kSymZero = static_cast<float>(1 << (BITS - 1));      // 8 or 128
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    // n_words is a multiple of kLanes and kLanes divides 64, so a group's
    // lanes are either all in range or all out of range.
    if (t >= n_words) return;

    const uint4 raw = reinterpret_cast<const uint4*>(w)[t];
    const uint32_t parts[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(parts[i] & 0xFFFFu)));
        v[2 * i + 1] = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(parts[i] >> 16)));
    }
    if (channel_scale != nullptr) {
        const int64_t k0 = (t % words_per_row) * 8;
        const float4 c0 = *reinterpret_cast<const float4*>(channel_scale + k0);
        const float4 c1 = *reinterpret_cast<const float4*>(channel_scale + k0 + 4);
        v[0] = v[0] * c0.x; v[1] = v[1] * c0.y; v[2] = v[2] * c0.z; v[3] = v[3] * c0.w;
        v[4] = v[4] * c1.x; v[5] = v[5] * c1.y; v[6] = v[6] * c1.z; v[7] = v[7] * c1.w;
    }

    float lo, hi;
    if constexpr (CLIP) {
        // Walk the distinct values upwards from the bottom and downwards from
        // the top at once: each round takes the next value on each side
        // (group min / max over what is left) and its multiplicity (group
        // count of equal values), so after round r the ranks covered on each
        // side are known. Every round covers at least one rank per side, so
        // i + 2 rounds reach ranks i and i + 1 from both ends; the trip count
        // is fixed by the launch, the same for every wave.
        float cur_lo = -__builtin_inff(), cur_hi = __builtin_inff();
        int below = 0, above = 0;            // ranks covered from the bottom / top
        float c0 = 0.f, c1 = 0.f, c2 = 0.f, c3 = 0.f;
        const int r0 = clip.i, r1 = clip.i + 1;
        for (int it = 0; it < clip.i + 2; ++it) {
            float nl = __builtin_inff(), nh = -__builtin_inff();
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                nl = v[j] > cur_lo ? fminf(nl, v[j]) : nl;
                nh = v[j] < cur_hi ? fmaxf(nh, v[j]) : nh;
            }
#pragma unroll
            for (int o = 1; o < kLanes; o <<= 1) {
                nl = fminf(nl, __shfl_xor(nl, o, kLanes));
                nh = fmaxf(nh, __shfl_xor(nh, o, kLanes));
            }
            int cnt = 0;                     // low count | high count << 16
#pragma unroll
            for (int j = 0; j < 8; ++j) cnt += (v[j] == nl ? 1 : 0) + (v[j] == nh ? 0x10000 : 0);
#pragma unroll
            for (int o = 1; o < kLanes; o <<= 1) cnt += __shfl_xor(cnt, o, kLanes);
            const int cl = cnt & 0xFFFF, ch = cnt >> 16;
            if (below <= r0 && r0 < below + cl) c0 = nl;
            if (below <= r1 && r1 < below + cl) c1 = nl;
            if (above <= r0 && r0 < above + ch) c2 = nh;
            if (above <= r1 && r1 < above + ch) c3 = nh;
            below += cl;
            above += ch;
            cur_lo = nl;
            cur_hi = nh;
        }
        lo = c0 + clip.f * (c1 - c0);
        hi = c2 - clip.f * (c2 - c3);
    } else {
        lo = v[0];
        hi = v[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            lo = fminf(lo, v[i]);
            hi = fmaxf(hi, v[i]);
        }
#pragma unroll
        for (int o = 1; o < kLanes; o <<= 1) {
            lo = fminf(lo, __shfl_xor(lo, o, kLanes));
            hi = fmaxf(hi, __shfl_xor(hi, o, kLanes));
        }
    }

    float s32, z;
    if constexpr (SYM) {
        const float a = fmaxf(fmaxf(-lo, hi), kRangeFloor);   // max |w| (lo <= hi)
        s32 = a / kSymQ;                                      // IEEE divide
    } else {
        const float range = fmaxf(hi - lo, kRangeFloor);
        s32 = range / kQ;                                     // IEEE divide
    }
    const half_t s16 = static_cast<half_t>(s32);              // round-to-nearest-even
    const float sf = static_cast<float>(s16);
    if constexpr (SYM) {
        z = kSymZero;
    } else {
        const int zi = static_cast<int>(fminf(fmaxf(rintf(-lo / sf), 0.0f), kQ));
        z = static_cast<float>(zi);
    }

    // rint(v / s) with the correctly rounded quotient, taken through the
    // product v * (1 / s): its error is below 1e-4 for |v / s| <= 256 (the
    // reciprocal and the product each round once), so away from the
    // half-way points it rounds to the same integer. Within kTieBand of a
    // half-way point the exact IEEE divide decides.
    const float rinv = 1.0f / sf;
    uint32_t code[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float r = v[j] * rinv;
        float q = rintf(r);
        if (fabsf(fabsf(r - q) - 0.5f) < kTieBand) q = rintf(v[j] / sf);
        code[j] = static_cast<uint32_t>(fminf(fmaxf(q + z, 0.0f), kQ));
    }
    if constexpr (BITS == 4) {
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) packed |= code[j] << (4 * j);
        qweight[t] = packed;
    } else {
        const uint2 packed = make_uint2(code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24),
                                        code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24));
        reinterpret_cast<uint2*>(qweight)[t] = packed;
    }
    if ((t & (kLanes - 1)) == 0) {
        const int64_t gi = t / kLanes;
        scales[gi] = s16;
        zeros[gi] = static_cast<half_t>(z);
    }
}

template <int G, bool SYM, bool CLIP, int BITS>
void launch_g(const half_t* w, const float* channel_scale, int64_t n_words, int64_t words_per_row,
              uint32_t* qweight, half_t* scales, half_t* zeros, Clip clip, hipStream_t stream) {
    const int threads = 256;
    const int64_t blocks = ceil_div(n_words, threads);
    hipLaunchKernelGGL((quantize_kernel<G, SYM, CLIP, BITS>), dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                       stream, w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip);
}

template <bool SYM, bool CLIP, int BITS>
void launch_sym(const half_t* w, const float* channel_scale, int64_t n_words, int64_t words_per_row,
                int group_size, uint32_t* qweight, half_t* scales, half_t* zeros, Clip clip,
                hipStream_t stream) {
    switch (group_size) {
        case 32:
            launch_g<32, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip, stream);
            break;
        case 64:
            launch_g<64, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip, stream);
            break;
        case 128:
            launch_g<128, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip, stream);
            break;
        case 256:
            launch_g<256, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip, stream);
            break;
        default:
            launch_g<512, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip, stream);
            break;
    }
}

template <int BITS>
void launch_bits(const half_t* w, const float* channel_scale, int64_t n_words, int64_t words_per_row,
                 int group_size, bool symmetric, bool c, uint32_t* qweight, half_t* scales, half_t* zeros,
                 Clip clip, hipStream_t stream) {
    if (symmetric && c)
        launch_sym<true, true, BITS>(w, channel_scale, n_words, words_per_row, group_size, qweight, scales, zeros,
                                     clip, stream);
    else if (symmetric)
        launch_sym<true, false, BITS>(w, channel_scale, n_words, words_per_row, group_size, qweight, scales, zeros,
                                      clip, stream);
    else if (c)
        launch_sym<false, true, BITS>(w, channel_scale, n_words, words_per_row, group_size, qweight, scales, zeros,
                                      clip, stream);
    else
        launch_sym<false, false, BITS>(w, channel_scale, n_words, words_per_row, group_size, qweight, scales,
                                       zeros, clip, stream);
}

}  // namespace

bool clip_fraction_ok(double p) { return p >= 0.0 && p < 0.25; }

awq_status launch_quantize(const half_t* w, const float* channel_scale, int64_t N, int64_t K,
                           int group_size, bool symmetric, double clip_fraction, uint32_t* qweight,
                           half_t* scales, half_t* zeros, hipStream_t stream, int bits) {
    const int64_t words_per_row = K / 8;
    const int64_t n_words = N * words_per_row;
    if (n_words == 0) return AWQ_OK;
    if (!clip_fraction_ok(clip_fraction)) return AWQ_ERR_CONFIG;
    Clip clip;
    const double h = (group_size - 1) * clip_fraction;
    clip.i = static_cast<int>(std::floor(h));
    clip.f = static_cast<float>(h - clip.i);
    const bool c = clip_fraction > 0.0;
    if (bits == 8)
        launch_bits<8>(w, channel_scale, n_words, words_per_row, group_size, symmetric, c, qweight, scales, zeros,
                       clip, stream);
    else
        launch_bits<4>(w, channel_scale, n_words, words_per_row, group_size, symmetric, c, qweight, scales, zeros,
                       clip, stream);
    return last_launch_status();
}

}  // namespace awq
