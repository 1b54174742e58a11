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
// group min/max is a 2- to 6-step butterfly over lanes (group_reduce). Codes, scales and
// zeros are bit-identical to a plain IEEE fp32 evaluation (correctly rounded
// divides, round-half-to-even rint), reached without the divide sequence
// where that is provably the same (div_const, rint_plus).
#include <cmath>

#include "awq_internal.h"

namespace awq {
namespace {

#pragma clang fp contract(off)

constexpr float kTieBand = 1e-3f;   // |frac(v / s) - 1/2| below which the exact divide decides
constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23: in its binade the last bits are the integer part

// a / d as the IEEE quotient for the constant divisors d = 7, 15, 127 and
// 255: q0 = a * RN(1/d) is off by at most one unit; the fma gives its
// residual a - q0 d exactly, and one more fma rounds q0 + residual / d. For
// these four d this equals the correctly rounded a / d at every fp32
// significand (checked exhaustively in tests/test_quantize_arith_host.py; a
// scale by 2^k scales every step exactly), for any normal a.
__device__ __forceinline__ float div_const(float a, float d) {
    const float y = 1.0f / d;   // folded at compile time
    const float q0 = a * y;
    return fmaf(fmaf(-q0, d, a), y, q0);
}

// Value of the lane that DPP control CTRL pairs with this one (row_mask and
// bank_mask full; every pairing used stays inside a 16-lane row).
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Reduction over the LANES adjacent lanes of a group, every lane getting the
// result. Up to 16 lanes the pairings are DPP row moves: swap neighbours
// (quad_perm 1,0,3,2), swap pairs (2,3,0,1), then mirror each half-row and
// each row; after the quad steps every lane holds its quad's value, and each
// mirror pairs every lane with one in the other quad / half. Wider groups
// add lane xors 16 and 32 through LDS.
template <int LANES, class T, class Op>
__device__ __forceinline__ T group_reduce(T x, Op op) {
    if constexpr (LANES >= 2) x = op(x, dpp_partner<0xB1>(x));
    if constexpr (LANES >= 4) x = op(x, dpp_partner<0x4E>(x));
    if constexpr (LANES >= 8) x = op(x, dpp_partner<0x141>(x));
    if constexpr (LANES >= 16) x = op(x, dpp_partner<0x140>(x));
    if constexpr (LANES >= 32) x = op(x, __shfl_xor(x, 16, LANES));
    if constexpr (LANES >= 64) x = op(x, __shfl_xor(x, 32, LANES));
    return x;
}

// base + rint(x / s) with the correctly rounded quotient, base an integer in
// [kMagic, kMagic + 255]. t = fma(x, 1/s, base) rounds the exact x * (1/s)
// + base once, onto the integers of kMagic's binade; 1/s comes from the
// hardware reciprocal (error within one unit, so x * (1/s) is within 2^-23
// |x / s| of x / s). For |x / s| <= 1024 that, with the quotient's own
// rounding, is under 2e-4, so unless x * (1/s) lies within kTieBand of a
// half-way point (its distance from t - base is exact through the second
// fma) both round to the same integer; near one the IEEE divide decides.
// Beyond 1024 both clamp to the same end code: read as signed integers, the
// bits of t keep the order of every t >= 0 and put every t < 0 below code 0.
__device__ __forceinline__ float rint_plus(float x, float s, float rinv, float base) {
    const float t = fmaf(x, rinv, base);
    if (fabsf(fmaf(x, rinv, -(t - base))) > 0.5f - kTieBand) return base + rintf(x / s);
    return t;
}

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
                                                       half_t* __restrict__ zeros, Clip clip,
                                                       int64_t tiled_nk) {
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
            // lane xors through LDS here: in these dependent rounds the DPP
            // moves' wait states cost more (69.9 against 70.4 us at p = 1%)
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
        lo = group_reduce<kLanes>(lo, [](float a, float b) { return fminf(a, b); });
        hi = group_reduce<kLanes>(hi, [](float a, float b) { return fmaxf(a, b); });
    }

    // s = range / kQ (or max|w| / kSymQ) as the IEEE quotient, taken as the
    // product by the rounded reciprocal of the constant plus one fma
    // correction of its residual (div_const).
    float s32;
    if constexpr (SYM) {
        s32 = div_const(fmaxf(fmaxf(-lo, hi), kRangeFloor), kSymQ);   // max |w| (lo <= hi)
    } else {
        s32 = div_const(fmaxf(hi - lo, kRangeFloor), kQ);
    }
    // the fp32 quotient is rounded to fp16 on its own (an empty asm keeps the
    // last fma and the conversion from merging into one fp16-rounding fma)
    asm volatile("" : "+v"(s32));
    const half_t s16 = static_cast<half_t>(s32);              // round-to-nearest-even
    const float sf = static_cast<float>(s16);
    const float rinv = __builtin_amdgcn_rcpf(sf);

    // base = kMagic + z: every code is then one fma, t = v * (1 / s) + base,
    // whose bits are bits(kMagic) + rint(v / s) + z (see rint_plus)
    float base;
    if constexpr (SYM) {
        base = kMagic + kSymZero;
    } else {
        const float tz = rint_plus(-lo, sf, rinv, kMagic);
        base = fminf(fmaxf(tz, kMagic), kMagic + kQ);          // z = clamp(rint(-lo / s), 0, kQ)
    }
    const float z = base - kMagic;

    float tq[8];
    bool near_tie = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        tq[j] = fmaf(v[j], rinv, base);
        near_tie |= fabsf(fmaf(v[j], rinv, -(tq[j] - base))) > 0.5f - kTieBand;
    }
    if (near_tie) {
#pragma unroll
        for (int j = 0; j < 8; ++j) tq[j] = rint_plus(v[j], sf, rinv, base);
    }
    // clamp(rint(v / s) + z, 0, kQ) + bits(kMagic), on the bits as signed
    // integers (order-preserving for the values that can occur, and any
    // value below kMagic clamps to code 0)
    constexpr int kLoBits = 0x4B400000;   // bits of kMagic
    int32_t code[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int32_t b = __builtin_bit_cast(int32_t, tq[j]);
        code[j] = min(max(b, kLoBits), kLoBits + static_cast<int32_t>(kQ));
    }
    // each code still carries bits(kMagic); the shifted sums drop it at once
    // (arithmetic mod 2^32)
    if constexpr (BITS == 4) {
        uint32_t packed = 0u - static_cast<uint32_t>(kLoBits) * 0x11111111u;
#pragma unroll
        for (int j = 0; j < 8; ++j) packed += static_cast<uint32_t>(code[j]) << (4 * j);
        if (tiled_nk == 0) {
            qweight[t] = packed;
        } else {
            // tiled order of the searches' loss GEMM: word c of row n goes to
            // lane (c / 4 % 2) * 32 + n % 32 of the 1 KB piece of 32-row group
            // n / 32 and 64-k step c / 8, at word c % 4 of the lane's 16 bytes
            const int64_t n = t / words_per_row, c = t - n * words_per_row;
            qweight[(((n >> 5) * tiled_nk + (c >> 3)) * 64 + ((c >> 2) & 1) * 32 + (n & 31)) * 4 + (c & 3)] = packed;
        }
    } else {
        uint32_t lo_w = 0u - static_cast<uint32_t>(kLoBits) * 0x01010101u, hi_w = lo_w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo_w += static_cast<uint32_t>(code[j]) << (8 * j);
            hi_w += static_cast<uint32_t>(code[4 + j]) << (8 * j);
        }
        const uint2 packed = make_uint2(lo_w, hi_w);
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
              uint32_t* qweight, half_t* scales, half_t* zeros, Clip clip, hipStream_t stream,
              int64_t tiled_nk) {
    const int threads = 256;
    const int64_t blocks = ceil_div(n_words, threads);
    hipLaunchKernelGGL((quantize_kernel<G, SYM, CLIP, BITS>), dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                       stream, w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip, tiled_nk);
}

template <bool SYM, bool CLIP, int BITS>
void launch_sym(const half_t* w, const float* channel_scale, int64_t n_words, int64_t words_per_row,
                int group_size, uint32_t* qweight, half_t* scales, half_t* zeros, Clip clip,
                hipStream_t stream, int64_t tiled_nk) {
    switch (group_size) {
        case 32:
            launch_g<32, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip,
                                      stream, tiled_nk);
            break;
        case 64:
            launch_g<64, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip,
                                      stream, tiled_nk);
            break;
        case 128:
            launch_g<128, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip,
                                      stream, tiled_nk);
            break;
        case 256:
            launch_g<256, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip,
                                      stream, tiled_nk);
            break;
        default:
            launch_g<512, SYM, CLIP, BITS>(w, channel_scale, n_words, words_per_row, qweight, scales, zeros, clip,
                                      stream, tiled_nk);
            break;
    }
}

template <int BITS>
void launch_bits(const half_t* w, const float* channel_scale, int64_t n_words, int64_t words_per_row,
                 int group_size, bool symmetric, bool c, uint32_t* qweight, half_t* scales, half_t* zeros,
                 Clip clip, hipStream_t stream, int64_t tiled_nk) {
    if (symmetric && c)
        launch_sym<true, true, BITS>(w, channel_scale, n_words, words_per_row, group_size, qweight, scales, zeros,
                                     clip, stream, tiled_nk);
    else if (symmetric)
        launch_sym<true, false, BITS>(w, channel_scale, n_words, words_per_row, group_size, qweight, scales, zeros,
                                      clip, stream, tiled_nk);
    else if (c)
        launch_sym<false, true, BITS>(w, channel_scale, n_words, words_per_row, group_size, qweight, scales, zeros,
                                      clip, stream, tiled_nk);
    else
        launch_sym<false, false, BITS>(w, channel_scale, n_words, words_per_row, group_size, qweight, scales,
                                       zeros, clip, stream, tiled_nk);
}

}  // namespace

bool clip_fraction_ok(double p) { return p >= 0.0 && p < 0.25; }

awq_status launch_quantize(const half_t* w, const float* channel_scale, int64_t N, int64_t K,
                           int group_size, bool symmetric, double clip_fraction, uint32_t* qweight,
                           half_t* scales, half_t* zeros, hipStream_t stream, int bits, bool tiled) {
    const int64_t words_per_row = K / 8;
    const int64_t n_words = N * words_per_row;
    if (n_words == 0) return AWQ_OK;
    if (!clip_fraction_ok(clip_fraction)) return AWQ_ERR_CONFIG;
    Clip clip;
    const double h = (group_size - 1) * clip_fraction;
    clip.i = static_cast<int>(std::floor(h));
    clip.f = static_cast<float>(h - clip.i);
    const bool c = clip_fraction > 0.0;
    // the tiled order is for INT4 words whose rows are whole 64-k steps
    if (tiled && (bits != 4 || K % 64 != 0)) return AWQ_ERR_CONFIG;
    const int64_t tiled_nk = tiled ? K / 64 : 0;
    if (bits == 8)
        launch_bits<8>(w, channel_scale, n_words, words_per_row, group_size, symmetric, c, qweight, scales, zeros,
                       clip, stream, tiled_nk);
    else
        launch_bits<4>(w, channel_scale, n_words, words_per_row, group_size, symmetric, c, qweight, scales, zeros,
                       clip, stream, tiled_nk);
    return last_launch_status();
}

}  // namespace awq
