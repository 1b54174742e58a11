// Prefill GEMM of the W4A16 linear layer on the fp16 matrix cores
// (the batched "GEMM" kernel choice of the rskf.cn AWQ article, §3.3, with
// the INT4 dequantization inside the matmul of §1.3), plus the two variants
// the scale search runs on the same core: an fp16-B product for the
// unquantized reference W . x^T and a fused squared-error epilogue.
//
// Exactness: the dequantized weight (q - z) * s has up to 15 significant bits,
// more than fp16 holds, and rounding it before the MFMA costs up to ~2e-2
// absolute on outputs fed by salient channels. So the B operand is the exact
// integer (q - z) in fp16, and the group's scale is applied in fp32: each
// group's MFMA partial T = A . (Q - Z)^T over its G columns of k accumulates
// in fresh registers, then C += s[n, g] * T (one FMA per element per group).
//
// Tiling (gfx950): a 256-thread block computes a BM x BN tile of y with 4
// wavefronts in a 2 x 2 arrangement; each wave owns (BM/2) x (BN/2) as a grid
// of v_mfma_f32_32x32x16_f16 tiles. K advances in steps of BK = 64 (a group
// is one or two steps):
//  * A (activations, fp16) is copied global -> LDS with 16-byte loads;
//  * B (packed INT4) is read one 16-byte word group (32 codes) per thread,
//    turned into exact fp16 (q - z) once per block and written to LDS in
//    natural k order; the fp16-B variant copies W directly;
//  * LDS rows are padded by 16 bytes so the 16-byte fragment reads of 32
//    consecutive rows spread over all banks;
//  * two LDS stages: the next step's global loads are issued before the
//    current step's MFMAs and stored after them.
// MFMA operand layout (32x32x16 f16): lane l supplies row (l mod 32) of A and
// column (l mod 32) of B, with k-slice 8 * (l / 32) .. +7 of the 16; the
// accumulator element i of lane l is C[8 * (i / 4) + 4 * (l / 32) + i mod 4]
// [l mod 32].
#include "awq_internal.h"

namespace awq {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;          // padded LDS row (halves)
constexpr int kThreads = 256;

__device__ inline half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ inline uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// One packed word (codes k0..k7) -> 8 exact fp16 values (q - z), natural k
// order, as 4 packed pairs. zc_hi = 1024 + z, zc_lo = 64 + z (both exact).
__device__ inline uint4 unpack_word(uint32_t wq, half2_t zc_hi, half2_t zc_lo) {
    const uint32_t w8 = wq >> 8;
    // OR-ing a nibble into an fp16 mantissa gives an exact integer:
    // (1024 + q0, 1024 + q4), (64 + q1, 64 + q5), (1024 + q2, 1024 + q6), (64 + q3, 64 + q7)
    const half2_t a = as_h2((wq & 0x000F000Fu) | 0x64006400u) - zc_hi;
    const half2_t b = as_h2((wq & 0x00F000F0u) | 0x54005400u) - zc_lo;
    const half2_t c = as_h2((w8 & 0x000F000Fu) | 0x64006400u) - zc_hi;
    const half2_t d = as_h2((w8 & 0x00F000F0u) | 0x54005400u) - zc_lo;
    const uint32_t ua = as_u32(a), ub = as_u32(b), uc = as_u32(c), ud = as_u32(d);
    uint4 r;
    r.x = (ua & 0xFFFFu) | (ub << 16);          // (k0, k1)
    r.y = (uc & 0xFFFFu) | (ud << 16);          // (k2, k3)
    r.z = (ua >> 16) | (ub & 0xFFFF0000u);      // (k4, k5)
    r.w = (uc >> 16) | (ud & 0xFFFF0000u);      // (k6, k7)
    return r;
}

template <int BM, int BN, GemmB BMODE, GemmOut OMODE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs args, int tiles_n) {
    constexpr int WTM = BM / 2;                 // wave tile rows
    constexpr int WTN = BN / 2;                 // wave tile cols
    constexpr int TM = WTM / 32;                // 32x32 MFMA tiles per wave (M)
    constexpr int TN = WTN / 32;                // 32x32 MFMA tiles per wave (N)
    constexpr int A_VECS = BM * BK / 8 / kThreads;   // uint4 of A per thread per step
    constexpr bool INT4 = BMODE == GemmB::kInt4;
    constexpr int B_VECS = INT4 ? 1 : BN * BK / 8 / kThreads;
    static_assert(TM >= 1 && TN >= 1 && A_VECS >= 1 && B_VECS >= 1, "tile shape");
    static_assert(!INT4 || BN * 2 == kThreads, "int4 B staging assumes 2 threads per row");

    __shared__ __attribute__((aligned(16))) half_t As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) half_t Bs[2][BN * LDK];

    const int M = static_cast<int>(args.M);
    const int N = static_cast<int>(args.N);
    const int K = static_cast<int>(args.K);
    const int G = args.group_size;
    const int ngroups = K / G;
    const int tile = blockIdx.x;
    const int tm = (tile / tiles_n) * BM;
    const int tn = (tile % tiles_n) * BN;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = (wave >> 1) * WTM;
    const int wn = (wave & 1) * WTN;

    uint4 a_reg[A_VECS];
    uint4 b_reg[B_VECS];
    half2_t b_zhi, b_zlo;
    const int b_row = tid >> 1;          // int4 staging: row within tile
    const int b_half = tid & 1;          // int4 staging: which 32 codes of BK

    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_VECS; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx >> 3, c8 = (idx & 7) * 8;
            const int gm = tm + r;
            a_reg[i] = gm < M ? *reinterpret_cast<const uint4*>(args.a + static_cast<int64_t>(gm) * K + k0 + c8)
                              : make_uint4(0, 0, 0, 0);
        }
        if constexpr (INT4) {
            const int gn = tn + b_row;
            if (gn < N) {
                const int kq = k0 + b_half * 32;
                b_reg[0] = *reinterpret_cast<const uint4*>(args.qweight + static_cast<int64_t>(gn) * (K / 8) + kq / 8);
                const half_t z = args.zeros[static_cast<int64_t>(gn) * ngroups + kq / G];
                const half_t zh = static_cast<half_t>(1024.0f) + z;   // exact
                const half_t zl = static_cast<half_t>(64.0f) + z;     // exact
                b_zhi = half2_t{zh, zh};
                b_zlo = half2_t{zl, zl};
            } else {
                // rows past N: codes 0 with zero 0 -> exact zeros
                b_reg[0] = make_uint4(0, 0, 0, 0);
                b_zhi = half2_t{1024, 1024};
                b_zlo = half2_t{64, 64};
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_VECS; ++i) {
                const int idx = tid + i * kThreads;
                const int r = idx >> 3, c8 = (idx & 7) * 8;
                const int gn = tn + r;
                b_reg[i] = gn < N ? *reinterpret_cast<const uint4*>(args.w + static_cast<int64_t>(gn) * K + k0 + c8)
                                  : make_uint4(0, 0, 0, 0);
            }
        }
    };

    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_VECS; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx >> 3, c8 = (idx & 7) * 8;
            *reinterpret_cast<uint4*>(&As[buf][r * LDK + c8]) = a_reg[i];
        }
        if constexpr (INT4) {
            const uint32_t words[4] = {b_reg[0].x, b_reg[0].y, b_reg[0].z, b_reg[0].w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uint4*>(&Bs[buf][b_row * LDK + b_half * 32 + j * 8]) =
                    unpack_word(words[j], b_zhi, b_zlo);
        } else {
#pragma unroll
            for (int i = 0; i < B_VECS; ++i) {
                const int idx = tid + i * kThreads;
                const int r = idx >> 3, c8 = (idx & 7) * 8;
                *reinterpret_cast<uint4*>(&Bs[buf][r * LDK + c8]) = b_reg[i];
            }
        }
    };

    // scales of this lane's output columns for one group (int4 mode)
    const int lcol = lane & 31;
    auto load_scales = [&](int g, float (&s)[TN]) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = tn + wn + j * 32 + lcol;
            s[j] = n < N ? static_cast<float>(args.scales[static_cast<int64_t>(n) * ngroups + g]) : 0.f;
        }
    };

    float16_t acc[TM][TN];
    float16_t part[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int lrow = lane & 31;
    const int lk = (lane >> 5) * 8;
    const int nk = K / BK;
    float sc[TN];
    if constexpr (INT4) load_scales(0, sc);

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_stage((kt + 1) * BK);
        const int k0 = kt * BK;
        const bool group_start = INT4 && (k0 % G) == 0;
        const bool group_end = INT4 && ((k0 + BK) % G) == 0;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            half8_t af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const half8_t*>(&As[buf][(wm + i * 32 + lrow) * LDK + ks * 16 + lk]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = *reinterpret_cast<const half8_t*>(&Bs[buf][(wn + j * 32 + lrow) * LDK + ks * 16 + lk]);
            if constexpr (INT4) {
                if (group_start && ks == 0) {
                    const float16_t zero = {};
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], zero, 0, 0, 0);
                } else {
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], part[i][j], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
            }
        }
        if constexpr (INT4) {
            if (group_end) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[i][j][e] = fmaf(sc[j], part[i][j][e], acc[i][j][e]);
                if (more) load_scales((k0 + BK) / G, sc);
            }
        }
        if (more) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    const int lrow4 = (lane >> 5) * 4;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = tn + wn + j * 32 + lcol;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = tm + wm + i * 32 + (e >> 2) * 8 + lrow4 + (e & 3);
                if (m < M && n < N) {
                    const int64_t off = static_cast<int64_t>(m) * N + n;
                    const float v = acc[i][j][e];
                    if constexpr (OMODE == GemmOut::kF16) {
                        args.y16[off] = static_cast<half_t>(v);
                    } else if constexpr (OMODE == GemmOut::kF32) {
                        args.y32[off] = v;
                    } else {
                        const float d = v - args.yref[off];
                        sq += d * d;
                    }
                }
            }
        }
    }
    if constexpr (OMODE == GemmOut::kLoss) {
        __shared__ double red[kThreads / kWave];
        double v = static_cast<double>(sq);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
        if (lane == 0) red[wave] = v;
        __syncthreads();
        if (tid == 0) {
            double t = 0.0;
            for (int w = 0; w < kThreads / kWave; ++w) t += red[w];
            args.partials[tile] = t;
        }
    }
}

constexpr int kBM = 128;
constexpr int kBN = 128;

template <GemmB BMODE, GemmOut OMODE>
void launch_cfg(const GemmArgs& args, hipStream_t stream) {
    const int64_t tiles_n = ceil_div(args.N, kBN);
    const int64_t tiles = ceil_div(args.M, kBM) * tiles_n;
    hipLaunchKernelGGL((gemm_kernel<kBM, kBN, BMODE, OMODE>), dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0,
                       stream, args, static_cast<int>(tiles_n));
}

}  // namespace

int64_t gemm_tile_count(int64_t M, int64_t N) { return ceil_div(M, kBM) * ceil_div(N, kBN); }

awq_status launch_gemm(const GemmArgs& args, GemmB b, GemmOut out, hipStream_t stream) {
    if (args.M == 0 || args.N == 0) return AWQ_OK;
    if (b == GemmB::kInt4) {
        switch (out) {
            case GemmOut::kF16: launch_cfg<GemmB::kInt4, GemmOut::kF16>(args, stream); break;
            case GemmOut::kF32: launch_cfg<GemmB::kInt4, GemmOut::kF32>(args, stream); break;
            case GemmOut::kLoss: launch_cfg<GemmB::kInt4, GemmOut::kLoss>(args, stream); break;
        }
    } else {
        switch (out) {
            case GemmOut::kF16: launch_cfg<GemmB::kF16, GemmOut::kF16>(args, stream); break;
            case GemmOut::kF32: launch_cfg<GemmB::kF16, GemmOut::kF32>(args, stream); break;
            case GemmOut::kLoss: return AWQ_ERR_CONFIG;
        }
    }
    return last_launch_status();
}

}  // namespace awq
