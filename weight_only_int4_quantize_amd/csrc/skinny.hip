// Skinny W4A16 GEMM, y[M, N] = x[M, K] . dequant(Wq)^T for 4 < M <= 64 (a
// batch of decode tokens), on gfx950 MFMA.
//
// The operation is the grouped affine dequantization followed by the matrix
// product (xxmr.cn §1.2 inverse map; rskf.cn §1.3 and §3.3, the W4A16 GEMM
// kernel). At these M the product is still bound by streaming the packed
// weights from HBM, but each weight now feeds up to 64 rows, which is MFMA
// work rather than VALU work.
//
// * v_mfma_f32_16x16x32_f16. Its B operand gives every lane 8 consecutive k
//   of one column: exactly one packed word. A lane turns its word into 8
//   exact fp16 values (q - z) with the exponent trick, (w & 0x000F000F) |
//   0x6400_6400 = (1024 + q0, 1024 + q4) and (w & 0x00F000F0) | 0x5400_5400
//   = (64 + q1, 64 + q5), minus (1024 + z) or (64 + z). That leaves the 8
//   values in the order (0,4,1,5,2,6,3,7); x is staged in LDS in the same
//   order, so the pairs line up and nothing is shuffled per weight.
// * The group scale is applied per group: acc += s * (x . (q - z)_group),
//   with the inner sum accumulated exactly by the MFMA in fp32.
// * A block is 4 waves over 128 output columns (two 16-column MFMA tiles per
//   wave) and up to 64 rows; x goes through LDS in double-buffered 256-k
//   chunks, padded so the 16 rows of a fragment read fall in distinct banks.
//   The packed weights stream straight into registers through a ring of
//   groups in flight; they never touch LDS.
// * With a workspace the K range is split across blocks so that narrow
//   layers still fill the GPU. A block parks its fp32 partial tile, bumps a
//   per-column-tile counter, and the last block to arrive adds every split
//   in order and writes y: deterministic, and nobody waits on anybody.
#include <algorithm>

#include "awq_internal.h"

namespace awq {
namespace {

constexpr int kSkThreads = 256;
constexpr int kSkBN = 128;              // output columns per block
constexpr int kSkCK = 256;              // k per staged x chunk
constexpr int kSkLdx = kSkCK + 8;       // LDS row in halves (528 bytes)
constexpr int kSkDepth = 4;             // weight groups in flight per wave
constexpr int kSc1 = 16;                // cache-policy bit sc1 (device scope)
constexpr int kTargetBlocks = 2;        // blocks per CU the split aims for

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}

struct SkConsts {
    uint32_t lo_mask, hi_mask, lo_magic, hi_magic;
};
// In VGPRs: gfx9 VOP3 takes no 32-bit literal, so (w & mask) | magic is one
// v_and_or_b32 only with register operands.
__device__ inline SkConsts sk_consts() {
    SkConsts k{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
    asm volatile("" : "+v"(k.lo_mask), "+v"(k.hi_mask), "+v"(k.lo_magic), "+v"(k.hi_magic));
    return k;
}

// one packed word -> 8 exact fp16 (q - z) in the order (0,4,1,5,2,6,3,7)
__device__ inline half8_t unpack8(uint32_t w, half2_t zc_hi, half2_t zc_lo, const SkConsts& k) {
    const uint32_t w8 = w >> 8;
    const half2_t a = as_h2((w & k.lo_mask) | k.lo_magic) - zc_hi;   // (q0, q4)
    const half2_t b = as_h2((w & k.hi_mask) | k.hi_magic) - zc_lo;   // (q1, q5)
    const half2_t c = as_h2((w8 & k.lo_mask) | k.lo_magic) - zc_hi;  // (q2, q6)
    const half2_t d = as_h2((w8 & k.hi_mask) | k.hi_magic) - zc_lo;  // (q3, q7)
    return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 consecutive x values (natural order) -> the order (0,4,1,5,2,6,3,7)
__device__ inline uint4 permute8(uint4 v) {
    uint4 p;
    p.x = (v.x & 0xFFFFu) | (v.z << 16);
    p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    p.z = (v.y & 0xFFFFu) | (v.w << 16);
    p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return p;
}

// WPL packed words per lane per group: G / 32 (4 for G = 128, 2 for G = 64).
template <int WPL>
struct GroupLoad {
    uint32_t w[2][WPL];     // two column tiles
    uint16_t s[2], z[2];    // raw fp16 bits
};

template <int MB, int WPL>
__global__ __launch_bounds__(kSkThreads, 2) void skinny_kernel(const half_t* __restrict__ x,
                                                              const uint32_t* __restrict__ qweight,
                                                              const half_t* __restrict__ scales,
                                                              const half_t* __restrict__ zeros,
                                                              half_t* __restrict__ y, int M, int N, int K,
                                                              int splits, float* __restrict__ partials,
                                                              int* __restrict__ counters) {
    constexpr int G = WPL * 32;
    constexpr int MP = 16 * MB;                          // padded rows
    constexpr int XPT = MP * (kSkCK / 8) / kSkThreads;   // x pieces per thread per chunk
    __shared__ __attribute__((aligned(16))) half_t xs[2][MP * kSkLdx];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;
    const int lg = lane >> 4;                            // lane group: k sub-block
    const int tiles = (N + kSkBN - 1) / kSkBN;
    const int tile = blockIdx.x % tiles;
    const int split = blockIdx.x / tiles;
    const int ng = K / G;
    const int g0 = static_cast<int>(static_cast<int64_t>(split) * ng / splits);
    const int g1 = static_cast<int>(static_cast<int64_t>(split + 1) * ng / splits);
    const int k0 = g0 * G, k1 = g1 * G;
    const int nchunks = (k1 - k0 + kSkCK - 1) / kSkCK;

    // ---- weights: buffer loads; an offset at or past a buffer's size
    //      reads zero, which is how columns past N and groups past the
    //      block's range are loaded (the size check on the host keeps every
    //      such offset below 2^32) ----
    const int n_base = tile * kSkBN + wave * 32;
    const uint32_t w_bytes = static_cast<uint32_t>(static_cast<int64_t>(N) * (K / 2));
    const uint32_t sz_bytes = static_cast<uint32_t>(static_cast<int64_t>(N) * ng * 2);
    const auto rw = rsrc(qweight, w_bytes);
    const auto rs = rsrc(scales, sz_bytes);
    const auto rz = rsrc(zeros, sz_bytes);
    uint32_t w_off[2], sz_off[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int n = n_base + 16 * t + col;
        const bool ok = n < N;
        w_off[t] = ok ? static_cast<uint32_t>(n) * static_cast<uint32_t>(K / 2) + lg * WPL * 4 : w_bytes;
        sz_off[t] = ok ? static_cast<uint32_t>(n) * static_cast<uint32_t>(ng) * 2 : sz_bytes;
    }
    auto load_group = [&](GroupLoad<WPL>& gl, int g) {
        const bool ok = g < g1;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t wo = ok ? w_off[t] + static_cast<uint32_t>(g) * (G / 2) : w_bytes;
            const uint32_t so = ok ? sz_off[t] + static_cast<uint32_t>(g) * 2 : sz_bytes;
            if constexpr (WPL == 4) {
                const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 0, 0));
#pragma unroll
                for (int j = 0; j < 4; ++j) gl.w[t][j] = v[j];
            } else {
                const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rw, wo, 0, 0));
#pragma unroll
                for (int j = 0; j < 2; ++j) gl.w[t][j] = v[j];
            }
            gl.s[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
            gl.z[t] = __builtin_amdgcn_raw_buffer_load_b16(rz, so, 0, 0);
        }
    };

    // ---- x chunks: rows past M are zeros ----
    uint4 xr[XPT];
    auto load_x = [&](int c) {
        const int kc0 = k0 + c * kSkCK;
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int p = tid + i * kSkThreads;
            const int r = p / (kSkCK / 8), c8 = p % (kSkCK / 8);
            const int k = kc0 + c8 * 8;
            if (r < M && k < k1)
                xr[i] = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(r) * K + k);
            else
                xr[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int p = tid + i * kSkThreads;
            const int r = p / (kSkCK / 8), c8 = p % (kSkCK / 8);
            *reinterpret_cast<uint4*>(&xs[buf][r * kSkLdx + c8 * 8]) = permute8(xr[i]);
        }
    };

    float4_t acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[mb][t] = float4_t{0.f, 0.f, 0.f, 0.f};
    const SkConsts uk = sk_consts();

    // Ring slot d holds group gb + d. x chunk c lives in LDS buffer c & 1:
    // it is loaded into registers while chunk c - 1 is consumed and written
    // to LDS on entering chunk c (that buffer was last read in chunk c - 2,
    // which every wave left before the barrier on entering chunk c - 1).
    constexpr int CG = kSkCK / G;                        // groups per chunk
    GroupLoad<WPL> ring[kSkDepth];
#pragma unroll
    for (int d = 0; d < kSkDepth; ++d) load_group(ring[d], g0 + d);
    load_x(0);
    store_x(0);
    if (nchunks > 1) load_x(1);
    __syncthreads();

    for (int gb = g0; gb < g1; gb += kSkDepth) {
#pragma unroll
        for (int d = 0; d < kSkDepth; ++d) {
            const int gg = gb + d;
            if (gg < g1) {
                const int gi = gg - g0;
                const int c = gi / CG;
                if (gi % CG == 0 && c > 0) {
                    store_x(c & 1);
                    __syncthreads();
                    if (c + 1 < nchunks) load_x(c + 1);
                }
                GroupLoad<WPL>& gl = ring[d];
                half8_t bf[2][WPL];
                float s[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const half_t z = __builtin_bit_cast(half_t, gl.z[t]);
                    const half_t zh = static_cast<half_t>(1024.0f) + z;   // exact
                    const half_t zl = static_cast<half_t>(64.0f) + z;     // exact
#pragma unroll
                    for (int j = 0; j < WPL; ++j) bf[t][j] = unpack8(gl.w[t][j], half2_t{zh, zh}, half2_t{zl, zl}, uk);
                    s[t] = static_cast<float>(__builtin_bit_cast(half_t, gl.s[t]));
                }
                load_group(gl, gg + kSkDepth);                     // refill the slot
                const half_t* xb = &xs[c & 1][col * kSkLdx + (gi % CG) * G + 8 * lg * WPL];
                float4_t part[MB][2];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int t = 0; t < 2; ++t) part[mb][t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < WPL; ++j) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const half8_t a = *reinterpret_cast<const half8_t*>(xb + 16 * mb * kSkLdx + 8 * j);
#pragma unroll
                        for (int t = 0; t < 2; ++t)
                            part[mb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[t][j], part[mb][t], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[mb][t][e] += s[t] * part[mb][t][e];
            }
        }
    }

    // ---- epilogue: lane holds rows 16 mb + 4 lg + e of column n ----
    auto emit = [&](const float4_t (&v)[MB][2]) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int n = n_base + 16 * t + col;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 16 * mb + 4 * lg + e;
                    if (m < M && n < N) y[static_cast<int64_t>(m) * N + n] = static_cast<half_t>(v[mb][t][e]);
                }
            }
    };
    if (splits == 1) {
        emit(acc);
        return;
    }
    // partial tile of this (tile, split): [MB * 2 float4 chunks][256 threads]
    constexpr uint32_t kPartBytes = MB * 2 * kSkThreads * 16;
    auto part_rsrc = [&](int sp) {
        return rsrc(reinterpret_cast<char*>(partials) +
                        (static_cast<int64_t>(tile) * splits + sp) * static_cast<int64_t>(kPartBytes),
                    kPartBytes);
    };
    {
        const auto pr = part_rsrc(split);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[mb][t]), pr, tid * 16,
                                                       (mb * 2 + t) * kSkThreads * 16, kSc1);
    }
    // sc1 stores and loads bypass the per-XCD L2s; every store is complete
    // before the counter moves, and the loads are issued after it is read
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(&counters[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 splits - 1;
    __syncthreads();
    if (!s_last) return;
    float4_t sum[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 2; ++t) sum[mb][t] = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < splits; ++sp) {
        const auto pr = part_rsrc(sp);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                sum[mb][t] += __builtin_bit_cast(
                    float4_t, __builtin_amdgcn_raw_buffer_load_b128(pr, tid * 16, (mb * 2 + t) * kSkThreads * 16, kSc1));
    }
    emit(sum);
    if (tid == 0) __hip_atomic_store(&counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int64_t sk_tiles(int64_t N) { return (N + kSkBN - 1) / kSkBN; }

int sk_mb(int64_t M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

// partial tiles a workspace holds: splits x column tiles never exceed it
int64_t sk_max_parts() { return 3 * static_cast<int64_t>(cu_count()); }

// K splits when a workspace is given: enough blocks for kTargetBlocks per
// CU, each split keeping at least two groups.
int sk_splits(int64_t N, int64_t K, int group_size) {
    const int64_t tiles = sk_tiles(N);
    if (tiles > split_counter_slots()) return 1;
    const int64_t ng = K / group_size;
    int64_t s = (kTargetBlocks * cu_count() + tiles / 2) / tiles;
    s = std::min<int64_t>(s, ng / 2);
    while (s > 1 && s * tiles > sk_max_parts()) --s;
    return static_cast<int>(std::max<int64_t>(1, s));
}

size_t sk_partial_bytes(int64_t M) { return static_cast<size_t>(sk_mb(M)) * 2 * kSkThreads * 16; }

template <int MB, int WPL>
void launch_cfg(const half_t* x, const uint32_t* qweight, const half_t* scales, const half_t* zeros, int M, int N,
                int K, half_t* y, int splits, float* partials, int* counters, hipStream_t stream) {
    const int64_t blocks = sk_tiles(N) * splits;
    hipLaunchKernelGGL((skinny_kernel<MB, WPL>), dim3(static_cast<unsigned>(blocks)), dim3(kSkThreads), 0, stream, x,
                       qweight, scales, zeros, y, M, N, K, splits, partials, counters);
}

template <int WPL>
void launch_wpl(const half_t* x, const uint32_t* qweight, const half_t* scales, const half_t* zeros, int M, int N,
                int K, half_t* y, int splits, float* partials, int* counters, hipStream_t stream) {
    switch (sk_mb(M)) {
        case 1: launch_cfg<1, WPL>(x, qweight, scales, zeros, M, N, K, y, splits, partials, counters, stream); break;
        case 2: launch_cfg<2, WPL>(x, qweight, scales, zeros, M, N, K, y, splits, partials, counters, stream); break;
        default: launch_cfg<4, WPL>(x, qweight, scales, zeros, M, N, K, y, splits, partials, counters, stream); break;
    }
}

}  // namespace

bool skinny_supported(int64_t M, int64_t N, int64_t K) {
    // buffer offsets are 32-bit: the packed matrix plus one row of slack
    // (the largest offset a zero-reading lane forms) must stay below 4 GiB
    return M >= 1 && M <= kSkinnyMaxM && N >= 1 && (N + 1) * (K / 2) + 64 < (int64_t{1} << 32);
}

size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!skinny_supported(M, N, K)) return 0;
    return split_counter_bytes() + static_cast<size_t>(sk_max_parts()) * sk_partial_bytes(M);
}

awq_status launch_skinny(const half_t* x, const uint32_t* qweight, const half_t* scales, const half_t* zeros,
                         int64_t M, int64_t N, int64_t K, int group_size, half_t* y, void* workspace,
                         hipStream_t stream) {
    if (M == 0 || N == 0) return AWQ_OK;
    if (!skinny_supported(M, N, K)) return AWQ_ERR_SHAPE;
    int splits = 1;
    float* partials = nullptr;
    int* counters = nullptr;
    if (workspace != nullptr) {
        splits = sk_splits(N, K, group_size);
        if (splits > 1) {
            counters = static_cast<int*>(workspace);
            partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + split_counter_bytes());
        }
    }
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    if (group_size == 128)
        launch_wpl<4>(x, qweight, scales, zeros, m, n, k, y, splits, partials, counters, stream);
    else
        launch_wpl<2>(x, qweight, scales, zeros, m, n, k, y, splits, partials, counters, stream);
    return last_launch_status();
}

}  // namespace awq
