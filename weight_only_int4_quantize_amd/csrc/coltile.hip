// Column-tile W4A16 kernel for small decode batches, y[M, N] = x[M, K] .
// dequant(Wq)^T with 2 <= M <= 32 (the W4A16 linear layer of the rskf.cn AWQ
// article, §1.3 / §3.3, at a handful of tokens; the dequantization map of
// xxmr.cn §1.2).
//
// At these M the layer is bound by streaming the packed weights from HBM,
// and every weight feeds M outputs, which the fp16 matrix cores take: one
// v_mfma_f32_16x16x32_f16 multiplies 16 rows of x by 16 columns of W over
// 32 k. The layout puts the whole K range of CT 16-column tiles in one
// thread block, so no partial sums leave the block:
//  * a block of NW waves owns 16 CT output columns and all of K; wave w
//    takes the groups [w ng / NW, (w + 1) ng / NW) and keeps a 16 x 16
//    accumulator per 16 rows of x and tile; every x operand a wave reads
//    feeds the CT tiles' MFMAs; the waves' accumulators are added through
//    LDS in a fixed order at the end (deterministic);
//  * within a group a lane of k-quarter q (lane / 16) takes the G / 4
//    consecutive k of words [q WPL, (q + 1) WPL) of its column, WPL = G / 32
//    packed words, so its weights are one contiguous 4 WPL-byte load and its
//    x one contiguous 16 WPL-byte load per row. The MFMA's k order is free
//    as long as both operands follow it: step j of the group pairs word
//    q WPL + j of every column with the same 8 k of x;
//  * x is read straight from global memory (L2) into the A operand, no LDS:
//    each 16-column tile uses each x value once, so staging would not save a
//    byte. x costs M / 4 times the weight bytes, from L2 rather than HBM;
//  * weights and x stream through a ring of DEPTH groups in flight per wave;
//    the loads are issued unconditionally at fixed places (past-the-end
//    offsets read zero without touching memory), so the compiler's wait
//    counts follow the ring;
//  * the group's scale and zero-point come from LDS, staged once per block
//    with coalesced loads; the scale is applied per group in fp32,
//    acc += s * (x . (q - z)), the inner sum exact in the MFMA.
// Nibble unpack: (w & 0x000F000F) | 0x6400_6400 = (1024 + q0, 1024 + q4) and
// (w & 0x00F000F0) | 0x5400_5400 = (64 + q1, 64 + q5), the same on w >> 8
// for (q2, q6) and (q3, q7); minus (1024 + z) or (64 + z) this is the exact
// fp16 (q - z) in the order (0,4,1,5,2,6,3,7), and x is permuted to match.
#include <algorithm>

#include "awq_internal.h"

namespace awq {
namespace {

constexpr int kCtCols = 16;      // columns of one MFMA tile
constexpr int kCtSZ = 4;          // (scale, zero) pairs per thread loaded ahead of the ring
// LDS: the (scale, zero) pairs [16 ct][ng | 1] words, then (16-byte aligned)
// the waves' x buffers, later reused for the waves' sums
__host__ __device__ inline int ct_x_offset(int ng, int ct) { return (kCtCols * ct * (ng | 1) + 3) & ~3; }

__device__ inline half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}

struct CtConsts {
    uint32_t lo_mask, hi_mask, lo_magic, hi_magic;
};
// In VGPRs: gfx9 VOP3 takes no 32-bit literal, so (w & mask) | magic is one
// v_and_or_b32 only with register operands.
__device__ inline CtConsts ct_consts() {
    CtConsts k{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
    asm volatile("" : "+v"(k.lo_mask), "+v"(k.hi_mask), "+v"(k.lo_magic), "+v"(k.hi_magic));
    return k;
}

// one packed word -> 8 exact fp16 (q - z) in the order (0,4,1,5,2,6,3,7)
__device__ inline half8_t unpack8(uint32_t w, half2_t zc_hi, half2_t zc_lo, const CtConsts& k) {
    const uint32_t w8 = w >> 8;
    const half2_t a = as_h2((w & k.lo_mask) | k.lo_magic) - zc_hi;   // (q0, q4)
    const half2_t b = as_h2((w & k.hi_mask) | k.hi_magic) - zc_lo;   // (q1, q5)
    const half2_t c = as_h2((w8 & k.lo_mask) | k.lo_magic) - zc_hi;  // (q2, q6)
    const half2_t d = as_h2((w8 & k.hi_mask) | k.hi_magic) - zc_lo;  // (q3, q7)
    return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 consecutive x values (natural order) -> the order (0,4,1,5,2,6,3,7)
__device__ inline half8_t permute8(uint4 v) {
    uint4 p;
    p.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);   // (x0, x4)
    p.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);   // (x1, x5)
    p.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);   // (x2, x6)
    p.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);   // (x3, x7)
    return __builtin_bit_cast(half8_t, p);
}

// Ring depth and occupancy of a kernel instance: four groups in flight while
// a slot (CT WPL weight words and XP 16-byte x pieces) is at most 24 VGPRs,
// else two; four waves per SIMD (128 VGPRs) for the single-tile instances
// with small slots, else two.
constexpr int ct_xp(int xr, int wpl) { return (xr * wpl * 4 + 63) / 64; }
constexpr int ct_depth(int xr, int wpl, int ct) { return ct * wpl + 4 * ct_xp(xr, wpl) <= 24 ? 4 : 2; }
constexpr int ct_waves_per_eu(int xr, int wpl, int ct, int nw) {
    return nw >= 16 || (ct == 1 && xr * wpl <= 64) ? 4 : 2;
}

// One group's operands of a lane: WPL packed words of its column, and MB WPL
// 16-byte pieces of the group's x in row-run order.
template <int WPL, int XP, int CT>
struct CtSlot {
    uint32_t w[CT][WPL];   // per column tile
    uint4 x[XP];           // coalesced pieces of the group's x, re-laid through LDS
};

// XR: rows of x staged (M rounded up to 4, 8, 16 or 32); MB = XR / 16
// rounded up MFMA row blocks; XP 16-byte x pieces per lane and group; CT
// 16-column MFMA tiles per block, which share every x operand read.
// The block's work: block `blk` of the layer (qweight, scales, zeros, y, N).
template <int XR, int WPL, int NW, int DEPTH, int CT>
__device__ __forceinline__ void coltile_body(const half_t* __restrict__ x, const uint32_t* __restrict__ qweight,
                                             const half_t* __restrict__ scales, const half_t* __restrict__ zeros,
                                             half_t* __restrict__ y, int M, int N, int K, int blk) {
    constexpr int G = WPL * 32;
    constexpr int MB = (XR + 15) / 16;
    constexpr int COLS = kCtCols * CT;
    constexpr int XPIECES = XR * (G / 8);                       // 16-byte pieces of x per group
    constexpr int XP = (XPIECES + 63) / 64;
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];   // (s, z) pairs [COLS][szst], then sums
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int kq = lane >> 4;                       // k-quarter of every group
    const int n0 = blk * COLS;
    const int ng = K / G;
    const int szst = ng | 1;                        // odd: 16 columns at one group hit distinct banks

    // ---- the tile's (scale, zero) pairs: consecutive threads read
    //      consecutive groups of one column (coalesced). The first
    //      kCtSZ per thread are loaded into registers before the ring's
    //      loads are issued and written to LDS after them (loads complete in
    //      order, so that write waits for these loads only); any rest
    //      (more than kCtSZ * 64 NW pairs) is staged after the ring's loads ----
    const int cols = min(COLS, N - n0);
    const uint32_t sz_bytes = static_cast<uint32_t>(cols) * static_cast<uint32_t>(ng) * 2;
    const auto rs = rsrc(scales + static_cast<int64_t>(n0) * ng, sz_bytes);
    const auto rz = rsrc(zeros + static_cast<int64_t>(n0) * ng, sz_bytes);
    uint16_t sr[kCtSZ], zr[kCtSZ];
#pragma unroll
    for (int i = 0; i < kCtSZ; ++i) {
        const int e = tid + i * NW * 64;       // column e / ng, group e % ng
        const uint32_t so = e < COLS * ng ? static_cast<uint32_t>(e) * 2 : sz_bytes;
        sr[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
        zr[i] = __builtin_amdgcn_raw_buffer_load_b16(rz, so, 0, 0);
    }

    // ---- this wave's groups and buffer offsets; offsets at or past a
    //      buffer's size read zero without touching memory ----
    const int g0 = static_cast<int>(static_cast<int64_t>(wave) * ng / NW);
    const int g1 = static_cast<int>(static_cast<int64_t>(wave + 1) * ng / NW);
    const uint32_t w_bytes = static_cast<uint32_t>(cols) * static_cast<uint32_t>(K / 2);
    const auto rw = rsrc(qweight + static_cast<int64_t>(n0) * (K / 8), w_bytes);
    // weights in MFMA lane order: lane (col, kq) of tile t reads words
    // [kq WPL, (kq + 1) WPL) of the group in column 16 t + col
    uint32_t w_lane[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
        const int c = kCtCols * t + col;
        w_lane[t] = c < cols ? static_cast<uint32_t>(c) * (K / 2) + kq * WPL * 4 : w_bytes;
    }
    // x of one group, XR rows x G values, as XP 16-byte pieces per lane:
    // piece p = lane + 64 i is 16 bytes of row p / (G / 8), so each load
    // instruction reads whole rows' runs (coalesced)
    const uint32_t x_bytes = static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2;
    const auto rx = rsrc(x, x_bytes);
    uint32_t x_piece[XP];
#pragma unroll
    for (int i = 0; i < XP; ++i) {
        const int p = lane + 64 * i;
        const int row = p / (G / 8), c8 = p % (G / 8);
        x_piece[i] = p < XPIECES && row < M ? (static_cast<uint32_t>(row) * K + c8 * 8) * 2 : x_bytes;
    }
    auto load = [&](CtSlot<WPL, XP, CT>& sl, int g) {
        const bool ok = g < g1;
#pragma unroll
        for (int t = 0; t < CT; ++t) {
            const uint32_t wo = ok && w_lane[t] < w_bytes ? w_lane[t] + static_cast<uint32_t>(g) * (G / 2) : w_bytes;
            if constexpr (WPL == 8) {
                const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 0, 0));
                const uint4 b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 16, 0));
                sl.w[t][0] = a.x; sl.w[t][1] = a.y; sl.w[t][2] = a.z; sl.w[t][3] = a.w;
                sl.w[t][4] = b.x; sl.w[t][5] = b.y; sl.w[t][6] = b.z; sl.w[t][7] = b.w;
            } else if constexpr (WPL == 4) {
                const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 0, 0));
                sl.w[t][0] = a.x; sl.w[t][1] = a.y; sl.w[t][2] = a.z; sl.w[t][3] = a.w;
            } else if constexpr (WPL == 2) {
                const uint2 a = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rw, wo, 0, 0));
                sl.w[t][0] = a.x; sl.w[t][1] = a.y;
            } else {
                sl.w[t][0] = __builtin_amdgcn_raw_buffer_load_b32(rw, wo, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const uint32_t xo = ok && x_piece[i] < x_bytes ? x_piece[i] + static_cast<uint32_t>(g) * (G * 2) : x_bytes;
            sl.x[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0));
        }
    };

    CtSlot<WPL, XP, CT> ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        load(ring[d], g0 + d);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < kCtSZ; ++i) {
        const int e = tid + i * NW * 64;
        if (e < COLS * ng) {
            const int c = e / ng, g = e - c * ng;
            lds[c * szst + g] = static_cast<uint32_t>(sr[i]) | (static_cast<uint32_t>(zr[i]) << 16);
        }
    }
    for (int e = tid + kCtSZ * NW * 64; e < COLS * ng; e += NW * 64) {
        const int c = e / ng, g = e - c * ng;
        const uint32_t so = static_cast<uint32_t>(e) * 2;
        lds[c * szst + g] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0)) |
                            (static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rz, so, 0, 0)) << 16);
    }
    __syncthreads();   // the (scale, zero) pairs are in LDS

    float4_t acc[CT][MB];
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[t][mb] = float4_t{0.f, 0.f, 0.f, 0.f};
    const CtConsts uk = ct_consts();
    // the wave's x buffer: XR rows of G values, rows padded by 16 bytes so
    // the 16 rows of an MFMA operand read hit distinct banks; operand rows
    // past XR are zero and not read
    constexpr int XST = G + 8;
    half_t* xw = reinterpret_cast<half_t*>(lds + ct_x_offset(ng, CT)) + wave * (XR * XST);
    for (int gb = g0; gb < g1; gb += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int g = gb + d;
            CtSlot<WPL, XP, CT>& sl = ring[d];
            if (g < g1) {
                float s[CT];
                half2_t zh[CT], zl[CT];
#pragma unroll
                for (int t = 0; t < CT; ++t) {
                    const uint32_t sz = lds[(kCtCols * t + col) * szst + g];
                    const half_t z = __builtin_bit_cast(half_t, static_cast<uint16_t>(sz >> 16));
                    const half_t h = static_cast<half_t>(1024.0f) + z;   // exact
                    const half_t l = static_cast<half_t>(64.0f) + z;     // exact
                    zh[t] = half2_t{h, h};
                    zl[t] = half2_t{l, l};
                    s[t] = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(sz & 0xFFFFu)));
                }
                float4_t part[CT][MB];
#pragma unroll
                for (int t = 0; t < CT; ++t)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) part[t][mb] = float4_t{0.f, 0.f, 0.f, 0.f};
                // x pieces to the wave's LDS rows, then back in operand order:
                // lane (row col, quarter kq) takes 8 values at k = 8 (kq WPL + j)
                // (one wave's LDS accesses execute in order, so no barrier)
#pragma unroll
                for (int i = 0; i < XP; ++i) {
                    const int p = lane + 64 * i;
                    if (XPIECES % 64 == 0 || p < XPIECES)
                        *reinterpret_cast<uint4*>(&xw[(p / (G / 8)) * XST + (p % (G / 8)) * 8]) = sl.x[i];
                }
#pragma unroll
                for (int j = 0; j < WPL; ++j) {
                    half8_t b[CT];
#pragma unroll
                    for (int t = 0; t < CT; ++t) b[t] = unpack8(sl.w[t][j], zh[t], zl[t], uk);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        uint4 xv = {0u, 0u, 0u, 0u};
                        if (XR % 16 == 0 || 16 * mb + col < XR)
                            xv = *reinterpret_cast<const uint4*>(&xw[(16 * mb + col) * XST + (kq * WPL + j) * 8]);
                        const half8_t a = permute8(xv);
#pragma unroll
                        for (int t = 0; t < CT; ++t)
                            part[t][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[t], part[t][mb], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int t = 0; t < CT; ++t)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[t][mb][e] += s[t] * part[t][mb][e];
            }
            load(sl, g + DEPTH);                          // refill the slot
        }
    }

    // ---- the waves' sums, added in wave order: lane l holds rows
    //      16 mb + 4 (l / 16) + e of column 16 t + l % 16 (over the x
    //      buffers, which every wave is done with after the barrier) ----
    __syncthreads();
    float4_t* red = reinterpret_cast<float4_t*>(lds + ct_x_offset(ng, CT));
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) red[((wave * CT + t) * MB + mb) * 64 + lane] = acc[t][mb];
    __syncthreads();
    for (int i = tid; i < CT * MB * 256; i += NW * 64) {
        const int t = i / (MB * 256), r = i - t * (MB * 256);
        const int mb = r >> 8, l = (r >> 2) & 63, e = r & 3;
        float sum = 0.f;
        for (int w = 0; w < NW; ++w) sum += red[((w * CT + t) * MB + mb) * 64 + l][e];
        const int row = 16 * mb + 4 * (l >> 4) + e;
        const int n = n0 + kCtCols * t + (l & 15);
        if (row < M && n < N) y[static_cast<int64_t>(row) * N + n] = static_cast<half_t>(sum);
    }
}

template <int XR, int WPL, int NW, int DEPTH, int CT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(ct_waves_per_eu(XR, WPL, CT, NW)))) void coltile_kernel(
    const half_t* __restrict__ x, const uint32_t* __restrict__ qweight, const half_t* __restrict__ scales,
    const half_t* __restrict__ zeros, half_t* __restrict__ y, int M, int N, int K) {
    coltile_body<XR, WPL, NW, DEPTH, CT>(x, qweight, scales, zeros, y, M, N, K, blockIdx.x);
}

// Several layers that share x in one launch: layer i owns the blocks
// [first[i], first[i + 1]) (first[0] = 0; entries past the last layer are
// INT_MAX), each block working on its own layer's tensors. The layer comes
// from compares of the (uniform) block index with the bounds and scalar
// selects; an array indexed by a layer number would go to scratch memory.
struct CtLayerTable {
    const uint32_t* qweight[kGemvMaxLayers];
    const half_t* scales[kGemvMaxLayers];
    const half_t* zeros[kGemvMaxLayers];
    half_t* y[kGemvMaxLayers];
    int n[kGemvMaxLayers];
    int first[kGemvMaxLayers];
};
template <typename T>
__device__ inline T ct_pick(const CtLayerTable& L, int b, T a0, T a1, T a2, T a3) {
    T v = a0;
    v = b >= L.first[1] ? a1 : v;
    v = b >= L.first[2] ? a2 : v;
    v = b >= L.first[3] ? a3 : v;
    return v;
}
template <int XR, int WPL, int NW, int DEPTH, int CT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(ct_waves_per_eu(XR, WPL, CT, NW)))) void coltile_grouped_kernel(
    const half_t* __restrict__ x, int M, int K, CtLayerTable L) {
    const int b = blockIdx.x;
    const uint32_t* q = ct_pick(L, b, L.qweight[0], L.qweight[1], L.qweight[2], L.qweight[3]);
    const half_t* sc = ct_pick(L, b, L.scales[0], L.scales[1], L.scales[2], L.scales[3]);
    const half_t* zr = ct_pick(L, b, L.zeros[0], L.zeros[1], L.zeros[2], L.zeros[3]);
    half_t* y = ct_pick(L, b, L.y[0], L.y[1], L.y[2], L.y[3]);
    const int n = ct_pick(L, b, L.n[0], L.n[1], L.n[2], L.n[3]);
    const int f = ct_pick(L, b, L.first[0], L.first[1], L.first[2], L.first[3]);
    coltile_body<XR, WPL, NW, DEPTH, CT>(x, q, sc, zr, y, M, n, K, b - f);
}

// Two or three layers whose tensors (x, and each layer's packed weights,
// scales and zero-points) lie within 64 GB of the lowest of them: those ten
// pointers go as 32-bit offsets from that base in 16-byte units (each is
// 16-byte aligned) and the sizes in two
// dwords (mk = M | (K / 32) << 6 | n2 << 18, n01 = n0 | n1 << 16; M <= 32,
// K / 32 < 4096, n2 < 16384, n0 and n1 < 65536), so every argument a wave
// needs before its stores is in the 14 preloaded argument dwords; the
// output pointers follow as an aggregate. A layer's first block follows
// from the row counts, as the host computes it.
template <int NL>
struct CtOutTail {
    half_t* y[NL];
};
template <int XR, int WPL, int NW, int DEPTH, int CT, int NL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(ct_waves_per_eu(XR, WPL, CT, NW)))) void coltile_grouped_packed_kernel(
    const char* base, uint32_t ox, uint32_t oq0, uint32_t oq1, uint32_t oq2, uint32_t os0, uint32_t os1, uint32_t os2,
    uint32_t oz0, uint32_t oz1, uint32_t oz2, uint32_t mk, uint32_t n01, CtOutTail<NL> tail) {
    static_assert(NL == 2 || NL == 3, "two or three layers");
    constexpr int COLS = kCtCols * CT;
    const int M = static_cast<int>(mk & 63u);
    const int K = static_cast<int>((mk >> 6) & 0xFFFu) * 32;
    const int n0 = static_cast<int>(n01 & 0xFFFFu), n1 = static_cast<int>(n01 >> 16);
    const int n2 = static_cast<int>(mk >> 18);
    const int f1 = (n0 + COLS - 1) / COLS;
    const int f2 = f1 + (n1 + COLS - 1) / COLS;
    const int b = blockIdx.x;
    const bool in1 = b >= f1;
    const bool in2 = NL > 2 && b >= f2;
    const uint32_t oq = in2 ? oq2 : in1 ? oq1 : oq0;
    const uint32_t os = in2 ? os2 : in1 ? os1 : os0;
    const uint32_t oz = in2 ? oz2 : in1 ? oz1 : oz0;
    half_t* y = in2 ? tail.y[NL > 2 ? 2 : 0] : in1 ? tail.y[1] : tail.y[0];
    const int n = in2 ? n2 : in1 ? n1 : n0;
    const int f = in2 ? f2 : in1 ? f1 : 0;
    auto at = [&](uint32_t off) { return base + (static_cast<uint64_t>(off) << 4); };
    coltile_body<XR, WPL, NW, DEPTH, CT>(reinterpret_cast<const half_t*>(at(ox)),
                                         reinterpret_cast<const uint32_t*>(at(oq)),
                                         reinterpret_cast<const half_t*>(at(os)),
                                         reinterpret_cast<const half_t*>(at(oz)), y, M, n, K, b - f);
}

// rows of x a launch stages: M rounded up to 4, 8, 16 or 32
int ct_rows(int64_t M) { return M <= 4 ? 4 : M <= 8 ? 8 : M <= 16 ? 16 : 32; }
// largest tile count an instance takes without spilling
constexpr int ct_max_tiles(int xr, int wpl) { return xr * wpl >= 256 ? 2 : 4; }
// 16-column tiles per block. Each extra tile reuses every x operand read
// (x costs M / 4 times the weight bytes per tile), but leaves fewer blocks.
// From 16 rows of x up, the count that minimises the busiest CU's work in
// tile units: its blocks (one per CU per round) times each block's weights
// (ct tiles) and x (xr / 4 tiles). Measured (us, weights past every cache;
// 1 / 2 / 3 / 4 tiles): M = 16 on 11008 x 4096 13.5 / 13.4 / 9.8 / 11.5,
// 12288 x 4096 - / - / 10.1 / 11.7, 22016 x 4096 - / - / 16.3 / 21.8,
// 13824 x 5120 22.0 / 17.3 / 21.3 / 15.8, 5120 x 13824 25.8 / 22.2 / - /
// 32.3, 8192 x 28672 51.9 / 44.1 / - / 64.2, 4096 x 4096 6.5 / 8.2 / - /
// 11.1; M = 32 on 11008 x 4096 - / - / 13.1 / 15.1, 13824 x 5120
// - / - / 29.9 / 19.7; each the model's choice. Below 16 rows (weights
// dominate, and more waves per CU matter more): 2 from 1.25 column tiles
// per CU on rows of 40 groups and more, else 1; M = 4 on 13824 x 5120
// 15.5 / 14.4 / - / 17.4, 11008 x 4096 10.3 / 10.9 / - / 13.3.
// Blocks of a launch at ct tiles per block: N rows of one layer, or with L
// the layers of L, each on whole blocks of its own columns.
int64_t ct_blocks(int64_t N, int ct, const GemvLayers* L) {
    if (L == nullptr) return ceil_div(N, kCtCols * ct);
    int64_t b = 0;
    for (int i = 0; i < L->n; ++i) b += ceil_div(L->row0[i + 1] - L->row0[i], kCtCols * ct);
    return b;
}
int ct_tiles(int64_t M, int64_t N, int64_t K, int group_size, const GemvLayers* L = nullptr) {
    const int64_t cu = cu_count();
    const int64_t tiles = ceil_div(N, kCtCols);
    const int xr = ct_rows(M);
    const int most = ct_max_tiles(xr, group_size / 32);
    if (xr >= 16) {
        int best = 1;
        int64_t best_cost = INT64_MAX;
        for (int ct = 1; ct <= most; ++ct) {
            const int64_t cost = ceil_div(ct_blocks(N, ct, L), cu) * (ct + xr / 4);
            if (cost < best_cost) {
                best_cost = cost;
                best = ct;
            }
        }
        return best;
    }
    const int ct = tiles * 4 >= 5 * cu && K / group_size >= 40 ? 2 : 1;
    return std::min(ct, most);
}
// 16-wave blocks (4 per SIMD, 128 VGPRs) only for instances whose ring fits
constexpr bool ct_sixteen_ok(int xr, int wpl, int ct) { return ct == 1 && xr * wpl <= 64; }
// Waves per block, splitting K: 4 once the blocks fill the CUs (2.5 single-
// tile blocks or 1.6 multi-tile blocks per CU), else 8; single-tile blocks
// on rows of at most 32 groups take 4 from 16 rows of x up and 16 at 4 rows.
// Measured (us, 4 / 8 / 16 waves): 4096 x 4096 M = 4 6.8 / 6.3 / 5.9,
// M = 16 6.5 / 7.1 / 8.9; 4096 x 11008 M = 4 13.4 / 10.0 / 11.1;
// 13824 x 5120 at M = 4 on 2 tiles 14.4 / 15.9; 8192 x 28672 at M = 16 on
// 2 tiles 49.1 / 44.1.
int ct_waves(int64_t M, int64_t N, int64_t K, int group_size, int ct, const GemvLayers* L = nullptr) {
    const int64_t ng = K / group_size;
    if (ng < 16) return 4;
    const int64_t cu = cu_count();
    const int64_t blocks = ct_blocks(N, ct, L);
    const int xr = ct_rows(M);
    if (ct > 1) return blocks * 5 >= 8 * cu ? 4 : 8;
    if (blocks * 2 >= 5 * cu) return 4;
    if (ng <= 32) {
        if (xr >= 16) return 4;
        if (xr <= 4 && ct_sixteen_ok(xr, group_size / 32, 1)) return 16;
    }
    return 8;
}

size_t ct_lds_bytes(int64_t K, int group_size, int xr, int nw, int ct) {
    const size_t pairs = static_cast<size_t>(ct_x_offset(static_cast<int>(K / group_size), ct)) * 4;
    const size_t xbuf = static_cast<size_t>(nw) * xr * (group_size + 8) * 2;
    const size_t sums = static_cast<size_t>(nw) * ct * ((xr + 15) / 16) * 64 * 16;
    return pairs + std::max(xbuf, sums);
}

// LDS bytes a block may take: the device's limit, or gfx950's 160 KB when
// no device can be queried (host-only kernel-choice queries)
constexpr int kGfx950Lds = 160 * 1024;
int ct_max_shared() {
    static int cached = -1;
    if (cached < 0) {
        int dev = 0, v = kGfx950Lds;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            v = kGfx950Lds;
        cached = v;
    }
    return cached;
}

// What a launch computes: one layer (qweight, scales, zeros, y; N rows),
// or with layers != nullptr the layers of that list, each on whole blocks
// (N is then the layers' total, which sets the tile and wave counts).
struct CtTarget {
    const uint32_t* qweight;
    const half_t* scales;
    const half_t* zeros;
    half_t* y;
    const GemvLayers* layers;
};

template <typename Kernel>
awq_status ct_allow_lds(Kernel* kern) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            ct_max_shared()) != hipSuccess)
        return AWQ_ERR_HIP;
    return AWQ_OK;
}

template <int XR, int WPL, int NW, int CT>
awq_status launch_ct(const half_t* x, const CtTarget& tg, int M, int N, int K, hipStream_t stream) {
    constexpr int DEPTH = ct_depth(XR, WPL, CT);
    constexpr int COLS = kCtCols * CT;
    const size_t lds = ct_lds_bytes(K, WPL * 32, XR, NW, CT);
    if (tg.layers == nullptr) {
        static bool attr_set = false;
        if (!attr_set) {
            const awq_status st = ct_allow_lds(&coltile_kernel<XR, WPL, NW, DEPTH, CT>);
            if (st != AWQ_OK) return st;
            attr_set = true;
        }
        const int64_t blocks = ceil_div(N, COLS);
        hipLaunchKernelGGL((coltile_kernel<XR, WPL, NW, DEPTH, CT>), dim3(static_cast<unsigned>(blocks)),
                           dim3(NW * 64), lds, stream, x, tg.qweight, tg.scales, tg.zeros, tg.y, M, N, K);
        return last_launch_status();
    }
    const GemvLayers& lys = *tg.layers;
    if (lys.n == 2 || lys.n == 3) {
        // the packed-offset entry when every early pointer is 16-byte aligned,
        // within 64 GB of the lowest, and the sizes fit their fields
        const void* ptrs[10] = {x, lys.qweight[0], lys.qweight[1], lys.scales[0], lys.scales[1], lys.zeros[0],
                                lys.zeros[1], lys.n > 2 ? lys.qweight[2] : lys.qweight[0],
                                lys.n > 2 ? lys.scales[2] : lys.scales[0], lys.n > 2 ? lys.zeros[2] : lys.zeros[0]};
        uintptr_t lo = UINTPTR_MAX, hi = 0, bits = 0;
        for (const void* p : ptrs) {
            lo = std::min(lo, reinterpret_cast<uintptr_t>(p));
            hi = std::max(hi, reinterpret_cast<uintptr_t>(p));
            bits |= reinterpret_cast<uintptr_t>(p);
        }
        const int rows0 = lys.row0[1] - lys.row0[0], rows1 = lys.row0[2] - lys.row0[1];
        const int rows2 = lys.n > 2 ? lys.row0[3] - lys.row0[2] : 0;
        if ((bits & 15) == 0 && (hi - lo) >> 4 < (uintptr_t{1} << 32) && M <= 32 && (K >> 5) < 4096 && rows0 < 65536 && rows1 < 65536 &&
            rows2 < 16384) {
            auto off = [&](const void* p) { return static_cast<uint32_t>((reinterpret_cast<uintptr_t>(p) - lo) >> 4); };
            const uint32_t mk = static_cast<uint32_t>(M) | (static_cast<uint32_t>(K >> 5) << 6) |
                                (static_cast<uint32_t>(rows2) << 18);
            const uint32_t n01 = static_cast<uint32_t>(rows0) | (static_cast<uint32_t>(rows1) << 16);
            const int64_t blocks = ceil_div(rows0, COLS) + ceil_div(rows1, COLS) + ceil_div(rows2, COLS);
            if (lys.n == 3) {
                static bool attr3 = false;
                if (!attr3) {
                    const awq_status st = ct_allow_lds(&coltile_grouped_packed_kernel<XR, WPL, NW, DEPTH, CT, 3>);
                    if (st != AWQ_OK) return st;
                    attr3 = true;
                }
                CtOutTail<3> yt{{lys.y[0], lys.y[1], lys.y[2]}};
                hipLaunchKernelGGL((coltile_grouped_packed_kernel<XR, WPL, NW, DEPTH, CT, 3>),
                                   dim3(static_cast<unsigned>(blocks)), dim3(NW * 64), lds, stream,
                                   reinterpret_cast<const char*>(lo), off(x), off(ptrs[1]), off(ptrs[2]),
                                   off(ptrs[7]), off(ptrs[3]), off(ptrs[4]), off(ptrs[8]), off(ptrs[5]),
                                   off(ptrs[6]), off(ptrs[9]), mk, n01, yt);
            } else {
                static bool attr2 = false;
                if (!attr2) {
                    const awq_status st = ct_allow_lds(&coltile_grouped_packed_kernel<XR, WPL, NW, DEPTH, CT, 2>);
                    if (st != AWQ_OK) return st;
                    attr2 = true;
                }
                CtOutTail<2> yt{{lys.y[0], lys.y[1]}};
                hipLaunchKernelGGL((coltile_grouped_packed_kernel<XR, WPL, NW, DEPTH, CT, 2>),
                                   dim3(static_cast<unsigned>(blocks)), dim3(NW * 64), lds, stream,
                                   reinterpret_cast<const char*>(lo), off(x), off(ptrs[1]), off(ptrs[2]),
                                   off(ptrs[7]), off(ptrs[3]), off(ptrs[4]), off(ptrs[8]), off(ptrs[5]),
                                   off(ptrs[6]), off(ptrs[9]), mk, n01, yt);
            }
            return last_launch_status();
        }
    }
    static bool attr_set_grouped = false;
    if (!attr_set_grouped) {
        const awq_status st = ct_allow_lds(&coltile_grouped_kernel<XR, WPL, NW, DEPTH, CT>);
        if (st != AWQ_OK) return st;
        attr_set_grouped = true;
    }
    const GemvLayers& ly = *tg.layers;
    CtLayerTable T{};
    int64_t blocks = 0;
    for (int i = 0; i < kGemvMaxLayers; ++i) {
        if (i < ly.n) {
            const int rows = ly.row0[i + 1] - ly.row0[i];
            T.qweight[i] = ly.qweight[i];
            T.scales[i] = ly.scales[i];
            T.zeros[i] = ly.zeros[i];
            T.y[i] = ly.y[i];
            T.n[i] = rows;
            T.first[i] = static_cast<int>(blocks);
            blocks += ceil_div(rows, COLS);
        } else {
            T.first[i] = INT32_MAX;
        }
    }
    hipLaunchKernelGGL((coltile_grouped_kernel<XR, WPL, NW, DEPTH, CT>), dim3(static_cast<unsigned>(blocks)),
                       dim3(NW * 64), lds, stream, x, M, K, T);
    return last_launch_status();
}

template <int XR, int WPL, int CT>
awq_status launch_ct_nw(const half_t* x, const CtTarget& tg, int M, int N, int K, hipStream_t stream) {
    switch (ct_waves(M, N, K, WPL * 32, CT, tg.layers)) {
        case 16:
            if constexpr (ct_sixteen_ok(XR, WPL, CT)) return launch_ct<XR, WPL, 16, CT>(x, tg, M, N, K, stream);
            return launch_ct<XR, WPL, 8, CT>(x, tg, M, N, K, stream);
        case 8: return launch_ct<XR, WPL, 8, CT>(x, tg, M, N, K, stream);
        default: return launch_ct<XR, WPL, 4, CT>(x, tg, M, N, K, stream);
    }
}

template <int XR, int WPL>
awq_status launch_ct_tiles(const half_t* x, const CtTarget& tg, int M, int N, int K, hipStream_t stream) {
    switch (ct_tiles(M, N, K, WPL * 32, tg.layers)) {
        case 1: return launch_ct_nw<XR, WPL, 1>(x, tg, M, N, K, stream);
        case 2: return launch_ct_nw<XR, WPL, 2>(x, tg, M, N, K, stream);
        case 3:
            if constexpr (ct_max_tiles(XR, WPL) >= 3 && XR >= 16) return launch_ct_nw<XR, WPL, 3>(x, tg, M, N, K, stream);
            return AWQ_ERR_CONFIG;
        default: return launch_ct_nw<XR, WPL, ct_max_tiles(XR, WPL)>(x, tg, M, N, K, stream);
    }
}

template <int WPL>
awq_status launch_ct_mb(const half_t* x, const CtTarget& tg, int M, int N, int K, hipStream_t stream) {
    switch (ct_rows(M)) {
        case 4: return launch_ct_tiles<4, WPL>(x, tg, M, N, K, stream);
        case 8: return launch_ct_tiles<8, WPL>(x, tg, M, N, K, stream);
        case 16: return launch_ct_tiles<16, WPL>(x, tg, M, N, K, stream);
        default: return launch_ct_tiles<32, WPL>(x, tg, M, N, K, stream);
    }
}

awq_status launch_ct_g(const half_t* x, const CtTarget& tg, int M, int N, int K, int group_size, hipStream_t stream) {
    switch (group_size) {
        case 32: return launch_ct_mb<1>(x, tg, M, N, K, stream);
        case 64: return launch_ct_mb<2>(x, tg, M, N, K, stream);
        case 128: return launch_ct_mb<4>(x, tg, M, N, K, stream);
        case 256: return launch_ct_mb<8>(x, tg, M, N, K, stream);
        default: return AWQ_ERR_CONFIG;
    }
}

}  // namespace

// The automatic kernel choice (awq_gemm): column tiles from 3 rows of x up
// where they beat the GEMV and the skinny kernel. Measured (us, weights past
// every cache; column tiles against the skinny kernel with K splits):
// 4096 x 4096 at M = 4 / 16 / 32 5.9 / 6.5 / 8.6 (10.5 / 10.6 / 13.0);
// 11008 x 4096 10.2 / 11.7 / 15.4 (13.4 / 13.7 / 16.4); 4096 x 11008
// 10.2 / 13.2 / 18.0 (15.1 / 15.3 / 19.6); 13824 x 5120 14.7 / 16.2 / 20.3
// (17.3 / 16.7 / 22.2); the skinny kernel leads on long rows of large
// layers: 5120 x 13824 18.0 / 22.2 / 27.7 (17.5 / 17.8 / 24.6), 8192 x
// 28672 37.6 / 45.0 / 55.3 (35.7 / 35.8 / 53.8). The GEMV leads at M = 2;
// at M = 4 it takes 6.2 us on 4096 x 4096 and 12.6 on 11008 x 4096. Without
// a workspace the skinny kernel walks K in phases (2-5x slower), so column
// tiles take every shape they support.
bool coltile_preferred(int64_t M, int64_t N, int64_t K, int group_size, bool have_workspace) {
    if (M < 3 || !coltile_supported(M, N, K, group_size)) return false;
    if (!have_workspace) return true;
    const int64_t weights = N * K;
    return weights <= (int64_t{48} << 20) || (K <= 8192 && weights <= (int64_t{96} << 20));
}

namespace {
bool ct_supported(int64_t M, int64_t N, int64_t K, int group_size, const GemvLayers* L) {
    if (group_size < 32 || group_size > 256) return false;
    if (M < 1 || M > kColTileMaxM || N < 1 || K < group_size || K % group_size != 0) return false;
    // 32-bit buffer offsets: x, and one 16-column tile of packed weights
    const int ct = ct_tiles(M, N, K, group_size, L);
    if (M * K * 2 >= (int64_t{1} << 31) || kCtCols * ct * (K / 2) >= (int64_t{1} << 31)) return false;
    return ct_lds_bytes(K, group_size, ct_rows(M), ct_waves(M, N, K, group_size, ct, L), ct) <=
           static_cast<size_t>(ct_max_shared());
}
}  // namespace

bool coltile_supported(int64_t M, int64_t N, int64_t K, int group_size) {
    return ct_supported(M, N, K, group_size, nullptr);
}

bool coltile_grouped_supported(int64_t M, const GemvLayers& layers, int64_t K, int group_size) {
    return layers.n >= 1 && ct_supported(M, layers.row0[layers.n], K, group_size, &layers);
}

awq_status launch_coltile(const half_t* x, const uint32_t* qweight, const half_t* scales, const half_t* zeros,
                          int64_t M, int64_t N, int64_t K, int group_size, half_t* y, hipStream_t stream) {
    if (M == 0 || N == 0) return AWQ_OK;
    if (!coltile_supported(M, N, K, group_size)) return AWQ_ERR_CONFIG;
    const CtTarget tg{qweight, scales, zeros, y, nullptr};
    return launch_ct_g(x, tg, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), group_size, stream);
}

awq_status launch_coltile_grouped(const half_t* x, const GemvLayers& layers, int64_t M, int64_t K, int group_size,
                                  hipStream_t stream) {
    const int64_t total = layers.row0[layers.n];
    if (M == 0 || total == 0) return AWQ_OK;
    if (!coltile_grouped_supported(M, layers, K, group_size)) return AWQ_ERR_CONFIG;
    const CtTarget tg{nullptr, nullptr, nullptr, nullptr, &layers};
    return launch_ct_g(x, tg, static_cast<int>(M), static_cast<int>(total), static_cast<int>(K), group_size, stream);
}

}  // namespace awq
