// Decode GEMV of the W4A16 linear layer, y[M, N] = x[M, K] . dequant(Wq)^T
// (and of the W8A16 form, BITS = 8: a 16-byte chunk holds 16 byte codes)
// for small M (single-stream decode: the "GEMV" kernel choice of the rskf.cn
// AWQ article, §3.3; the dequantize-in-the-matmul step of §1.3). Decode is
// bound by streaming the packed weights from HBM, so the kernel is built to
// put all of a wave's weight bytes in flight at once with 16-byte coalesced
// loads, and to keep everything else on chip.
//
// Work split:
//  * a block of NW wavefronts (4, or 8 in the persistent form) owns NW * RPW
//    consecutive output rows at a time; a wavefront owns RPW rows. Lane l handles the 32-weight chunks c = l + 64 j
//    (j < CPL), one uint4 of qweight per row and chunk, so each wave-wide load
//    is 1 KB of contiguous packed weights;
//  * the wave first issues all RPW * CPL weight loads (plus the matching
//    scale and zero-point), then the block stages x in LDS while those loads
//    are in flight: x is rearranged into the fp16 pairs that match the
//    nibble unpack below, with two sums per chunk;
//  * the partial dot products are reduced across the wavefront with xor
//    shuffles (no atomics: results are deterministic). K beyond 64 * CPL
//    chunks is walked in further passes of the same shape.
//
// Nibble unpack (8 codes of one word, code j in bits 4j..4j+3): OR-ing a
// nibble into the mantissa of an fp16 constant gives an exact fp16 integer:
//   (w & 0x000F000F) | 0x64006400 = (1024 + q0, 1024 + q4)
//   (w & 0x00F000F0) | 0x54005400 = (  64 + q1,   64 + q5)
// and the same on w >> 8 for (q2, q6) and (q3, q7). v_dot2_f32_f16 multiplies
// these with the matching x pairs (exact products, fp32 sums); the constant
// offsets and the zero-point are removed per chunk with precomputed sums
//   off = 1024 * sum_{j even} x_j + 64 * sum_{j odd} x_j,   xs = sum_j x_j,
// so sum_k x_k (q_k - z) = dot - off - z * xs, then scaled by the group's
// scale in fp32. The weight is never rounded to fp16.
#include <algorithm>
#include <type_traits>

#include "awq_internal.h"

namespace awq {

constexpr int64_t kGemvBlocksPerCu = 1;
namespace {

__device__ inline half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ inline float h_lo(uint32_t u) {
    return static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(u & 0xFFFFu)));
}
__device__ inline float h_hi(uint32_t u) {
    return static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(u >> 16)));
}

// The four unpack constants, held in VGPRs: gfx9 VOP3 instructions cannot
// take 32-bit literals and read at most one SGPR, so only with register
// operands does (w & mask) | magic become a single v_and_or_b32.
struct UnpackConsts {
    uint32_t lo_mask, hi_mask, lo_magic, hi_magic;
};
template <int BITS>
__device__ inline UnpackConsts unpack_consts() {
    UnpackConsts k = BITS == 4 ? UnpackConsts{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u}
                               : UnpackConsts{0x00FF00FFu, 0x00FF00FFu, 0x64006400u, 0x64006400u};
    asm volatile("" : "+v"(k.lo_mask), "+v"(k.hi_mask), "+v"(k.lo_magic), "+v"(k.hi_magic));
    return k;
}

// dot of one packed word (8 codes, offset-encoded) with its 4 x pairs
__device__ inline float word_dot(uint32_t wq, const uint4& p, float acc, const UnpackConsts& k) {
    const uint32_t w8 = wq >> 8;
    const uint32_t a = (wq & k.lo_mask) | k.lo_magic;
    const uint32_t b = (wq & k.hi_mask) | k.hi_magic;
    const uint32_t c = (w8 & k.lo_mask) | k.lo_magic;
    const uint32_t d = (w8 & k.hi_mask) | k.hi_magic;
    acc = __builtin_amdgcn_fdot2(as_h2(a), as_h2(p.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(b), as_h2(p.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(c), as_h2(p.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(d), as_h2(p.w), acc, false);
    return acc;
}

// dot of one W8 word (4 byte codes) with its 2 x pairs (x0, x2), (x1, x3):
//   (w & 0x00FF00FF) | 0x64006400 = (1024 + b0, 1024 + b2), the same on w >> 8
__device__ inline float byte_dot(uint32_t wq, uint32_t p_even, uint32_t p_odd, float acc, const UnpackConsts& k) {
    const uint32_t a = (wq & k.lo_mask) | k.lo_magic;
    const uint32_t b = ((wq >> 8) & k.hi_mask) | k.hi_magic;
    acc = __builtin_amdgcn_fdot2(as_h2(a), as_h2(p_even), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(b), as_h2(p_odd), acc, false);
    return acc;
}

// Chunk geometry: a chunk is one 16-byte load of packed weights per lane:
// 32 INT4 or 16 W8 weights, staged against XV uint4 of x pairs.
template <int BITS>
struct Chunk {
    static constexpr int kShift = BITS == 4 ? 5 : 4;     // log2(weights per chunk)
    static constexpr int kXV = BITS == 4 ? 4 : 2;        // uint4 of x pairs per chunk
};

template <int RPW, int CPL>
struct WeightBatch {
    uint4 w[RPW][CPL];
    uint16_t s[RPW][CPL];   // raw fp16 bits, converted when consumed
    uint16_t z[RPW][CPL];
};

// Buffer descriptor over `bytes` bytes at p (raw, stride 0). A load at or
// past `bytes` returns zero and touches no memory, so out-of-range chunks and
// items need no branches.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), bytes, 0x00020000);
}

// The layer table of a grouped launch of up to four layers (built in the
// kernel from its arguments, as scalars: an array indexed by the layer
// number went to scratch memory). The layers' packed-weight pointers and
// the first stacked rows of layers 1-3 arrive in preloaded SGPRs (up to
// three layers), so a wave's weight loads wait for no scalar load; the
// scale, zero-point and output pointers come by scalar loads issued at the
// start, which the weight loads do not wait for.
struct GemvLayerTable {
    const uint32_t *q0, *q1, *q2, *q3;
    const half_t *s0, *s1, *s2, *s3;
    const half_t *z0, *z1, *z2, *z3;
    half_t *y0, *y1, *y2, *y3;
    int b1, b2, b3;   // first stacked rows of layers 1-3
};
// the value of stacked row r's layer among NL: selects on compares with
// the bounds (a select chain on a layer number was turned into an indexed
// stack array, in scratch memory)
template <int NL, typename T>
__device__ inline T pick_row(const GemvLayerTable& L, int r, T a0, T a1, T a2, T a3) {
    T v = a0;
    if constexpr (NL > 1) v = r >= L.b1 ? a1 : v;
    if constexpr (NL > 2) v = r >= L.b2 ? a2 : v;
    if constexpr (NL > 3) v = r >= L.b3 ? a3 : v;
    return v;
}
struct NoLayers {};
template <int NL>
using LayersArg = std::conditional_t<(NL > 0), GemvLayerTable, NoLayers>;

// Issues the loads of one item: RPW rows x CPL chunks per lane (chunk
// c = base + lane + 64 j), with each chunk's scale and zero-point. Rows past
// N or items past the wave's last (valid == false) read as zero. NL > 0 (a
// grouped launch): row r is row r - start of its layer's tensors, and every
// weight load is issued before the scale and zero-point loads, whose
// pointers come later.
template <int BITS, int RPW, int CPL, int NL, bool SZL = false>
__device__ inline void load_batch(WeightBatch<RPW, CPL>& b, const uint32_t* __restrict__ qweight,
                                  const half_t* __restrict__ scales, const half_t* __restrict__ zeros,
                                  const LayersArg<NL>& L, int row0, bool valid, int N, int nchunk, int ngroups,
                                  int log2g, int base, int lane) {
    if constexpr (NL > 0) {
        int lay[RPW];   // the stacked row
        int64_t lr[RPW];
        bool ok[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int row = row0 + i;
            ok[i] = valid && row < N;
            const int r = ok[i] ? row : 0;
            lay[i] = r;
            lr[i] = r - pick_row<NL>(L, r, 0, L.b1, L.b2, L.b3);
            const auto rw = rsrc(pick_row<NL>(L, r, L.q0, L.q1, L.q2, L.q3) + lr[i] * (nchunk * 4),
                                 ok[i] ? nchunk * 16 : 0);
#pragma unroll
            for (int j = 0; j < CPL; ++j)
                b.w[i][j] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, (base + lane + 64 * j) * 16, 0, 0));
        }
        // keeps the scale and zero-point addressing (which waits for the
        // scalar loads of their pointers) behind every weight load
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = lay[i];
            const auto rs = rsrc(pick_row<NL>(L, r, L.s0, L.s1, L.s2, L.s3) + lr[i] * ngroups, ok[i] ? ngroups * 2 : 0);
            const auto rz = rsrc(pick_row<NL>(L, r, L.z0, L.z1, L.z2, L.z3) + lr[i] * ngroups, ok[i] ? ngroups * 2 : 0);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int g = ((base + lane + 64 * j) << Chunk<BITS>::kShift) >> log2g;
                b.s[i][j] = __builtin_amdgcn_raw_buffer_load_b16(rs, g * 2, 0, 0);
                b.z[i][j] = __builtin_amdgcn_raw_buffer_load_b16(rz, g * 2, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int row = row0 + i;
            const bool ok = valid && row < N;
            const int64_t r = ok ? row : 0;
            const auto rw = rsrc(qweight + r * (nchunk * 4), ok ? nchunk * 16 : 0);
            const auto rs = rsrc(scales + r * ngroups, ok ? ngroups * 2 : 0);
            const auto rz = rsrc(zeros + r * ngroups, ok ? ngroups * 2 : 0);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = base + lane + 64 * j;
                const int g = (c << Chunk<BITS>::kShift) >> log2g;
                b.w[i][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, c * 16, 0, 0));
                if constexpr (!SZL) {
                    b.s[i][j] = __builtin_amdgcn_raw_buffer_load_b16(rs, g * 2, 0, 0);
                    b.z[i][j] = __builtin_amdgcn_raw_buffer_load_b16(rz, g * 2, 0, 0);
                }
            }
        }
    }
}

// Consumes one item: chunks past the row end have scale 0 (zero-filled
// loads) and read a clamped, in-range slot of the staged x.
// SZL: the (scale, zero) pairs come from the block's LDS copy (szrow: the
// item's first row, ngroups words per row), where chunks past the row end
// read a clamped group and are masked to scale 0 instead.
template <int BITS, int MT, int RPW, int CPL, bool SZL = false>
__device__ inline void compute_batch(const WeightBatch<RPW, CPL>& b, const uint4* __restrict__ xp,
                                     const float2* __restrict__ xo, float (&acc)[RPW][MT], int nchunk,
                                     int base, int lane, const UnpackConsts& k,
                                     const uint32_t* __restrict__ szrow = nullptr, int ngroups = 0,
                                     int log2g = 0) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        [[maybe_unused]] const bool in_row = base + lane + 64 * j < nchunk;
        const int c = min(base + lane + 64 * j, nchunk - 1);
        [[maybe_unused]] const int g = (c << Chunk<BITS>::kShift) >> log2g;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float2 o = xo[m * nchunk + c];
            uint4 p[Chunk<BITS>::kXV];
#pragma unroll
            for (int v = 0; v < Chunk<BITS>::kXV; ++v) p[v] = xp[(m * Chunk<BITS>::kXV + v) * nchunk + c];
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                float d = 0.f;
                if constexpr (BITS == 4) {
                    d = word_dot(b.w[i][j].x, p[0], d, k);
                    d = word_dot(b.w[i][j].y, p[1], d, k);
                    d = word_dot(b.w[i][j].z, p[2], d, k);
                    d = word_dot(b.w[i][j].w, p[Chunk<BITS>::kXV - 1], d, k);
                } else {
                    d = byte_dot(b.w[i][j].x, p[0].x, p[0].y, d, k);
                    d = byte_dot(b.w[i][j].y, p[0].z, p[0].w, d, k);
                    d = byte_dot(b.w[i][j].z, p[Chunk<BITS>::kXV - 1].x, p[Chunk<BITS>::kXV - 1].y, d, k);
                    d = byte_dot(b.w[i][j].w, p[Chunk<BITS>::kXV - 1].z, p[Chunk<BITS>::kXV - 1].w, d, k);
                }
                float s, z;
                if constexpr (SZL) {
                    const uint32_t sz = szrow[i * ngroups + g];
                    s = in_row ? static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(sz & 0xFFFFu)))
                               : 0.f;
                    z = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(sz >> 16)));
                } else {
                    s = static_cast<float>(__builtin_bit_cast(half_t, b.s[i][j]));
                    z = static_cast<float>(__builtin_bit_cast(half_t, b.z[i][j]));
                }
                acc[i][m] += s * (d - (o.x + z * o.y));
            }
        }
    }
}

// Sum over the 64 lanes of a wavefront with DPP moves (no LDS traffic):
// quad swaps, two rotations within each 16-lane row, then two row
// broadcasts. The total lands in lane 63.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false);
    return v + __builtin_bit_cast(float, t);
}
__device__ inline float wave_sum_lane63(float v) {
    v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v = dpp_add<0x124, 0xF>(v);   // row_ror:4
    v = dpp_add<0x128, 0xF>(v);   // row_ror:8
    v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// Persistent streaming kernel. Each wavefront walks a sequence of items
// (RPW rows x one batch of CPL chunks per lane): its row sets stride over the
// grid, the k-batches of a row set come in order. A ring of DEPTH register
// batches keeps DEPTH items in flight: item t is consumed while the next
// DEPTH - 1 are still loading, and its slot is refilled with item t + DEPTH
// right after. The loads are branch-free, so the compiler's wait counts track
// the ring exactly. Finished rows go to LDS and are written out at the end.
//
// NL > 0: the rows of NL layers sharing x, stacked (L); N is the total, and
// each row's weights and output belong to its layer.
//
// SZL (streaming, single layer): the (scale, zero) pairs of the block's rows
// are staged once in LDS as packed words instead of being loaded with every
// chunk (two 2-byte loads per 16-byte weight load). A wave's row sets are
// set = wid + k W, so for each k the block's rows form one run of NW RPW
// consecutive rows, whose pairs are contiguous in memory; run k lands at
// word k NW RPW ngroups, so row i of wave w in set k is word
// ((k NW + w) RPW + i) ngroups. Needs (N ngroups) % 8 == 0 (16-byte pieces
// never straddle the end of the tensors) and NW RPW ngroups % 8 == 0.
constexpr int kSzPre = 4;   // 16-byte (scale, zero) pieces per thread loaded ahead of the ring
// word offset of the packed pairs in the block's LDS: after x pairs
// [MT][XV][nchunk] (uint4), offsets [MT][nchunk] (float2) and the parked sums
// [slots][MT] (float), rounded up to 16 bytes
__host__ __device__ inline int gemv_sz_word_offset(int mt, int nchunk, int xv, int slots) {
    return (mt * nchunk * xv * 4 + mt * nchunk * 2 + slots * mt + 3) & ~3;
}
template <int BITS, int MT, int RPW, int CPL, int DEPTH, bool ONESHOT, int NW, int NL, bool SZL = false>
__device__ __forceinline__ void gemv_body(const half_t* __restrict__ x, const uint32_t* __restrict__ qweight,
                                          const half_t* __restrict__ scales, const half_t* __restrict__ zeros,
                                          half_t* __restrict__ y, int N, int K, int log2g, int max_sets,
                                          int nblocks, const LayersArg<NL>& L) {
    extern __shared__ uint4 smem[];
    constexpr int XV = Chunk<BITS>::kXV;
    const int nchunk = K >> Chunk<BITS>::kShift;    // 32 (INT4) or 16 (W8) weights per chunk
    // x pairs [MT][XV][nchunk]: lanes reading one v of consecutive chunks
    // hit consecutive 16-byte slots (no bank conflicts)
    uint4* xp = smem;
    float2* xo = reinterpret_cast<float2*>(smem + MT * nchunk * XV);  // [MT][nchunk] (off, xs)
    float* yl = reinterpret_cast<float*>(xo + MT * nchunk);          // [NW][max_sets][RPW][MT]
    // SZL: packed (s, z) words, 16-byte aligned after yl
    uint32_t* szl = reinterpret_cast<uint32_t*>(smem) + gemv_sz_word_offset(MT, nchunk, XV, NW * max_sets * RPW);

    // wave index as a scalar: the buffer descriptors built from it must be
    // wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ngroups = K >> log2g;

    const int kbs = (nchunk + 64 * CPL - 1) / (64 * CPL);      // k-batches per row
    const int nsets = (N + RPW - 1) / RPW;                      // row sets
    const int W = nblocks * NW;
    const int wid = blockIdx.x * NW + wave;
    const int my_sets = wid < nsets ? (nsets - 1 - wid) / W + 1 : 0;
    const int n_items = my_sets * kbs;

    // x staging: one chunk of x (32 values per activation row) is loaded,
    // rearranged into the pairs word_dot expects and written to LDS with its
    // two sums.
    auto load_x = [&](int c, uint4 (&r)[MT][XV]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4* src = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(m) * K) + c * XV;
#pragma unroll
            for (int j = 0; j < XV; ++j) r[m][j] = src[j];
        }
    };
    auto store_x = [&](int c, const uint4 (&r)[MT][XV]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float even = 0.f, odd = 0.f;
#pragma unroll
            for (int j = 0; j < XV; ++j) {
                const uint4 v = r[m][j];  // halves (0,1) (2,3) (4,5) (6,7)
                uint4 p;
                if constexpr (BITS == 4) {
                    // the pairs of one packed word: (x0, x4) (x1, x5) (x2, x6) (x3, x7)
                    p.x = (v.x & 0xFFFFu) | (v.z << 16);
                    p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
                    p.z = (v.y & 0xFFFFu) | (v.w << 16);
                    p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
                } else {
                    // the pairs of two W8 words: (x0, x2) (x1, x3) (x4, x6) (x5, x7)
                    p.x = (v.x & 0xFFFFu) | (v.y << 16);
                    p.y = (v.x >> 16) | (v.y & 0xFFFF0000u);
                    p.z = (v.z & 0xFFFFu) | (v.w << 16);
                    p.w = (v.z >> 16) | (v.w & 0xFFFF0000u);
                }
                xp[(m * XV + j) * nchunk + c] = p;
                even += (h_lo(v.x) + h_lo(v.y)) + (h_lo(v.z) + h_lo(v.w));
                odd += (h_hi(v.x) + h_hi(v.y)) + (h_hi(v.z) + h_hi(v.w));
            }
            // offsets the magic constants add: 1024 on even halves and 64 on
            // odd halves of an INT4 word, 1024 on every W8 byte
            const float off = BITS == 4 ? 1024.0f * even + 64.0f * odd : 1024.0f * (even + odd);
            xo[m * nchunk + c] = make_float2(off, even + odd);
        }
    };

    // 1. this thread's first x chunks, then the first DEPTH items of weights,
    //    all in flight together (loads complete in order, so x is issued
    //    first and can be consumed without waiting for the weights)
    constexpr int XPRE = MT <= 2 ? 2 : 1;
    const int c0 = threadIdx.x;
    uint4 xr[XPRE][MT][XV];
#pragma unroll
    for (int p = 0; p < XPRE; ++p)
        if (c0 + p * NW * 64 < nchunk) load_x(c0 + p * NW * 64, xr[p]);

    // SZL: the block's (scale, zero) runs, 8 groups per 16-byte piece; the
    // first kSzPre pieces per thread are in flight with the weights, offsets
    // at or past the tensors' end read zero
    [[maybe_unused]] const int sz_run = NW * RPW * ngroups;
    [[maybe_unused]] const int sz_pieces = SZL ? max_sets * sz_run / 8 : 0;
    [[maybe_unused]] const uint32_t sz_bytes = static_cast<uint32_t>(N) * static_cast<uint32_t>(ngroups) * 2u;
    auto sz_offset = [&](int e) {
        const int k = (8 * e) / sz_run;
        const int off = 8 * e - k * sz_run;
        const uint32_t row0 = static_cast<uint32_t>((blockIdx.x * NW + k * W) * RPW);
        return e < sz_pieces && row0 < static_cast<uint32_t>(N)
                   ? (row0 * static_cast<uint32_t>(ngroups) + static_cast<uint32_t>(off)) * 2u
                   : sz_bytes;
    };
    auto sz_store = [&](int e, uint4 sv, uint4 zv) {
        // word j = s_j | z_j << 16
        uint4 lo, hi;
        lo.x = __builtin_amdgcn_perm(zv.x, sv.x, 0x05040100u);
        lo.y = __builtin_amdgcn_perm(zv.x, sv.x, 0x07060302u);
        lo.z = __builtin_amdgcn_perm(zv.y, sv.y, 0x05040100u);
        lo.w = __builtin_amdgcn_perm(zv.y, sv.y, 0x07060302u);
        hi.x = __builtin_amdgcn_perm(zv.z, sv.z, 0x05040100u);
        hi.y = __builtin_amdgcn_perm(zv.z, sv.z, 0x07060302u);
        hi.z = __builtin_amdgcn_perm(zv.w, sv.w, 0x05040100u);
        hi.w = __builtin_amdgcn_perm(zv.w, sv.w, 0x07060302u);
        reinterpret_cast<uint4*>(szl)[2 * e] = lo;
        reinterpret_cast<uint4*>(szl)[2 * e + 1] = hi;
    };
    [[maybe_unused]] const auto rs_sz = rsrc(scales, SZL ? static_cast<int>(sz_bytes) : 0);
    [[maybe_unused]] const auto rz_sz = rsrc(zeros, SZL ? static_cast<int>(sz_bytes) : 0);
    [[maybe_unused]] uint4 szv[SZL ? kSzPre : 1], zzv[SZL ? kSzPre : 1];
    if constexpr (SZL) {
#pragma unroll
        for (int p = 0; p < kSzPre; ++p) {
            const uint32_t o = sz_offset(static_cast<int>(threadIdx.x) + p * NW * 64);
            szv[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_sz, o, 0, 0));
            zzv[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rz_sz, o, 0, 0));
        }
    }

    WeightBatch<RPW, CPL> ring[DEPTH];
    int l_item = 0, l_set = 0, l_kb = 0;            // load cursor
    auto issue = [&](WeightBatch<RPW, CPL>& b) {
        load_batch<BITS, RPW, CPL, NL, SZL>(b, qweight, scales, zeros, L, (wid + l_set * W) * RPW,
                                                 l_item < n_items, N, nchunk, ngroups, log2g, l_kb * 64 * CPL, lane);
        ++l_item;
        if (++l_kb == kbs) { l_kb = 0; ++l_set; }
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(ring[d]);

    // 2. stage x in LDS while the weights are in flight
#pragma unroll
    for (int p = 0; p < XPRE; ++p)
        if (c0 + p * NW * 64 < nchunk) store_x(c0 + p * NW * 64, xr[p]);
    for (int c = c0 + XPRE * NW * 64; c < nchunk; c += NW * 64) {
        load_x(c, xr[0]);
        store_x(c, xr[0]);
    }
    if constexpr (SZL) {
#pragma unroll
        for (int p = 0; p < kSzPre; ++p) {
            const int e = static_cast<int>(threadIdx.x) + p * NW * 64;
            if (e < sz_pieces) sz_store(e, szv[p], zzv[p]);
        }
        for (int e = static_cast<int>(threadIdx.x) + kSzPre * NW * 64; e < sz_pieces; e += NW * 64) {
            const uint32_t o = sz_offset(e);
            sz_store(e, __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_sz, o, 0, 0)),
                     __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rz_sz, o, 0, 0)));
        }
    }
    __syncthreads();

    // output element (m, stacked row r)
    auto store_y = [&](int m, int r, float v) {
        if constexpr (NL > 0) {
            const int start = pick_row<NL>(L, r, 0, L.b1, L.b2, L.b3);
            const int end = pick_row<NL>(L, r, NL > 1 ? L.b1 : N, NL > 2 ? L.b2 : N, NL > 3 ? L.b3 : N, N);
            pick_row<NL>(L, r, L.y0, L.y1, L.y2, L.y3)[static_cast<int64_t>(m) * (end - start) + (r - start)] =
                static_cast<half_t>(v);
        } else {
            y[static_cast<int64_t>(m) * N + r] = static_cast<half_t>(v);
        }
    };

    // 3. stream
    float acc[RPW][MT];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[i][m] = 0.f;
    int c_set = 0, c_kb = 0;            // compute cursor
    const UnpackConsts uk = unpack_consts<BITS>();
    for (int t = 0; t < n_items; t += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            if (t + d < n_items) {
                compute_batch<BITS, MT, RPW, CPL, SZL>(ring[d], xp, xo, acc, nchunk, c_kb * 64 * CPL, lane, uk,
                                                       szl + (c_set * NW + wave) * RPW * ngroups, ngroups, log2g);
                if (++c_kb == kbs) {
                    // row set finished: reduce; lane 63 stores the sums (one-shot)
                    // or parks them in LDS (streaming: no stores among the loads)
                    const int r0 = (wid + c_set * W) * RPW;
#pragma unroll
                    for (int i = 0; i < RPW; ++i) {
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            const float v = wave_sum_lane63(acc[i][m]);
                            if (ONESHOT) {
                                if (lane == 63 && r0 + i < N) store_y(m, r0 + i, v);
                            } else if (lane == 63) {
                                yl[((wave * max_sets + c_set) * RPW + i) * MT + m] = v;
                            }
                            acc[i][m] = 0.f;
                        }
                    }
                    c_kb = 0;
                    ++c_set;
                }
            }
            if (!ONESHOT) issue(ring[d]);
        }
    }
    if (ONESHOT) return;

    // 4. write the block's rows
    __syncthreads();
    const int slots = NW * max_sets * RPW;
    for (int sl = threadIdx.x; sl < slots; sl += NW * 64) {
        const int w = sl / (max_sets * RPW);
        const int rem = sl - w * max_sets * RPW;
        const int cs = rem / RPW;
        const int i = rem - cs * RPW;
        const int wg = blockIdx.x * NW + w;
        const int sets_w = wg < nsets ? (nsets - 1 - wg) / W + 1 : 0;
        const int row = (wg + cs * W) * RPW + i;
        if (cs < sets_w && row < N) {
#pragma unroll
            for (int m = 0; m < MT; ++m) store_y(m, row, yl[sl * MT + m]);
        }
    }
}

// The kernels. Every argument of the single-layer form, the grid size
// included (nblocks == gridDim.x), is in its first 14 dwords (log2 G and
// max_sets share one: shape = log2g | max_sets << 8), which the build has the
// hardware preload into SGPRs, so no wave waits on a kernel-argument load.
// Reading past them costs: a launch that also read the hidden grid-size
// argument, on a second 64-byte line, took 4-9% longer on the one-shot
// shapes (4096 x 4096: 4.06 -> 4.42 us).
template <int BITS, int MT, int RPW, int CPL, int DEPTH, bool ONESHOT, int NW, bool SZL = false>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(const half_t* __restrict__ x,
                                                   const uint32_t* __restrict__ qweight,
                                                   const half_t* __restrict__ scales,
                                                   const half_t* __restrict__ zeros,
                                                   half_t* __restrict__ y, int N, int K, int shape,
                                                   int nblocks) {
    gemv_body<BITS, MT, RPW, CPL, DEPTH, ONESHOT, NW, 0, SZL>(x, qweight, scales, zeros, y, N, K, shape & 0xFF,
                                                               shape >> 8, nblocks, NoLayers{});
}
// The grouped form takes the weight pointers of up to four layers and the
// first stacked rows of layers 1-3 as separate arguments: preloading covers
// scalar arguments only (not an aggregate), and with up to three layers
// these end within the 14 preloaded dwords. The rest of the table (scales,
// zero-points, outputs) is an aggregate loaded as usual.
template <int NL>
struct GemvLayerTail {
    const half_t* scales[NL];
    const half_t* zeros[NL];
    half_t* y[NL];
};
template <int BITS, int MT, int RPW, int CPL, int DEPTH, bool ONESHOT, int NW, int NL>
__global__ __launch_bounds__(NW * 64) void gemv_grouped_kernel(const half_t* __restrict__ x, int N, int K, int shape,
                                                           int nblocks, const uint32_t* q0, const uint32_t* q1,
                                                           const uint32_t* q2, int b1, int b2,
                                                           const uint32_t* q3, int b3, GemvLayerTail<NL> tail) {
    const GemvLayerTable L{q0, q1, q2, q3,
                           tail.scales[0], NL > 1 ? tail.scales[NL > 1 ? 1 : 0] : nullptr,
                           NL > 2 ? tail.scales[NL > 2 ? 2 : 0] : nullptr, NL > 3 ? tail.scales[NL > 3 ? 3 : 0] : nullptr,
                           tail.zeros[0], NL > 1 ? tail.zeros[NL > 1 ? 1 : 0] : nullptr,
                           NL > 2 ? tail.zeros[NL > 2 ? 2 : 0] : nullptr, NL > 3 ? tail.zeros[NL > 3 ? 3 : 0] : nullptr,
                           tail.y[0], NL > 1 ? tail.y[NL > 1 ? 1 : 0] : nullptr,
                           NL > 2 ? tail.y[NL > 2 ? 2 : 0] : nullptr, NL > 3 ? tail.y[NL > 3 ? 3 : 0] : nullptr,
                           b1, b2, b3};
    gemv_body<BITS, MT, RPW, CPL, DEPTH, ONESHOT, NW, NL>(x, nullptr, nullptr, nullptr, nullptr, N, K, shape & 0xFF,
                                                           shape >> 8, nblocks, L);
}

// One-shot grouped launches of 2 or 3 layers whose tensors (x, and each
// layer's packed weights, scales and zero-points) all lie within 64 GB of the
// lowest of them: every pointer the waves need before their first dot is a
// 32-bit offset from that base in 16-byte units (every such pointer is
// 16-byte aligned), and with the sizes packed in two dwords the whole set
// fits in the 14 preloaded argument dwords. No wave then waits on a
// kernel-argument load until its outputs are stored (the output pointers
// follow as an aggregate). nb1 = N | b1 << 16, b2k = b2 | (K / 32) << 16 |
// (log2 G - 5) << 28 (N < 65536, K / 32 < 4096). The one-shot launch shape
// gives every wave at most one row set, so the grid size follows from N.
template <int NL>
struct GemvOutTail {
    half_t* y[NL];
};
template <int BITS, int MT, int RPW, int CPL, int DEPTH, int NW, int NL>
__global__ __launch_bounds__(NW * 64) void gemv_grouped_packed_kernel(
    const char* base, uint32_t ox, uint32_t oq0, uint32_t oq1, uint32_t oq2, uint32_t os0, uint32_t os1,
    uint32_t os2, uint32_t oz0, uint32_t oz1, uint32_t oz2, uint32_t nb1, uint32_t b2k, GemvOutTail<NL> tail) {
    static_assert(NL == 2 || NL == 3, "two or three layers");
    const int N = static_cast<int>(nb1 & 0xFFFFu);
    const int K = static_cast<int>((b2k >> 16) & 0xFFFu) * 32;
    const int log2g = static_cast<int>(b2k >> 28) + 5;
    const int nblocks = ((N + RPW - 1) / RPW + NW - 1) / NW;
    auto at = [&](uint32_t off) { return base + (static_cast<uint64_t>(off) << 4); };
    const GemvLayerTable L{reinterpret_cast<const uint32_t*>(at(oq0)), reinterpret_cast<const uint32_t*>(at(oq1)),
                           NL > 2 ? reinterpret_cast<const uint32_t*>(at(oq2)) : nullptr, nullptr,
                           reinterpret_cast<const half_t*>(at(os0)), reinterpret_cast<const half_t*>(at(os1)),
                           NL > 2 ? reinterpret_cast<const half_t*>(at(os2)) : nullptr, nullptr,
                           reinterpret_cast<const half_t*>(at(oz0)), reinterpret_cast<const half_t*>(at(oz1)),
                           NL > 2 ? reinterpret_cast<const half_t*>(at(oz2)) : nullptr, nullptr,
                           tail.y[0], tail.y[1], NL > 2 ? tail.y[NL > 2 ? 2 : 0] : nullptr, nullptr,
                           static_cast<int>(nb1 >> 16), NL > 2 ? static_cast<int>(b2k & 0xFFFFu) : INT32_MAX,
                           INT32_MAX};
    gemv_body<BITS, MT, RPW, CPL, DEPTH, true, NW, NL>(reinterpret_cast<const half_t*>(at(ox)), nullptr, nullptr,
                                                        nullptr, nullptr, N, K, log2g, 1, nblocks, L);
}

}  // namespace

// INT4 rows of 2-4 items (4096 < K <= 16384) at M <= 4, with every row within
// one round of resident waves of the one-shot 8-wave instances (one row per
// wave; two blocks per CU at 2 items and M <= 3, one otherwise, by their
// registers: 97-102, 133-146 and 169-253 VGPRs). There every item in flight
// at once beats the persistent grid, whose few busy waves walk their rows
// through a 2-deep ring. Measured (us): M = 1 512 x 13824 7.12 -> 4.70,
// 2048 x 13824 7.41 -> 5.79, 4096 x 5120 4.99 -> 4.45, 512 x 11008
// 4.41 -> 3.94; M = 2 512 x 5120 5.71 -> 3.62, 512 x 11008 7.92 -> 5.21,
// 2048 x 13824 9.55 -> 7.14; M = 4 512 x 11008 11.39 -> 7.92, 1024 x 8192
// 8.36 -> 5.71. Past one round it loses (M = 1: 3072 x 13824 7.90 -> 9.46,
// 2560 x 11008 6.28 -> 7.09). Rows of more items would spill.
bool gemv_few_rows(int64_t M, int64_t N, int64_t K, int bits) {
    if (bits != 4 || M < 1 || M > 4 || N < 1) return false;
    const int64_t kbs = ceil_div(K >> 5, 128);
    return kbs >= 2 && kbs <= 4 && N <= 8 * cu_count() * (kbs == 2 && M <= 3 ? 2 : 1);
}

namespace {

// LDS bytes a block may take: the device's limit, or gfx950's 160 KB when no
// device can be queried (host-only kernel-choice queries)
int max_shared_bytes() {
    static int cached = -1;
    if (cached < 0) {
        int dev = 0, v = 160 * 1024;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess) {
            cached = v;
        } else {
            cached = 160 * 1024;
        }
    }
    return cached;
}

size_t gemv_lds_bytes(int64_t M, int64_t K, int bits) {
    return bits == 4 ? static_cast<size_t>(M) * static_cast<size_t>(K / 32) * 72
                     : static_cast<size_t>(M) * static_cast<size_t>(K / 16) * 40;
}

// A launch: one layer (qweight, scales, zeros, y of N rows), or with NL > 0
// the stacked layers of L (N rows in all).
template <int NL>
struct GemvTarget {
    const uint32_t* qweight;
    const half_t* scales;
    const half_t* zeros;
    half_t* y;
    LayersArg<NL> L;
};

// LDS of a streaming launch with its (scale, zero) pairs staged (SZL), or 0
// when that form does not apply: single layer, whole 16-byte pieces of
// pairs, 32-bit byte offsets, and one block per CU still fitting.
template <int BITS, int MT, int RPW, int NW>
size_t gemv_szl_lds_bytes(int64_t N, int64_t K, int log2g, int64_t blocks) {
    const int64_t ngroups = K >> log2g;
    const int64_t nchunk = K >> Chunk<BITS>::kShift;
    if ((N * ngroups) % 8 != 0 || (NW * RPW * ngroups) % 8 != 0 || N * ngroups * 2 >= (int64_t{1} << 31)) return 0;
    const int64_t sets = ceil_div(N, RPW);
    const int64_t max_sets = ceil_div(sets, blocks * NW);
    const int64_t words = gemv_sz_word_offset(MT, static_cast<int>(nchunk), Chunk<BITS>::kXV,
                                              static_cast<int>(NW * max_sets * RPW)) +
                          max_sets * NW * RPW * ngroups;
    const size_t bytes = static_cast<size_t>(words) * 4;
    return bytes <= static_cast<size_t>(max_shared_bytes()) ? bytes : 0;
}

template <int BITS, int MT, int RPW, int CPL, int DEPTH, bool ONESHOT = false, int NW = 4, int NL = 0,
          bool SZL = false>
awq_status launch_t(const half_t* x, const GemvTarget<NL>& tg, int64_t N, int64_t K, int log2g,
                    int64_t blocks, hipStream_t stream) {
    static_assert(!SZL || (!ONESHOT && NL == 0), "staged pairs: the single-layer streaming form");
    const void* kern;
    if constexpr (NL > 0)
        kern = reinterpret_cast<const void*>(&gemv_grouped_kernel<BITS, MT, RPW, CPL, DEPTH, ONESHOT, NW, NL>);
    else
        kern = reinterpret_cast<const void*>(&gemv_kernel<BITS, MT, RPW, CPL, DEPTH, ONESHOT, NW, SZL>);
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, max_shared_bytes()) != hipSuccess)
            return AWQ_ERR_HIP;
        attr_set = true;
    }
    const int64_t sets = ceil_div(N, RPW);
    blocks = std::max<int64_t>(1, std::min<int64_t>(blocks, ceil_div(sets, NW)));
    const int64_t max_sets = ceil_div(sets, blocks * NW);
    const int64_t nchunk = K >> Chunk<BITS>::kShift;
    if (ONESHOT && max_sets * ceil_div(nchunk, 64 * CPL) > DEPTH) return AWQ_ERR_SHAPE;   // launch-shape bug
    if (max_sets >= (int64_t{1} << 23)) return AWQ_ERR_SHAPE;                              // packed with log2 G
    size_t lds = gemv_lds_bytes(MT, K, BITS) + (ONESHOT ? 0 : static_cast<size_t>(NW * max_sets * RPW * MT) * sizeof(float));
    if constexpr (SZL) {
        lds = gemv_szl_lds_bytes<BITS, MT, RPW, NW>(N, K, log2g, blocks);
        if (lds == 0) return AWQ_ERR_SHAPE;   // launch-shape bug: the caller checks
    }
    if (lds > static_cast<size_t>(max_shared_bytes())) return AWQ_ERR_SHAPE;
    if constexpr (NL > 0) {
        const GemvLayerTable& T = tg.L;
        if constexpr (ONESHOT && (NL == 2 || NL == 3)) {
            // the packed-offset entry when every early pointer is 16-byte
            // aligned, within 64 GB of the lowest, and the sizes fit their fields
            const void* ptrs[10] = {x, T.q0, T.q1, T.s0, T.s1, T.z0, T.z1, NL > 2 ? T.q2 : T.q0,
                                    NL > 2 ? T.s2 : T.s0, NL > 2 ? T.z2 : T.z0};
            uintptr_t lo = UINTPTR_MAX, hi = 0, bits = 0;
            for (const void* p : ptrs) {
                lo = std::min(lo, reinterpret_cast<uintptr_t>(p));
                hi = std::max(hi, reinterpret_cast<uintptr_t>(p));
                bits |= reinterpret_cast<uintptr_t>(p);
            }
            const int64_t nsets = ceil_div(N, RPW);
            if ((bits & 15) == 0 && (hi - lo) >> 4 < (uintptr_t{1} << 32) && N < 65536 && (K >> 5) < 4096 && log2g >= 5 && log2g < 21 &&
                blocks == ceil_div(nsets, NW) && max_sets == 1) {
                const char* base = reinterpret_cast<const char*>(lo);
                auto off = [&](const void* p) {
                    return static_cast<uint32_t>((reinterpret_cast<uintptr_t>(p) - lo) >> 4);
                };
                static bool packed_attr_set = false;
                if (!packed_attr_set) {
                    if (hipFuncSetAttribute(
                            reinterpret_cast<const void*>(&gemv_grouped_packed_kernel<BITS, MT, RPW, CPL, DEPTH, NW, NL>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, max_shared_bytes()) != hipSuccess)
                        return AWQ_ERR_HIP;
                    packed_attr_set = true;
                }
                GemvOutTail<NL> ytail;
                ytail.y[0] = T.y0;
                ytail.y[1] = T.y1;
                if constexpr (NL > 2) ytail.y[2] = T.y2;
                const uint32_t nb1 = static_cast<uint32_t>(N) | (static_cast<uint32_t>(T.b1) << 16);
                const uint32_t b2k = (NL > 2 ? static_cast<uint32_t>(T.b2) : 0u) |
                                     (static_cast<uint32_t>(K >> 5) << 16) | (static_cast<uint32_t>(log2g - 5) << 28);
                hipLaunchKernelGGL((gemv_grouped_packed_kernel<BITS, MT, RPW, CPL, DEPTH, NW, NL>),
                                   dim3(static_cast<unsigned>(blocks)), dim3(NW * 64), lds, stream, base, off(x),
                                   off(T.q0), off(T.q1), off(ptrs[7]), off(T.s0), off(T.s1), off(ptrs[8]), off(T.z0),
                                   off(T.z1), off(ptrs[9]), nb1, b2k, ytail);
                return last_launch_status();
            }
        }
        GemvLayerTail<NL> tail;
        const half_t* sc[4] = {T.s0, T.s1, T.s2, T.s3};
        const half_t* zr[4] = {T.z0, T.z1, T.z2, T.z3};
        half_t* yy[4] = {T.y0, T.y1, T.y2, T.y3};
        for (int i = 0; i < NL; ++i) {
            tail.scales[i] = sc[i];
            tail.zeros[i] = zr[i];
            tail.y[i] = yy[i];
        }
        hipLaunchKernelGGL((gemv_grouped_kernel<BITS, MT, RPW, CPL, DEPTH, ONESHOT, NW, NL>),
                           dim3(static_cast<unsigned>(blocks)), dim3(NW * 64), lds, stream, x, static_cast<int>(N),
                           static_cast<int>(K), log2g | static_cast<int>(max_sets << 8), static_cast<int>(blocks),
                           T.q0, T.q1, T.q2, T.b1, T.b2, T.q3, T.b3, tail);
    }
    else
        hipLaunchKernelGGL((gemv_kernel<BITS, MT, RPW, CPL, DEPTH, ONESHOT, NW, SZL>), dim3(static_cast<unsigned>(blocks)),
                           dim3(NW * 64), lds, stream, x, tg.qweight, tg.scales, tg.zeros, tg.y, static_cast<int>(N),
                           static_cast<int>(K), log2g | static_cast<int>(max_sets << 8), static_cast<int>(blocks));
    return last_launch_status();
}

// Launch shape. Items are RPW rows x 2 chunks (64 packed words) per lane.
//  * Rows of one item (4096 weights), or of two for W8: one row set per
//    wavefront and all of it in flight from the start; 2 rows per wave share
//    each staged x read, as long as that leaves >= 512 blocks. With two or
//    more activation rows, every weight costs one LDS read of x per row, so
//    4 weight rows per wave share each read (2 in the streaming form):
//    M = 4 on 11008 x 4096 takes 12.5 us against 14.4 us with 2.
//  * Longer rows, and INT4 rows of 2 items (13824 x 5120: M = 1 11.5 ->
//    11.0 us, M = 4 32.9 -> 21.8 us; 11008 x 8192, M = 1: 11.7 -> 10.8 us;
//    W8 rows of 2 items are faster one-shot): a persistent grid of one
//    8-wave block per CU, so that
//    staging x (2 bytes per input channel per block) stays small against the
//    weights while two waves per SIMD hide each other's unpack latency, each
//    wave streaming its rows through a 2-deep ring, 2 rows at a time for rows
//    of more than 3 items. Against 4 waves with a 4-deep ring (the same bytes
//    in flight): 4096 x 11008 7.85 -> 7.13 us, 8192 x 28672 25.4 -> 24.1 us;
//    8 waves with a 4-deep ring or 16 waves with a 2-deep one are slower.
//  * Except INT4 rows of 2-4 items at M <= 4 when all rows fit in one round
//    of resident waves (layers of few rows, such as one GPU's share of a
//    split layer): one-shot 8-wave blocks, one row per wave, every item in
//    flight (gemv_few_rows).
template <int BITS, int MT, int NL = 0>
awq_status launch_m(const half_t* x, const GemvTarget<NL>& tg, int64_t N, int64_t K, int log2g,
                    hipStream_t stream) {
    const int64_t kbs = ceil_div(K >> Chunk<BITS>::kShift, 128);
    if (kbs == 1) {
        if (MT >= 2 && ceil_div(N, 16) >= 256)
            return launch_t<BITS, MT, 4, 2, 1, true, 4, NL>(x, tg, N, K, log2g, ceil_div(N, 16), stream);
        if (ceil_div(N, 8) >= 512)
            return launch_t<BITS, MT, 2, 2, 1, true, 4, NL>(x, tg, N, K, log2g, ceil_div(N, 8), stream);
        return launch_t<BITS, MT, 1, 2, 1, true, 4, NL>(x, tg, N, K, log2g, ceil_div(N, 4), stream);
    }
    if (kbs == 2 && BITS == 8)
        return launch_t<BITS, MT, 1, 2, 2, true, 4, NL>(x, tg, N, K, log2g, ceil_div(N, 4), stream);
    // Layers of few rows (gemv_few_rows): one-shot 8-wave blocks.
    if constexpr (BITS == 4 && MT <= 4) {
        if (gemv_few_rows(MT, N, K, BITS)) {
            if (kbs == 2) return launch_t<BITS, MT, 1, 2, 2, true, 8, NL>(x, tg, N, K, log2g, ceil_div(N, 8), stream);
            if (kbs == 3) return launch_t<BITS, MT, 1, 2, 3, true, 8, NL>(x, tg, N, K, log2g, ceil_div(N, 8), stream);
            return launch_t<BITS, MT, 1, 2, 4, true, 8, NL>(x, tg, N, K, log2g, ceil_div(N, 8), stream);
        }
    }
    const int64_t x_lds = static_cast<int64_t>(gemv_lds_bytes(MT, K, BITS));
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(kGemvBlocksPerCu, max_shared_bytes() / (x_lds + 2048)));
    const int64_t blocks = per_cu * cu_count();
    // Rows per wave. Two rows per item share every x read from LDS, and a
    // wave's two rows are in flight together; one row per wave balances
    // better when it gives the busiest wave fewer rows (5120 rows over 2048
    // waves: 3 rows against 2 sets of 2). Measured in one process (us,
    // graph-timed, weights rotated, outputs bit-identical), two rows against
    // one: M = 1 5120 x 13824 11.84 -> 9.94, 6144 x 16384 12.96 -> 11.29;
    // M = 2 5120 x 13824 15.22 -> 13.10; with equal busiest waves two rows
    // stay ahead or level: M = 2 8192 x 28672 26.55 against 28.68, 11008 x
    // 8192 12.54 against 13.04, M = 1 2560 x 28672 (G = 64) 11.38 against
    // 12.43. At M >= 3 two rows always.
    const int64_t waves = blocks * 8;
    const bool one_row = MT == 1 ? (kbs <= 3 || ceil_div(N, waves) < 2 * ceil_div(ceil_div(N, 2), waves))
                                 : MT == 2 && ceil_div(N, waves) < 2 * ceil_div(ceil_div(N, 2), waves);
    // Staged (scale, zero) pairs (SZL): at M = 1 on rows of 5 items and
    // more, and at M = 2 with two rows per wave. Measured against per-chunk
    // pairs (us, as above): M = 2 4096 x 11008 9.37 -> 8.95, 8192 x 28672
    // 27.26 -> 26.59; M = 1 8192 x 28672 23.76 -> 23.43 (G = 64: 24.88 ->
    // 24.53). Shorter rows at M = 1 lose to the staging ahead of the first
    // item: 4096 x 11008 6.69 -> 6.85, 13824 x 5120 10.68 -> 10.83, 11008 x
    // 8192 10.29 -> 10.45; so does one row per wave at M = 2 (5120 x 13824
    // 13.10 -> 13.30, 13824 x 5120 13.84 -> 14.48).
    const bool szl = NL == 0 && MT <= 2 && per_cu == 1 && (MT == 1 ? kbs >= 5 : !one_row);
    if (!one_row) {
        if constexpr (NL == 0 && MT <= 2)
            if (szl && gemv_szl_lds_bytes<BITS, MT, 2, 8>(N, K, log2g, blocks) != 0)
                return launch_t<BITS, MT, 2, 2, 2, false, 8, NL, true>(x, tg, N, K, log2g, blocks, stream);
        return launch_t<BITS, MT, 2, 2, 2, false, 8, NL>(x, tg, N, K, log2g, blocks, stream);
    }
    if constexpr (NL == 0 && MT <= 2)
        if (szl && gemv_szl_lds_bytes<BITS, MT, 1, 8>(N, K, log2g, blocks) != 0)
            return launch_t<BITS, MT, 1, 2, 2, false, 8, NL, true>(x, tg, N, K, log2g, blocks, stream);
    return launch_t<BITS, MT, 1, 2, 2, false, 8, NL>(x, tg, N, K, log2g, blocks, stream);
}

}  // namespace

bool gemv_supported(int64_t M, int64_t K, int bits) {
    if (M < 1 || M > kGemvMaxM) return false;
    if (K % (bits == 4 ? 32 : 16) != 0 || K > (int64_t(1) << 30)) return false;
    return gemv_lds_bytes(M, K, bits) <= static_cast<size_t>(max_shared_bytes());
}

namespace {
template <int BITS>
awq_status launch_gemv_bits(const half_t* x, const uint32_t* qweight, const half_t* scales, const half_t* zeros,
                            int64_t M, int64_t N, int64_t K, int log2g, half_t* y, hipStream_t stream) {
    const GemvTarget<0> tg{qweight, scales, zeros, y, NoLayers{}};
    switch (M) {
        case 1: return launch_m<BITS, 1>(x, tg, N, K, log2g, stream);
        case 2: return launch_m<BITS, 2>(x, tg, N, K, log2g, stream);
        case 3: return launch_m<BITS, 3>(x, tg, N, K, log2g, stream);
        case 4: return launch_m<BITS, 4>(x, tg, N, K, log2g, stream);
        case 5: return launch_m<BITS, 5>(x, tg, N, K, log2g, stream);
        case 6: return launch_m<BITS, 6>(x, tg, N, K, log2g, stream);
        case 7: return launch_m<BITS, 7>(x, tg, N, K, log2g, stream);
        case 8: return launch_m<BITS, 8>(x, tg, N, K, log2g, stream);
        default: return AWQ_ERR_SHAPE;
    }
}
}  // namespace

awq_status launch_gemv(const half_t* x, const uint32_t* qweight, const half_t* scales,
                       const half_t* zeros, int64_t M, int64_t N, int64_t K, int group_size,
                       half_t* y, hipStream_t stream, int bits) {
    const int log2g = 31 - __builtin_clz(static_cast<unsigned>(group_size));   // G is a power of two >= 32
    if (bits == 8) return launch_gemv_bits<8>(x, qweight, scales, zeros, M, N, K, log2g, y, stream);
    return launch_gemv_bits<4>(x, qweight, scales, zeros, M, N, K, log2g, y, stream);
}

namespace {
template <int NL>
awq_status launch_grouped_n(const half_t* x, const GemvLayers& layers, int64_t M, int64_t K, int log2g,
                            hipStream_t stream) {
    auto at = [&](auto a, int i) { return i < layers.n ? a[i] : nullptr; };
    const GemvLayerTable T{at(layers.qweight, 0), at(layers.qweight, 1), at(layers.qweight, 2), at(layers.qweight, 3),
                           at(layers.scales, 0),  at(layers.scales, 1),  at(layers.scales, 2),  at(layers.scales, 3),
                           at(layers.zeros, 0),   at(layers.zeros, 1),   at(layers.zeros, 2),   at(layers.zeros, 3),
                           at(layers.y, 0),       at(layers.y, 1),       at(layers.y, 2),       at(layers.y, 3),
                           layers.n > 1 ? layers.row0[1] : INT32_MAX, layers.n > 2 ? layers.row0[2] : INT32_MAX,
                           layers.n > 3 ? layers.row0[3] : INT32_MAX};
    const GemvTarget<NL> tg{nullptr, nullptr, nullptr, nullptr, T};
    const int64_t N = layers.row0[NL];
    switch (M) {
        case 1: return launch_m<4, 1, NL>(x, tg, N, K, log2g, stream);
        case 2: return launch_m<4, 2, NL>(x, tg, N, K, log2g, stream);
        default: return AWQ_ERR_SHAPE;
    }
}
}  // namespace

awq_status launch_gemv_grouped(const half_t* x, const GemvLayers& layers, int64_t M, int64_t K, int group_size,
                               hipStream_t stream) {
    const int log2g = 31 - __builtin_clz(static_cast<unsigned>(group_size));
    switch (layers.n) {
        case 1:
            return launch_gemv(x, layers.qweight[0], layers.scales[0], layers.zeros[0], M, layers.row0[1], K,
                               group_size, layers.y[0], stream);
        case 2: return launch_grouped_n<2>(x, layers, M, K, log2g, stream);
        case 3: return launch_grouped_n<3>(x, layers, M, K, log2g, stream);
        case 4: return launch_grouped_n<4>(x, layers, M, K, log2g, stream);
        default: return AWQ_ERR_CONFIG;
    }
}

}  // namespace awq
