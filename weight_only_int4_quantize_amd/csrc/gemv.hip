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

// Issues the loads of one item: RPW rows x CPL chunks per lane (chunk
// c = base + lane + 64 j), with each chunk's scale and zero-point. Rows past
// N or items past the wave's last (valid == false) read as zero.
template <int BITS, int RPW, int CPL>
__device__ inline void load_batch(WeightBatch<RPW, CPL>& b, const uint32_t* __restrict__ qweight,
                                  const half_t* __restrict__ scales, const half_t* __restrict__ zeros,
                                  int row0, bool valid, int N, int nchunk, int ngroups, int log2g, int base,
                                  int lane) {
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
            b.s[i][j] = __builtin_amdgcn_raw_buffer_load_b16(rs, g * 2, 0, 0);
            b.z[i][j] = __builtin_amdgcn_raw_buffer_load_b16(rz, g * 2, 0, 0);
        }
    }
}

// Consumes one item: chunks past the row end have scale 0 (zero-filled
// loads) and read a clamped, in-range slot of the staged x.
template <int BITS, int MT, int RPW, int CPL>
__device__ inline void compute_batch(const WeightBatch<RPW, CPL>& b, const uint4* __restrict__ xp,
                                     const float2* __restrict__ xo, float (&acc)[RPW][MT], int nchunk,
                                     int base, int lane, const UnpackConsts& k) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = min(base + lane + 64 * j, nchunk - 1);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4* pp = xp + (m * nchunk + c) * Chunk<BITS>::kXV;
            const float2 o = xo[m * nchunk + c];
            uint4 p[Chunk<BITS>::kXV];
#pragma unroll
            for (int v = 0; v < Chunk<BITS>::kXV; ++v) p[v] = pp[v];
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
                const float s = static_cast<float>(__builtin_bit_cast(half_t, b.s[i][j]));
                const float z = static_cast<float>(__builtin_bit_cast(half_t, b.z[i][j]));
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
template <int BITS, int MT, int RPW, int CPL, int DEPTH, bool ONESHOT, int NW>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(const half_t* __restrict__ x,
                                                   const uint32_t* __restrict__ qweight,
                                                   const half_t* __restrict__ scales,
                                                   const half_t* __restrict__ zeros,
                                                   half_t* __restrict__ y, int N, int K,
                                                   int log2g, int max_sets) {
    extern __shared__ uint4 smem[];
    constexpr int XV = Chunk<BITS>::kXV;
    const int nchunk = K >> Chunk<BITS>::kShift;    // 32 (INT4) or 16 (W8) weights per chunk
    uint4* xp = smem;                               // [MT][nchunk][XV] x pairs
    float2* xo = reinterpret_cast<float2*>(smem + MT * nchunk * XV);  // [MT][nchunk] (off, xs)
    float* yl = reinterpret_cast<float*>(xo + MT * nchunk);          // [NW][max_sets][RPW][MT]

    // wave index as a scalar: the buffer descriptors built from it must be
    // wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ngroups = K >> log2g;

    const int kbs = (nchunk + 64 * CPL - 1) / (64 * CPL);      // k-batches per row
    const int nsets = (N + RPW - 1) / RPW;                      // row sets
    const int W = gridDim.x * NW;
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
                xp[(m * nchunk + c) * XV + j] = p;
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

    WeightBatch<RPW, CPL> ring[DEPTH];
    int l_item = 0, l_set = 0, l_kb = 0;            // load cursor
    auto issue = [&](WeightBatch<RPW, CPL>& b) {
        load_batch<BITS>(b, qweight, scales, zeros, (wid + l_set * W) * RPW, l_item < n_items, N, nchunk, ngroups,
                   log2g, l_kb * 64 * CPL, lane);
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
    __syncthreads();

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
                compute_batch<BITS>(ring[d], xp, xo, acc, nchunk, c_kb * 64 * CPL, lane, uk);
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
                                if (lane == 63 && r0 + i < N)
                                    y[static_cast<int64_t>(m) * N + r0 + i] = static_cast<half_t>(v);
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
            for (int m = 0; m < MT; ++m)
                y[static_cast<int64_t>(m) * N + row] = static_cast<half_t>(yl[sl * MT + m]);
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

size_t gemv_lds_bytes(int64_t M, int64_t K, int bits) {
    return bits == 4 ? static_cast<size_t>(M) * static_cast<size_t>(K / 32) * 72
                     : static_cast<size_t>(M) * static_cast<size_t>(K / 16) * 40;
}

template <int BITS, int MT, int RPW, int CPL, int DEPTH, bool ONESHOT = false, int NW = 4>
awq_status launch_t(const half_t* x, const uint32_t* qweight, const half_t* scales,
                    const half_t* zeros, int64_t N, int64_t K, int log2g, half_t* y,
                    int64_t blocks, hipStream_t stream) {
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<BITS, MT, RPW, CPL, DEPTH, ONESHOT, NW>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, max_shared_bytes()) != hipSuccess)
            return AWQ_ERR_HIP;
        attr_set = true;
    }
    const int64_t sets = ceil_div(N, RPW);
    blocks = std::max<int64_t>(1, std::min<int64_t>(blocks, ceil_div(sets, NW)));
    const int64_t max_sets = ceil_div(sets, blocks * NW);
    const int64_t nchunk = K >> Chunk<BITS>::kShift;
    if (ONESHOT && max_sets * ceil_div(nchunk, 64 * CPL) > DEPTH) return AWQ_ERR_SHAPE;   // launch-shape bug
    const size_t lds = gemv_lds_bytes(MT, K, BITS) + (ONESHOT ? 0 : static_cast<size_t>(NW * max_sets * RPW * MT) * sizeof(float));
    if (lds > static_cast<size_t>(max_shared_bytes())) return AWQ_ERR_SHAPE;
    hipLaunchKernelGGL((gemv_kernel<BITS, MT, RPW, CPL, DEPTH, ONESHOT, NW>), dim3(static_cast<unsigned>(blocks)), dim3(NW * 64), lds,
                       stream, x, qweight, scales, zeros, y, static_cast<int>(N), static_cast<int>(K),
                       log2g, static_cast<int>(max_sets));
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
template <int BITS, int MT>
awq_status launch_m(const half_t* x, const uint32_t* qweight, const half_t* scales,
                    const half_t* zeros, int64_t N, int64_t K, int log2g, half_t* y,
                    hipStream_t stream) {
    const int64_t kbs = ceil_div(K >> Chunk<BITS>::kShift, 128);
    if (kbs == 1) {
        if (MT >= 2 && ceil_div(N, 16) >= 256)
            return launch_t<BITS, MT, 4, 2, 1, true>(x, qweight, scales, zeros, N, K, log2g, y, ceil_div(N, 16),
                                                     stream);
        if (ceil_div(N, 8) >= 512)
            return launch_t<BITS, MT, 2, 2, 1, true>(x, qweight, scales, zeros, N, K, log2g, y, ceil_div(N, 8),
                                                     stream);
        return launch_t<BITS, MT, 1, 2, 1, true>(x, qweight, scales, zeros, N, K, log2g, y, ceil_div(N, 4), stream);
    }
    if (kbs == 2 && BITS == 8)
        return launch_t<BITS, MT, 1, 2, 2, true>(x, qweight, scales, zeros, N, K, log2g, y, ceil_div(N, 4), stream);
    const int64_t x_lds = static_cast<int64_t>(gemv_lds_bytes(MT, K, BITS));
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(kGemvBlocksPerCu, max_shared_bytes() / (x_lds + 2048)));
    if (MT >= 2 || kbs > 3)
        return launch_t<BITS, MT, 2, 2, 2, false, 8>(x, qweight, scales, zeros, N, K, log2g, y, per_cu * cu_count(),
                                                     stream);
    return launch_t<BITS, MT, 1, 2, 2, false, 8>(x, qweight, scales, zeros, N, K, log2g, y, per_cu * cu_count(), stream);
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
    switch (M) {
        case 1: return launch_m<BITS, 1>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 2: return launch_m<BITS, 2>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 3: return launch_m<BITS, 3>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 4: return launch_m<BITS, 4>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 5: return launch_m<BITS, 5>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 6: return launch_m<BITS, 6>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 7: return launch_m<BITS, 7>(x, qweight, scales, zeros, N, K, log2g, y, stream);
        case 8: return launch_m<BITS, 8>(x, qweight, scales, zeros, N, K, log2g, y, stream);
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

}  // namespace awq
