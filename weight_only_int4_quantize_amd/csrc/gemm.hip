// Prefill GEMM of the W4A16 linear layer on the fp16 matrix cores
// (the batched "GEMM" kernel choice of the rskf.cn AWQ article, §3.3, with
// the INT4 dequantization inside the matmul of §1.3), plus the two variants
// the scale search runs on the same core: an fp16-B product for the
// unquantized reference W . x^T and a fused squared-error epilogue.
//
// Exactness: the dequantized weight (q - z) * s has up to 15 significant bits,
// more than fp16 holds, and rounding it before the MFMA costs up to ~2e-2
// absolute on outputs fed by salient channels. So the B operand is the exact
// integer (q - z) in fp16, and the group's scale is applied in fp32 to the
// accumulator, which is kept in units of the current group's scale:
// C' = C / s_g. Crossing into group g + 1 multiplies C' by s_g / s_{g+1}
// (one v_mul per accumulator element per group); the end multiplies by the
// last scale. Each step rounds once in fp32, ~1e-7 relative per group.
//
// Two forms share the epilogues and the scheduling below.
//  * Direct-B form (quantized B with G >= 64, the default): a block owns a
//    256 x 128 tile (4 waves, 2 blocks per CU) or a 256 x 256 tile (8 waves,
//    1 per CU); each wave owns 256 x 32 outputs as 8 accumulators. K moves
//    in steps of 64. Each lane loads its column's packed words for the
//    step straight into registers in MFMA operand order and dequantizes
//    them there; only A goes through LDS, by LDS-DMA loads (see
//    run_segment_direct).
//  * The fp16-B reference of the searches runs the direct form too, its
//    B columns loaded as 4 16-byte pieces per lane and step, already fp16.
//  * Older form (G = 32, and the fp16-B reference when K is not a multiple
//    of 64):
//    a 256-thread block owns a 256 x 128 tile, 4 wavefronts in a 2 x 2
//    arrangement, each with 128 x 64 outputs as 4 x 2
//    v_mfma_f32_32x32x16_f16 accumulators (128 VGPRs), so every 16-byte
//    fragment read from LDS feeds 2-4 MFMAs. K advances in steps of BK = 32.
//    A (fp16) moves global -> registers -> LDS; B (packed INT4) is read as
//    raw words, turned into exact fp16 (q - z) once per block and written
//    to LDS in natural k order (the fp16-B variant copies W). The next
//    step's global loads are in flight while the current step's MFMAs run
//    (two LDS stages, 60 KB, so two blocks fit on a CU);
//  * LDS rows are 64 bytes with an XOR swizzle of their four 16-byte chunks
//    (see swz), so fragment reads and staging writes are bank-conflict free;
//  * blocks are dealt to the 8 XCDs round-robin by the dispatcher; the tile
//    order is remapped so each XCD works through a contiguous, m-major range
//    of tiles and keeps the shared A rows in its own L2.
// MFMA operand layout (32x32x16 f16): lane l supplies row (l mod 32) of A and
// column (l mod 32) of B, with k-slice 8 * (l / 32) .. +7 of the 16; the
// accumulator element i of lane l is C[8 * (i / 4) + 4 * (l / 32) + i mod 4]
// [l mod 32].
#include <algorithm>

#include "awq_internal.h"

namespace awq {
namespace {

constexpr int BK = 32;
constexpr int LDK = BK;              // LDS row (halves): 64 bytes, 4 chunks of 16 bytes

// gfx950 LDS: 64 banks of 4 bytes; a 16-byte-per-lane access is served 16
// lanes at a time, which is conflict-free when those 16 lanes hit 16 distinct
// 16-byte slots modulo 256 bytes. 16-byte chunk c of LDS row r is stored at
// chunk position c ^ ((r >> 2) & 3): the fragment reads (16 consecutive rows,
// one chunk), the A stores (4 rows x 4 chunks) and the B stores (8 rows x 2
// chunks) then each cover all 64 banks once.
__device__ __forceinline__ int swz(int r, int c) { return r * LDK + ((c ^ ((r >> 2) & 3)) << 3); }
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// Direct-B form (INT4 B, G >= 64): K steps of 64, A rows in LDS of 128 bytes
// (eight 16-byte chunks). Chunk c of row r is stored at c ^ ((r >> 1) & 7):
// 16 lanes reading one chunk of 16 consecutive rows, or writing the 8 chunks
// of 2 rows, then hit 16 distinct 16-byte slots of the 256-byte bank window.
constexpr int BKD = 64;
__device__ __forceinline__ int swz64(int r, int c) { return r * BKD + ((c ^ ((r >> 1) & 7)) << 3); }
// 16-byte load from global memory straight into LDS: lane L's bytes land at
// lds + 16 L (lds is wave-uniform). The builtin exists only in the device pass.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, half_t* lds, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#else
    (void)rs, (void)lds, (void)voff, (void)soff;
#endif
}
// A zero group scale would make the rescale ratio infinite; it is taken as
// the smallest positive fp16 value instead.
constexpr float kTinyScale = 5.9604645e-08f;

__device__ inline half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ inline uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

struct UnpackConsts {
    uint32_t lo_mask, hi_mask, lo_magic, hi_magic;
};
// Held in VGPRs so each (w & mask) | magic is one v_and_or_b32 (gfx9 VOP3
// takes no 32-bit literal and one SGPR at most).
__device__ inline UnpackConsts unpack_consts() {
    UnpackConsts k{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
    asm volatile("" : "+v"(k.lo_mask), "+v"(k.hi_mask), "+v"(k.lo_magic), "+v"(k.hi_magic));
    return k;
}

// One packed word (codes k0..k7) -> 8 exact fp16 values (q - z), natural k
// order, as 4 packed pairs. zc_hi = 1024 + z, zc_lo = 64 + z (both exact).
__device__ inline uint4 unpack_word(uint32_t wq, half2_t zc_hi, half2_t zc_lo, const UnpackConsts& k) {
    const uint32_t w8 = wq >> 8;
    // OR-ing a nibble into an fp16 mantissa gives an exact integer:
    // (1024 + q0, 1024 + q4), (64 + q1, 64 + q5), (1024 + q2, 1024 + q6), (64 + q3, 64 + q7)
    const half2_t a = as_h2((wq & k.lo_mask) | k.lo_magic) - zc_hi;
    const half2_t b = as_h2((wq & k.hi_mask) | k.hi_magic) - zc_lo;
    const half2_t c = as_h2((w8 & k.lo_mask) | k.lo_magic) - zc_hi;
    const half2_t d = as_h2((w8 & k.hi_mask) | k.hi_magic) - zc_lo;
    const uint32_t ua = as_u32(a), ub = as_u32(b), uc = as_u32(c), ud = as_u32(d);
    // v_perm_b32 picks bytes of {hi: first, lo: second operand}: 0x05040100
    // joins the low halves, 0x07060302 the high halves
    uint4 r;
    r.x = __builtin_amdgcn_perm(ub, ua, 0x05040100u);   // (k0, k1)
    r.y = __builtin_amdgcn_perm(ud, uc, 0x05040100u);   // (k2, k3)
    r.z = __builtin_amdgcn_perm(ub, ua, 0x07060302u);   // (k4, k5)
    r.w = __builtin_amdgcn_perm(ud, uc, 0x07060302u);   // (k6, k7)
    return r;
}

// Two W8 words (byte codes k0..k7) -> 8 exact fp16 values (b - z), natural k
// order. zc = 1024 + z (exact): (w & 0x00FF00FF) | 0x64006400 is
// (1024 + b0, 1024 + b2), the same on w >> 8 gives (1024 + b1, 1024 + b3).
__device__ inline uint4 unpack_bytes(uint32_t w0, uint32_t w1, half2_t zc) {
    const uint32_t mask = 0x00FF00FFu, magic = 0x64006400u;
    const uint32_t a0 = as_u32(as_h2((w0 & mask) | magic) - zc), b0 = as_u32(as_h2(((w0 >> 8) & mask) | magic) - zc);
    const uint32_t a1 = as_u32(as_h2((w1 & mask) | magic) - zc), b1 = as_u32(as_h2(((w1 >> 8) & mask) | magic) - zc);
    uint4 r;
    r.x = __builtin_amdgcn_perm(b0, a0, 0x05040100u);   // (k0, k1)
    r.y = __builtin_amdgcn_perm(b0, a0, 0x07060302u);   // (k2, k3)
    r.z = __builtin_amdgcn_perm(b1, a1, 0x05040100u);   // (k4, k5)
    r.w = __builtin_amdgcn_perm(b1, a1, 0x07060302u);   // (k6, k7)
    return r;
}

// Registers carrying one K step from global memory to LDS.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Registers carrying one K step from global memory to LDS (native vector
// types, which the compiler keeps in registers).
template <int A_VECS, int B_VECS>
struct Stage {
    u32x4 a[A_VECS];
    u32x4 b[B_VECS];      // fp16 B
    u32x2 braw;           // int4 B: 16 codes
    half_t bz;            // int4 B: their zero-point
};

// column (in halves) of the 16-byte A/B chunk a thread stages
__device__ __forceinline__ int c8_of(int tid) { return (tid % (BK / 8)) * 8; }

template <bool INT4, int A_VECS, int B_VECS>
__device__ __forceinline__ void load_stage(Stage<A_VECS, B_VECS>& st, const half_t* a_base, const int (&a_row)[A_VECS],
                                           int K, const uint32_t* b_words, const half_t* b_zeros, int G,
                                           const half_t* w_base, const int (&b_row)[B_VECS], int k0) {
#pragma unroll
    for (int i = 0; i < A_VECS; ++i)
        st.a[i] = *reinterpret_cast<const u32x4*>(a_base + static_cast<int64_t>(a_row[i]) * K + k0);
    if constexpr (INT4) {
        st.braw = *reinterpret_cast<const u32x2*>(b_words + k0 / 8);
        st.bz = b_zeros[k0 / G];
    } else {
#pragma unroll
        for (int i = 0; i < B_VECS; ++i)
            st.b[i] = *reinterpret_cast<const u32x4*>(w_base + static_cast<int64_t>(b_row[i]) * K + k0);
    }
}

template <bool INT4, int BM, int BN, int A_VECS, int B_VECS>
__device__ __forceinline__ void store_stage(const Stage<A_VECS, B_VECS>& st, half_t* as, half_t* bs, int tid,
                                            int b_row, int b_half, const UnpackConsts& uk) {
#pragma unroll
    for (int i = 0; i < A_VECS; ++i) {
        const int idx = tid + i * kThreads;
        *reinterpret_cast<u32x4*>(&as[swz(idx / (BK / 8), idx % (BK / 8))]) = st.a[i];
    }
    if constexpr (INT4) {
        const half_t zh = static_cast<half_t>(1024.0f) + st.bz;   // exact
        const half_t zl = static_cast<half_t>(64.0f) + st.bz;     // exact
        const half2_t zc_hi{zh, zh}, zc_lo{zl, zl};
        *reinterpret_cast<uint4*>(&bs[swz(b_row, b_half * 2)]) = unpack_word(st.braw.x, zc_hi, zc_lo, uk);
        *reinterpret_cast<uint4*>(&bs[swz(b_row, b_half * 2 + 1)]) = unpack_word(st.braw.y, zc_hi, zc_lo, uk);
    } else {
#pragma unroll
        for (int i = 0; i < B_VECS; ++i) {
            const int idx = tid + i * kThreads;
            *reinterpret_cast<u32x4*>(&bs[swz(idx / (BK / 8), idx % (BK / 8))]) = st.b[i];
        }
    }
}

// Block index -> tile index: XCD x (= block mod 8) gets a contiguous range.
__device__ inline int xcd_tile(int block, int tiles) {
    const int q = tiles / kXcds, r = tiles % kXcds;
    const int x = block % kXcds, local = block / kXcds;
    return x * q + min(x, r) + local;
}

// Stream-K bookkeeping. Work unit u = (tile t, K step k) = t * ipt + k, with
// total = tiles * ipt < 2^31 units split evenly over `grid` blocks: block b
// owns [start(b), start(b + 1)), start(b) = b * q + min(b, r) where
// total = q * grid + r, i.e. the first r blocks take q + 1 units.
struct StreamK {
    float* partials = nullptr;   // [grid][2][BM * BN] fp32
    int* counters = nullptr;     // [tiles], zero between launches
    int total = 0;               // split tiles * ipt
    int ipt = 0;                 // K steps per tile
    int grid = 0;                // blocks over the split tiles
    int q = 0, r = 0;            // total = q * grid + r, q >= 1
    int dp_tiles = 0;            // tiles [0, dp_tiles) go whole to the first dp_tiles blocks
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int sk_start(const StreamK& sk, int b) { return b * sk.q + min(b, sk.r); }
// block whose range contains unit u
__device__ __forceinline__ int sk_block_of(const StreamK& sk, int u) {
    const int big = sk.r * (sk.q + 1);
    return u < big ? u / (sk.q + 1) : sk.r + (u - big) / sk.q;
}

constexpr int kSc1 = 16;   // cache-policy bit sc1 of buffer loads/stores (device scope)

// buffer descriptor over one BM x BN fp32 partial tile
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(float* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, bytes, 0x00020000);
}

// DIRECT (INT4 B with G >= 64 only): each wave reads its own B columns'
// packed words straight into registers in the MFMA operand order and
// dequantizes them there; only A goes through LDS.
//
// WGM: waves along M (the 4 waves form WGM x 4 / WGM).
// TILEDB (INT4 or fp16 B, the direct form's one-column-tile waves): B in
// the tiled order of GemmArgs::b_tiled, so each wave's load of a K step is
// one contiguous 1 KB piece per 16 bytes a lane takes (8 cache lines against
// 32 for row-major B).
template <int BM, int BN, GemmB BMODE, GemmOut OMODE, bool STREAMK, bool DIRECT, int WGM = 2, int NT = kThreads,
          bool SKDMA = false, bool TILEDB = false>
__global__ __launch_bounds__(NT, 512 / NT) void gemm_kernel(GemmArgs args, int tiles_n, StreamK sk) {
    constexpr int WGN = NT / kWave / WGM;
    constexpr int WTM = BM / WGM;               // wave tile rows
    constexpr int WTN = BN / WGN;               // wave tile cols
    constexpr int TM = WTM / 32;                // 32x32 MFMA tiles per wave (M)
    constexpr int TN = WTN / 32;                // 32x32 MFMA tiles per wave (N)
    static_assert(DIRECT || NT == kThreads, "the older form runs 256-thread blocks");
    constexpr int A_VECS = BM * BK / 8 / kThreads;        // uint4 of A per thread per step
    constexpr bool INT4 = BMODE == GemmB::kInt4;
    // direct form: bits per B element (16: the fp16-B reference product,
    // which has no codes, zero-points or group scales)
    constexpr int BITS = BMODE == GemmB::kInt8 ? 8 : BMODE == GemmB::kF16 ? 16 : 4;
    constexpr bool QB = BMODE != GemmB::kF16;              // B carries codes and group scales
    constexpr int BW = BITS / 4;                            // 16-byte B loads per column and step
    constexpr int B_WORDS = BN * BK / 8 / kThreads;       // packed words per thread per step
    constexpr int B_VECS = BN * BK / 8 / kThreads;        // fp16 B: uint4 per thread per step (int4: unused)
    constexpr int ACC = TM * TN * 16;                     // accumulators per lane
    static_assert(TM >= 1 && TN >= 1 && A_VECS >= 1, "tile shape");
    static_assert(DIRECT || !INT4 || B_WORDS == 2, "int4 B staging: 2 words (16 codes) per thread");
    static_assert(DIRECT || INT4 || B_VECS >= 1, "fp16 B staging");
    static_assert(DIRECT || BMODE != GemmB::kInt8, "W8 B runs the direct form only");
    static_assert(!TILEDB || (DIRECT && BMODE != GemmB::kInt8 && TN == 1 && WTN == 32),
                  "tiled B: INT4 or fp16, 32-column waves");
    constexpr int LDS_A = DIRECT ? BM * BKD : BM * LDK;
    constexpr int LDS_B = DIRECT ? 8 : BN * LDK;

    __shared__ __attribute__((aligned(16))) half_t As[2][LDS_A];
    __shared__ __attribute__((aligned(16))) half_t Bs[2][LDS_B];
    __shared__ int s_flag;

    const int M = static_cast<int>(args.M);
    const int N = static_cast<int>(args.N);
    const int K = static_cast<int>(args.K);
    const int G = args.group_size;
    const int ngroups = K / G;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = (wave / WGN) * WTM;
    const int wn = (wave % WGN) * WTN;
    const int lcol = lane & 31;
    const int lrow = lane & 31;
    const int lchunk = lane >> 5;          // which 8-k half of a 16-k MFMA step
    const UnpackConsts uk = unpack_consts();
    const int nk = K / (DIRECT ? BKD : BK);
    const int b_row = tid >> 1;            // int4 staging: row t / 2,
    const int b_half = tid & 1;            //   codes 16 * (t % 2) .. +15 of the step

    float16_t acc[TM][TN];

    // K steps [kb, ke) of one tile into acc, in true (unscaled) units.
    auto run_segment = [&](int tm, int tn, int kb, int ke) {
        // ---- staging: rows past M / N read the last row (their outputs
        //      are never stored), so every load is in bounds ----
        Stage<A_VECS, B_VECS> st, st1;
        const half_t* a_base = args.a + c8_of(tid);
        int a_off[A_VECS];
#pragma unroll
        for (int i = 0; i < A_VECS; ++i) a_off[i] = min(tm + (tid + i * kThreads) / (BK / 8), M - 1);
        const int64_t b_n = min(tn + b_row, N - 1);
        const uint32_t* b_words = args.qweight + b_n * (K / 8) + b_half * 2;
        const half_t* b_zeros = args.zeros + b_n * ngroups;
        int b_off[B_VECS];
#pragma unroll
        for (int i = 0; i < B_VECS; ++i) b_off[i] = min(tn + (tid + i * kThreads) / (BK / 8), N - 1);

        // scales of this lane's output columns travel as raw fp16 bits and
        // are converted only when used, a group after their load, so no wait
        // is forced on the loads in flight
        const uint16_t* s_bits[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
            s_bits[j] = reinterpret_cast<const uint16_t*>(args.scales) +
                        static_cast<int64_t>(min(tn + wn + j * 32 + lcol, N - 1)) * ngroups;
        auto to_scale = [](uint16_t bits) {
            const float v = static_cast<float>(__builtin_bit_cast(half_t, bits));
            return v == 0.f ? kTinyScale : v;
        };

#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        int g = INT4 ? (kb * BK) / G : 0;
        float s_cur[TN];
        uint16_t s_next[TN];
        if constexpr (INT4) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                s_cur[j] = to_scale(s_bits[j][g]);
                s_next[j] = s_bits[j][min(g + 1, ngroups - 1)];
            }
        }

        // Two register stages: the loads for step kt + 2 are issued while
        // step kt computes and land in LDS at the end of step kt + 1. Loads
        // past the segment re-read its last step (in bounds, never used).
        const int last_k0 = (ke - 1) * BK;
        auto load = [&](Stage<A_VECS, B_VECS>& dst, int k0) {
            load_stage<INT4>(dst, a_base, a_off, K, b_words, b_zeros, G, args.w + c8_of(tid), b_off,
                             min(k0, last_k0));
        };
        auto compute = [&](const half_t* as, const half_t* bs, int kt) {
            if constexpr (INT4) {
                if (kt > kb && ((kt * BK) % G) == 0) {
                    // entering the next group: C' <- C' * s_g / s_{g+1}
                    ++g;
                    float r[TN];
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const float sn = to_scale(s_next[j]);
                        r[j] = s_cur[j] / sn;
                        s_cur[j] = sn;
                    }
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
#pragma unroll
                            for (int e = 0; e < 16; ++e) acc[i][j][e] *= r[j];
#pragma unroll
                    for (int j = 0; j < TN; ++j) s_next[j] = s_bits[j][min(g + 1, ngroups - 1)];
                }
            }
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                half8_t af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = *reinterpret_cast<const half8_t*>(&as[swz(wm + i * 32 + lrow, ks * 2 + lchunk)]);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bf[j] = *reinterpret_cast<const half8_t*>(&bs[swz(wn + j * 32 + lrow, ks * 2 + lchunk)]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
            }
        };

        load(st, kb * BK);
        load(st1, (kb + 1) * BK);
        store_stage<INT4, BM, BN>(st, As[0], Bs[0], tid, b_row, b_half, uk);
        __syncthreads();
        for (int kt = kb; kt < ke; kt += 2) {
            load(st, (kt + 2) * BK);
            compute(As[0], Bs[0], kt);
            store_stage<INT4, BM, BN>(st1, As[1], Bs[1], tid, b_row, b_half, uk);
            __syncthreads();
            if (kt + 1 < ke) {
                load(st1, (kt + 3) * BK);
                compute(As[1], Bs[1], kt + 1);
                store_stage<INT4, BM, BN>(st, As[0], Bs[0], tid, b_row, b_half, uk);
                __syncthreads();
            }
        }
        if constexpr (INT4) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] *= s_cur[j];
        }
    };

    // K steps [kb, ke) of 64 of one tile into acc (direct-B form).
    // Step kt: A(kt) is in LDS buffer kt & 1, B(kt) in registers. In the
    // DMA form the step issues the LDS-DMA loads of A(kt + 1) into the other
    // buffer (free since the barrier that ended step kt - 1) and the loads
    // of B(kt + 1), and waits for all of them before its closing barrier.
    // In the register form A(kt + 1) is already in registers: the step
    // writes it to the other buffer and loads A(kt + 2) and B(kt + 1).
    // Either way it then runs 4 slices of 16 k with 8 MFMAs each.
    // Lane half h of the MFMA takes k = 32 h + 8 ks .. + 7 of the step in
    // slice ks, in both operands, so one 16-byte load gives a lane its four
    // B words of a column for the whole step.
    auto run_segment_direct = [&](int tm, int tn, int kb, int ke) {
        constexpr int AV = BM * BKD / 8 / NT;              // 16-byte A chunks per thread per step
        // A goes to LDS by LDS-DMA loads, except under stream-K, where the
        // register round trip measured faster (2048x4096x11008: 185 us
        // against 196 us; without stream-K the DMA form is 4-12 % faster)
        constexpr bool DMA = !STREAMK || SKDMA;
        const int lh = lane >> 5;
        // Buffer loads from tile-relative bases (scalar) with 32-bit lane
        // offsets; rows past M / N are clamped to the last row, so every
        // access is inside the tensor and the range check never fires.
        const int rows_a = min(BM, M - tm), cols_b = min(BN, N - tn);
        const auto a_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(args.a) + static_cast<int64_t>(tm) * K,
                                                            0, rows_a * K * 2, 0x00020000);
        const char* b_src = QB ? reinterpret_cast<const char*>(args.qweight) : reinterpret_cast<const char*>(args.w);
        // tiled B: the tile's 32-column groups, whole (rows past N are
        // allocated and never stored from)
        const auto b_rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(b_src) + static_cast<int64_t>(tn) * (K * BITS / 8), 0,
            (TILEDB ? (cols_b + 31) / 32 * 32 : cols_b) * (K * BITS / 8), 0x00020000);
        const auto s_rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<half_t*>(args.scales) + static_cast<int64_t>(tn) * ngroups, 0, cols_b * ngroups * 2, 0x00020000);
        const auto z_rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<half_t*>(args.zeros) + static_cast<int64_t>(tn) * ngroups, 0, cols_b * ngroups * 2, 0x00020000);
        int a_off[AV];
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int row = tid / 8 + i * (NT / 8);
            // an LDS-DMA load writes lane L's 16 bytes at slot L of the wave's
            // 1 KB (8 rows): that slot holds logical chunk (L % 8) ^ swizzle
            const int chunk = DMA ? ((tid % 8) ^ ((row >> 1) & 7)) : tid % 8;
            a_off[i] = (min(row, rows_a - 1) * K + chunk * 8) * 2;
        }
        int b_off[TN], sz_off[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = min(wn + j * 32 + lcol, cols_b - 1);
            // tiled: piece (group (wn + 32 j) / 32, step 0), lane's 16 bytes
            b_off[j] = TILEDB ? (wn + j * 32) / 32 * nk * (1024 * BW) + lane * 16 : n * (K * BITS / 8) + lh * (4 * BITS);
            sz_off[j] = n * ngroups * 2;
        }
        auto s_bits_at = [&](int j, int gg) {
            return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(s_rs, sz_off[j], gg * 2, 0));
        };
        auto z_bits_at = [&](int j, int gg) {
            return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(z_rs, sz_off[j], gg * 2, 0));
        };
        auto to_scale = [](uint16_t bits) {
            const float v = static_cast<float>(__builtin_bit_cast(half_t, bits));
            return v == 0.f ? kTinyScale : v;
        };

#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        const int last = ke - 1;
        u32x4 areg[AV];
        u32x4 b0[TN][BW], b1[TN][BW];
        auto load_a = [&](int kt) {
            const int k0 = uniform(min(kt, last) * BKD * 2);
#pragma unroll
            for (int i = 0; i < AV; ++i) areg[i] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_off[i], k0, 0);
        };
        auto load_b = [&](u32x4 (&dst)[TN][BW], int kt) {
            const int w0 = uniform(min(kt, last) * (TILEDB ? 1024 * BW : BKD * BITS / 8));
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < BW; ++v)
                    dst[j][v] = __builtin_amdgcn_raw_buffer_load_b128(b_rs, b_off[j] + (TILEDB ? 1024 : 16) * v, w0, 0);
        };
        auto store_a = [&](half_t* as) {
#pragma unroll
            for (int i = 0; i < AV; ++i)
                *reinterpret_cast<u32x4*>(&as[swz64(tid / 8 + i * (NT / 8), tid % 8)]) = areg[i];
        };

        int g = (kb * BKD) / G;
        float s_cur[TN];
        uint16_t s_next[TN], z_next[TN];
        half2_t zc_hi[TN], zc_lo[TN];
        auto set_zero = [&](int j, uint16_t zb) {
            const half_t z = __builtin_bit_cast(half_t, zb);
            const half_t zh = static_cast<half_t>(1024.0f) + z;   // exact
            const half_t zl = static_cast<half_t>(64.0f) + z;     // exact
            zc_hi[j] = half2_t{zh, zh};
            zc_lo[j] = half2_t{zl, zl};
        };
        if constexpr (QB) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                s_cur[j] = to_scale(s_bits_at(j, g));
                set_zero(j, z_bits_at(j, g));
                s_next[j] = s_bits_at(j, min(g + 1, ngroups - 1));
                z_next[j] = z_bits_at(j, min(g + 1, ngroups - 1));
            }
        }

        // LDS-DMA loads i in [i0, i1) of A(kt) into buffer as
        auto dma_a = [&](half_t* as, int kt, int i0, int i1) {
            const int k0 = uniform(min(kt, last) * BKD * 2);
#pragma unroll
            for (int i = i0; i < i1; ++i) {
                half_t* dst = as + (wave * (kWave / 8) + i * (NT / 8)) * BKD;   // the wave's 8 rows
                load_lds16(a_rs, dst, a_off[i], k0);
            }
        };
        auto step = [&](int kt, const half_t* cur, half_t* nxt, const u32x4 (&bw)[TN][BW], u32x4 (&bn)[TN][BW]) {
            if constexpr (DMA) {
                if (kt + 1 < ke) dma_a(nxt, kt + 1, 0, AV);
            } else {
                if (kt + 1 < ke) store_a(nxt);
                load_a(kt + 2);
            }
            load_b(bn, kt + 1);
            if (QB && kt > kb && ((kt * BKD) % G) == 0) {
                // entering the next group: C' <- C' * s_g / s_{g+1}
                ++g;
                float r[TN];
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const float sn = to_scale(s_next[j]);
                    r[j] = s_cur[j] / sn;
                    s_cur[j] = sn;
                    set_zero(j, z_next[j]);
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[i][j][e] *= r[j];
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    s_next[j] = s_bits_at(j, uniform(min(g + 1, ngroups - 1)));
                    z_next[j] = z_bits_at(j, uniform(min(g + 1, ngroups - 1)));
                }
            }
            // slice ks + 1's fragments are read (and its B unpacked) before
            // slice ks's MFMAs, so LDS latency hides behind a whole slice
            half8_t af[2][TM], bf[2][TN];
            auto fetch = [&](int ks, half8_t (&a)[TM], half8_t (&b)[TN]) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    a[i] = *reinterpret_cast<const half8_t*>(&cur[swz64(wm + i * 32 + lrow, lh * 4 + ks)]);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (BITS == 16)
                        b[j] = __builtin_bit_cast(half8_t, bw[j][ks]);   // k = 32 h + 8 ks .. + 7
                    else if constexpr (BITS == 4)
                        b[j] = __builtin_bit_cast(half8_t, unpack_word(bw[j][0][ks], zc_hi[j], zc_lo[j], uk));
                    else
                        b[j] = __builtin_bit_cast(half8_t, unpack_bytes(bw[j][ks / 2][(ks % 2) * 2],
                                                                        bw[j][ks / 2][(ks % 2) * 2 + 1], zc_hi[j]));
                }
            };
            fetch(0, af[0], bf[0]);
#pragma unroll
            for (int ks = 0; ks < BKD / 16; ++ks) {
                if (ks + 1 < BKD / 16) fetch(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
                // keeps slice ks + 1's LDS reads ahead of slice ks's MFMAs
                // (the scheduler otherwise sinks each read next to its use);
                // the register form has no VGPRs to spare for it
                if constexpr (DMA) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ks & 1][i], bf[ks & 1][j], acc[i][j],
                                                                           0, 0, 0);
            }
        };

        load_b(b0, kb);
        if constexpr (DMA) {
            dma_a(As[0], kb, 0, AV);
            __builtin_amdgcn_s_waitcnt(0);
        } else {
            load_a(kb);
            store_a(As[0]);
            load_a(kb + 1);
        }
        __syncthreads();
        for (int kt = kb; kt < ke; kt += 2) {
            step(kt, As[0], As[1], b0, b1);
            if constexpr (DMA) __builtin_amdgcn_s_waitcnt(0);   // this step's DMA has landed
            __syncthreads();
            if (kt + 1 < ke) {
                step(kt + 1, As[1], As[0], b1, b0);
                if constexpr (DMA) __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
        }
        if constexpr (QB) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] *= s_cur[j];
        }
    };
    auto segment = [&](int tm, int tn, int kb, int ke) {
        if constexpr (DIRECT)
            run_segment_direct(tm, tn, kb, ke);
        else
            run_segment(tm, tn, kb, ke);
    };

    // ---- epilogue ----
    // accumulator element e of MFMA tile (i, j) is output (row, col) =
    // (tm + wm + 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4, tn + wn + 32 j + lane % 32)
    const int lrow4 = (lane >> 5) * 4;
    // fp32 results and loss references use the tiled layout of ref_offset
    const int64_t ref_tiles_n = (N + kRefTileN - 1) / kRefTileN;
    auto emit = [&](int tm, int tn, int i, int j, int e, float v, float& sq) {
        const int n = tn + wn + j * 32 + lcol;
        const int m = tm + wm + i * 32 + (e >> 2) * 8 + lrow4 + (e & 3);
        if (m < M && n < N) {
            if constexpr (OMODE == GemmOut::kF16) {
                args.y16[static_cast<int64_t>(m) * N + n] = static_cast<half_t>(v);
            } else if constexpr (OMODE == GemmOut::kF32) {
                args.y32[ref_offset(m, n, ref_tiles_n)] = v;
            } else {
                const float d = v - args.yref[ref_offset(m, n, ref_tiles_n)];
                sq += d * d;
            }
        }
    };
    auto finish_loss = [&](int tile, float sq) {
        if constexpr (OMODE == GemmOut::kLoss) {
            __shared__ double red[NT / kWave];
            double v = static_cast<double>(sq);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
            if (lane == 0) red[wave] = v;
            __syncthreads();
            if (tid == 0) {
                double t = 0.0;
                for (int w = 0; w < NT / kWave; ++w) t += red[w];
                args.partials[tile] = t;
            }
            __syncthreads();
        }
    };
    auto finish_tile = [&](int tile, int tm, int tn) {
        float sq = 0.f;
        if constexpr (OMODE == GemmOut::kF16) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) emit(tm, tn, i, j, e, acc[i][j][e], sq);
        } else {
            // tiled layout: a lane's 16 values of a sub-tile are contiguous.
            // Sub-tiles that start inside [0, M) x [0, N) lie inside the
            // padded buffer; their positions past M or N are padding.
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int m0 = tm + wm + i * 32, n0 = tn + wn + j * 32;
                    if (m0 >= M || n0 >= N) continue;
                    float4_t* p = reinterpret_cast<float4_t*>(
                        (OMODE == GemmOut::kF32 ? args.y32 : const_cast<float*>(args.yref)) +
                        ref_subtile_base(m0, n0, ref_tiles_n) + lane * 16);
                    if constexpr (OMODE == GemmOut::kF32) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            p[q] = float4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                            acc[i][j][4 * q + 3]};
                    } else {
                        float4_t r[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) r[q] = p[q];
                        const int n = n0 + lcol;
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int m = m0 + (e >> 2) * 8 + lrow4 + (e & 3);
                            if (m < M && n < N) {
                                const float d = acc[i][j][e] - r[e >> 2][e & 3];
                                sq += d * d;
                            }
                        }
                    }
                }
        }
        finish_loss(tile, sq);
    };

    if constexpr (!STREAMK) {
        const int tile = xcd_tile(blockIdx.x, gridDim.x);
        const int tm = (tile / tiles_n) * BM;
        const int tn = (tile % tiles_n) * BN;
        segment(tm, tn, 0, nk);
        finish_tile(tile, tm, tn);
    } else {
        // Units u = (tile, K step) = tile * ipt + step over all tiles. A block
        // of the data-parallel head owns one whole tile; the others own a
        // stream-K range of the split tiles' units (consecutive ranges,
        // which share tiles, go to the same XCD). One loop serves both.
        const int head = sk.dp_tiles * sk.ipt;
        int u, u1;
        int b = 0;
        if (static_cast<int>(blockIdx.x) < sk.dp_tiles) {
            u = uniform(xcd_tile(blockIdx.x, sk.dp_tiles) * sk.ipt);
            u1 = u + sk.ipt;
        } else {
            b = uniform(xcd_tile(blockIdx.x - sk.dp_tiles, gridDim.x - sk.dp_tiles));
            u = uniform(head + sk_start(sk, b));
            u1 = uniform(head + sk_start(sk, b + 1));
        }
        while (u < u1) {
            const int tile = uniform(u / sk.ipt);
            const int lt = tile - sk.dp_tiles;               // tile within the split range
            const int kb = uniform(u - tile * sk.ipt);
            const int ke = uniform(min(sk.ipt, kb + (u1 - u)));
            const int tm = (tile / tiles_n) * BM;
            const int tn = (tile % tiles_n) * BN;
            segment(tm, tn, kb, ke);
            u += ke - kb;
            if (kb == 0 && ke == sk.ipt) {
                finish_tile(tile, tm, tn);
                continue;
            }
            // Partial tile: park the sums, count in; the last of the tile's
            // blocks to arrive adds every part in segment order (so the
            // result does not depend on arrival order), finishes the tile and
            // resets its counter. Nobody waits on anybody.
            const int u_first = lt * sk.ipt;
            const int b_first = uniform(sk_block_of(sk, u_first));
            const int b_last = uniform(sk_block_of(sk, u_first + sk.ipt - 1));
            // a block holds at most two partial tiles: the one it starts in
            // (slot 0) and the one it ends in (slot 1)
            auto slot_of = [&](int bb) {
                const int slot = uniform(bb * 2 + (sk_start(sk, bb) / sk.ipt == lt ? 0 : 1));
                return sk.partials + static_cast<int64_t>(slot) * (BM * BN);
            };
            {
                // chunk-major layout [(i, j, e / 4)][thread][4]: one coalesced
                // 1 KB row per wave and chunk, addressed by a scalar offset
                const auto rs = partial_rsrc(slot_of(b), BM * BN * 4);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4_t v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                                acc[i][j][4 * q + 3]};
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, tid * 16,
                                                                   ((i * TN + j) * 4 + q) * NT * 16, kSc1);
                        }
            }
            // The parts are written and read with the sc1 (device-coherent)
            // cache policy, the form this target gives device-scope atomic
            // stores and loads, so they bypass the per-XCD L2s instead of
            // needing a device-wide L2 write-back/invalidate (a device fence),
            // which would also flush every other block's cached tiles. All
            // stores complete (vmcnt 0) before the counter is bumped, and the
            // finisher issues its loads only after reading the count.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0)
                s_flag = __hip_atomic_fetch_add(&sk.counters[tile], 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) == b_last - b_first;
            __syncthreads();
            if (!s_flag) continue;
            // Every part, this block's own included, is read back and summed
            // in segment order, eight float4 chunks (32 outputs) at a time,
            // each chunk's four outputs written as soon as they are complete.
            {
                constexpr int kChunks = TM * TN * 4;
                constexpr int kBatch = 8;
                float sq = 0.f;
#pragma unroll
                for (int c0 = 0; c0 < kChunks; c0 += kBatch) {
                    float4_t sum[kBatch];
#pragma unroll
                    for (int c = 0; c < kBatch; ++c) sum[c] = float4_t{0.f, 0.f, 0.f, 0.f};
                    for (int bb = b_first; bb <= b_last; ++bb) {
                        const auto rs = partial_rsrc(slot_of(bb), BM * BN * 4);
                        float4_t v[kBatch];
#pragma unroll
                        for (int c = 0; c < kBatch; ++c)
                            v[c] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    rs, tid * 16, (c0 + c) * NT * 16, kSc1));
#pragma unroll
                        for (int c = 0; c < kBatch; ++c) sum[c] += v[c];
                    }
#pragma unroll
                    for (int c = 0; c < kBatch; ++c) {
                        const int ij = (c0 + c) / 4, q = (c0 + c) % 4;
#pragma unroll
                        for (int r = 0; r < 4; ++r) emit(tm, tn, ij / TN, ij % TN, 4 * q + r, sum[c][r], sq);
                    }
                }
                finish_loss(tile, sq);
            }
            if (tid == 0) __hip_atomic_store(&sk.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    (void)ACC;
}

constexpr int kBM = 256;

// Block geometries: 256 x 128 tiles of 256 threads, two blocks per CU (every
// form), and 256 x 256 tiles of 512 threads (8 waves of 256 x 32), one block
// per CU (direct form), which stages each A step once for twice the columns.
struct Geometry {
    int bm, bn, threads, per_cu;
};
constexpr Geometry kNarrowTile{256, 128, 256, 2};
constexpr Geometry kWideTile{256, 256, 512, 1};

constexpr int kMinSteps = 8;        // K steps per block at least

// Segments per tile at most: 4, and up to 6 while every segment keeps 32 K
// steps of 64. Short segments cost more in fp32 partials than they gain in
// busy CUs (256 x 11008 x 4096, 64 steps: 4 segments 51.7 us, 6 segments
// 58.5 us); long rows gain (512 x 5120 x 13824, 40 wide tiles of 216 steps,
// 160 blocks at 4 segments: 114 -> 98.5 us at 6; 8 segments 106 us).
int max_split(int64_t steps) { return static_cast<int>(std::clamp<int64_t>(steps / 32, 4, 6)); }

int64_t resident_slots(const Geometry& g) { return static_cast<int64_t>(g.per_cu) * cu_count(); }
int64_t tiles_of(const Geometry& g, int64_t M, int64_t N) { return ceil_div(M, g.bm) * ceil_div(N, g.bn); }

// Stream-K pays off when there are well under one round of tiles: one tile
// per block would leave CUs idle or at one block each. Over more rounds
// nearly every tile would be split and its fp32 partials moved through
// memory: measured on 2048 x 11008 x 4096 with 256 x 256 tiles, 831 MB of
// traffic per launch against 282 MB unsplit, for a few percent of time
// (use_hybrid splits only a short last round instead).
bool use_stream_k(const Geometry& g, int64_t tiles, int64_t steps) {
    // up to two thirds of a round: nearer a full round, one tile per block
    // is faster than the partials (M = 1280 x 11008 x 4096: 129 us one tile
    // per block against 147 us split)
    if (tiles * 3 > resident_slots(g) * 2 || tiles > split_counter_slots()) return false;
    return tiles * steps < (int64_t{1} << 31);
}

// Over more than one round with a short last round (at most a quarter of
// the slots), the whole rounds run data-parallel and only the last round's
// tiles are split (stream-K over the resident slots), so the tail no longer
// runs at one block per CU: 516 tiles of 1536 x 11008 x 4096 take 158 us
// against 189 us. With longer tails the partials cost more than they save
// (688 tiles of 2048 x 11008 x 4096: 208 against 196 us).
bool use_hybrid(const Geometry& g, int64_t tiles, int64_t steps) {
    const int64_t slots = resident_slots(g);
    const int64_t tail = tiles % slots;
    if (tiles <= slots || tail == 0 || tail * 4 > slots || tiles > split_counter_slots()) return false;
    return tiles * steps < (int64_t{1} << 31);
}

int stream_k_grid(const Geometry& g, int64_t tiles, int64_t steps) {
    const int64_t total = tiles * steps;
    int64_t gr = std::min(resident_slots(g), tiles * max_split(steps));
    gr = std::min(gr, std::max<int64_t>(1, total / kMinSteps));
    return static_cast<int>(gr);
}

// two fp32 partial tiles per resident block, for either geometry
size_t partials_bytes() {
    const size_t a = static_cast<size_t>(resident_slots(kNarrowTile)) * 2 * kNarrowTile.bm * kNarrowTile.bn;
    const size_t b = static_cast<size_t>(resident_slots(kWideTile)) * 2 * kWideTile.bm * kWideTile.bn;
    return round_up(std::max(a, b) * sizeof(float), 256);
}

template <const Geometry& GEO, GemmB BMODE, GemmOut OMODE, bool DIRECT, int WGM = 2>
void launch_cfg(const GemmArgs& args, void* workspace, hipStream_t stream) {
    if constexpr (((OMODE == GemmOut::kLoss && BMODE == GemmB::kInt4) ||
                   (OMODE == GemmOut::kF32 && BMODE == GemmB::kF16)) && DIRECT && GEO.bn == 128) {
        if (args.b_tiled) {
            const int64_t tn = ceil_div(args.N, GEO.bn);
            hipLaunchKernelGGL((gemm_kernel<GEO.bm, GEO.bn, BMODE, OMODE, false, true, WGM, GEO.threads, false, true>),
                               dim3(static_cast<unsigned>(ceil_div(args.M, GEO.bm) * tn)), dim3(GEO.threads), 0,
                               stream, args, static_cast<int>(tn), StreamK{});
            return;
        }
    }
    const int64_t tiles_n = ceil_div(args.N, GEO.bn);
    const int64_t tiles = ceil_div(args.M, GEO.bm) * tiles_n;
    const int64_t steps = args.K / (DIRECT ? BKD : BK);
    StreamK sk;
    // Only fp16-output products take a workspace (the searches' fp32 and
    // loss forms never split), so the split instances exist for them alone.
    if constexpr (OMODE != GemmOut::kF16) workspace = nullptr;
    if (OMODE == GemmOut::kF16 && workspace != nullptr && use_stream_k(GEO, tiles, steps)) {
        sk.ipt = static_cast<int>(steps);
        sk.total = static_cast<int>(tiles * sk.ipt);
        sk.grid = stream_k_grid(GEO, tiles, steps);
        sk.q = sk.total / sk.grid;
        sk.r = sk.total % sk.grid;
        sk.counters = static_cast<int*>(workspace);
        sk.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + split_counter_bytes());
        if constexpr (OMODE == GemmOut::kF16)
            hipLaunchKernelGGL((gemm_kernel<GEO.bm, GEO.bn, BMODE, OMODE, true, DIRECT, WGM, GEO.threads>),
                               dim3(static_cast<unsigned>(sk.grid)), dim3(GEO.threads), 0, stream, args,
                               static_cast<int>(tiles_n), sk);
        return;
    }
    if constexpr (DIRECT && OMODE == GemmOut::kF16) {
        if (workspace != nullptr && use_hybrid(GEO, tiles, steps)) {
            sk.dp_tiles = static_cast<int>(tiles / resident_slots(GEO) * resident_slots(GEO));
            const int64_t tail = tiles - sk.dp_tiles;
            sk.ipt = static_cast<int>(steps);
            sk.total = static_cast<int>(tail * sk.ipt);
            sk.grid = stream_k_grid(GEO, tail, steps);
            sk.q = sk.total / sk.grid;
            sk.r = sk.total % sk.grid;
            sk.counters = static_cast<int*>(workspace);
            sk.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + split_counter_bytes());
            hipLaunchKernelGGL((gemm_kernel<GEO.bm, GEO.bn, BMODE, OMODE, true, DIRECT, WGM, GEO.threads, true>),
                               dim3(static_cast<unsigned>(sk.dp_tiles + sk.grid)), dim3(GEO.threads), 0, stream, args,
                               static_cast<int>(tiles_n), sk);
            return;
        }
    }
    hipLaunchKernelGGL((gemm_kernel<GEO.bm, GEO.bn, BMODE, OMODE, false, DIRECT, WGM, GEO.threads>),
                       dim3(static_cast<unsigned>(tiles)), dim3(GEO.threads), 0, stream, args,
                       static_cast<int>(tiles_n), sk);
}

// The direct-B form needs every K step of 64 inside one group, and 32-bit
// byte offsets within a 256-row tile of A. Its waves sit side by side along
// N (256 x 32 each): a wave's unpack work per MFMA halves against the 2 x 2
// arrangement (whose wave pairs would unpack the same columns twice).
constexpr int kDirectWgm = 1;
bool direct_ok(const GemmArgs& args) { return args.group_size >= BKD && args.K * kBM * 2 < (int64_t{1} << 31); }

// Narrow or wide tile, by the time of the rounds each takes (one-tile-per-
// block launches). In units where a round of the wide tile (one 256 x 256
// tile per CU) costs 20, a full round of the narrow tile (two 256 x 128 tiles
// per CU, the same area) costs 22 and a last round of at most one narrow tile
// per CU costs 12. Measured at N = 11008, K = 4096 (us, narrow against wide):
// M = 1024: 114 / 101; 1280: 125 / 112; 2048: 191 / 210; 3072: 307 / 330;
// 4096: 368 / 336. With a workspace, a shape of under two thirds of a round
// takes the wide tile under stream-K.
int64_t narrow_rounds_cost(int64_t tiles) {
    const int64_t cu = cu_count(), slots = resident_slots(kNarrowTile);
    const int64_t tail = tiles % slots;
    return tiles / slots * 22 + (tail == 0 ? 0 : tail <= cu ? 12 : 22);
}
int64_t wide_rounds_cost(int64_t tiles) { return ceil_div(tiles, resident_slots(kWideTile)) * 20; }
bool use_wide(const GemmArgs& args, bool have_workspace) {
    const int64_t t = tiles_of(kWideTile, args.M, args.N);
    const int64_t steps = args.K / BKD;
    if (have_workspace && use_stream_k(kWideTile, t, steps)) return true;
    return wide_rounds_cost(t) < narrow_rounds_cost(tiles_of(kNarrowTile, args.M, args.N));
}

// The loss form stays on the 256 x 128 tile: its epilogue streams an fp32
// reference tile, which two blocks per CU overlap with each other's MFMAs
// (the full-size scale search measured 153 ms there against 156 ms wide).
template <GemmB BMODE, GemmOut OMODE>
void launch_direct(const GemmArgs& args, void* workspace, hipStream_t stream) {
    if constexpr (OMODE != GemmOut::kLoss) {
        if (use_wide(args, workspace != nullptr)) {
            launch_cfg<kWideTile, BMODE, OMODE, true, kDirectWgm>(args, workspace, stream);
            return;
        }
    }
    launch_cfg<kNarrowTile, BMODE, OMODE, true, kDirectWgm>(args, workspace, stream);
}

template <GemmOut OMODE>
void launch_int4(const GemmArgs& args, void* workspace, hipStream_t stream) {
    if (args.b_tiled && (OMODE != GemmOut::kLoss || !direct_ok(args))) return;   // caller checks: see launch_gemm
    if (direct_ok(args))
        launch_direct<GemmB::kInt4, OMODE>(args, workspace, stream);
    else
        launch_cfg<kNarrowTile, GemmB::kInt4, OMODE, false>(args, workspace, stream);
}

}  // namespace

int64_t gemm_tile_count(int64_t M, int64_t N) { return tiles_of(kNarrowTile, M, N); }

bool gemm_tiled_ok(int64_t K, int group_size) {
    GemmArgs a;
    a.K = K;
    a.group_size = group_size;
    return K % BKD == 0 && direct_ok(a);
}

namespace {

// One thread per 16-byte piece of the tiled fp16 B (the order of
// launch_tile_fp16_b); a block's 256 pieces are one 32-row, 64-k block of W,
// so its reads are whole 128-byte rows.
__global__ __launch_bounds__(256) void tile_fp16_b_kernel(const half_t* __restrict__ w, int64_t N, int64_t K,
                                                          int64_t pieces, half_t* __restrict__ wt) {
    const int64_t p = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (p >= pieces) return;
    const int64_t nk = K / BKD;
    const int lane = static_cast<int>(p & 63), v = static_cast<int>((p >> 6) & 3);
    const int64_t t = (p >> 8) % nk, g = (p >> 8) / nk;
    const int64_t row = g * 32 + (lane & 31), col = t * BKD + (lane >> 5) * 32 + v * 8;
    u32x4 piece = {0u, 0u, 0u, 0u};
    if (row < N) piece = *reinterpret_cast<const u32x4*>(w + row * K + col);
    *reinterpret_cast<u32x4*>(wt + p * 8) = piece;
}

}  // namespace

bool gemm_ref_tiled_ok(int64_t K) { return K % BKD == 0 && K * kBM * 2 < (int64_t{1} << 31); }

awq_status launch_tile_fp16_b(const half_t* w, int64_t N, int64_t K, half_t* wt, hipStream_t stream) {
    if (!gemm_ref_tiled_ok(K)) return AWQ_ERR_SHAPE;
    const int64_t pieces = static_cast<int64_t>(tiled_fp16_halves(N, K) / 8);
    if (pieces == 0) return AWQ_OK;
    hipLaunchKernelGGL(tile_fp16_b_kernel, dim3(static_cast<unsigned>(ceil_div(pieces, 256))), dim3(256), 0, stream,
                       w, N, K, pieces, wt);
    return last_launch_status();
}

size_t gemm_workspace_bytes(int64_t M, int64_t N) {
    (void)M;
    (void)N;
    return split_counter_bytes() + partials_bytes();
}

awq_status launch_gemm(const GemmArgs& args, GemmB b, GemmOut out, hipStream_t stream, void* workspace) {
    if (args.M == 0 || args.N == 0) return AWQ_OK;
    // tiled B: the loss form (INT4 B) and the fp16-B reference, both on the
    // direct core only
    if (args.b_tiled && !((b == GemmB::kInt4 && out == GemmOut::kLoss && direct_ok(args)) ||
                          (b == GemmB::kF16 && out == GemmOut::kF32 && gemm_ref_tiled_ok(args.K))))
        return AWQ_ERR_CONFIG;
    if (b == GemmB::kInt8) {
        // W8 B: the direct form only, fp16 output
        if (!direct_ok(args) || out != GemmOut::kF16) return AWQ_ERR_CONFIG;
        launch_direct<GemmB::kInt8, GemmOut::kF16>(args, workspace, stream);
    } else if (b == GemmB::kInt4) {
        switch (out) {
            case GemmOut::kF16: launch_int4<GemmOut::kF16>(args, workspace, stream); break;
            case GemmOut::kF32: launch_int4<GemmOut::kF32>(args, workspace, stream); break;
            case GemmOut::kLoss: launch_int4<GemmOut::kLoss>(args, workspace, stream); break;
        }
    } else {
        switch (out) {
            case GemmOut::kF16: launch_cfg<kNarrowTile, GemmB::kF16, GemmOut::kF16, false>(args, workspace, stream); break;
            case GemmOut::kF32:
                // the searches' reference W . x^T: the direct form whenever K
                // is whole 64-k steps (fp16 B straight into the operand, no
                // unpack and no group scale), the older form otherwise
                if (args.K % BKD == 0 && args.K * kBM * 2 < (int64_t{1} << 31))
                    launch_cfg<kNarrowTile, GemmB::kF16, GemmOut::kF32, true, kDirectWgm>(args, nullptr, stream);
                else
                    launch_cfg<kNarrowTile, GemmB::kF16, GemmOut::kF32, false>(args, workspace, stream);
                break;
            case GemmOut::kLoss: return AWQ_ERR_CONFIG;
        }
    }
    return last_launch_status();
}

}  // namespace awq
