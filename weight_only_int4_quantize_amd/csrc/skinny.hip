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
// * A block is 8 waves over 256 output columns (two 16-column MFMA tiles per
//   wave) and up to 64 rows. It stages its whole K range of x in LDS once,
//   before the main loop (rows padded so the 16 rows of a fragment read fall
//   in distinct banks); the main loop then issues nothing but the packed
//   weights, streamed straight into registers through a ring of groups in
//   flight. Vector-memory loads complete in order, so keeping x out of the
//   loop is what lets the ring stay deep.
// * To fill the GPU when there are few column tiles, K is split across
//   blocks (this needs a workspace). A block parks its fp32 partial tile,
//   bumps a per-column-tile counter, and the last block to arrive adds every
//   split in order and writes y: deterministic, and nobody waits on anybody.
// * A K range larger than the LDS holds (no workspace, or more column tiles
//   than it counts) is walked in phases: stage a phase's x and pairs, stream
//   its groups, and stage the next phase between two barriers. The weight
//   ring runs on across the phases; they are a multiple of its depth long,
//   so each starts on slot 0.
#include <algorithm>

#include "awq_internal.h"

namespace awq {
namespace {

constexpr int kSkThreads = 512;         // 8 waves
constexpr int kSkBN = 256;              // output columns per block
constexpr int kSkLds = 152 * 1024;      // LDS budget for the staged x
constexpr int kSkXP = 19;               // x pieces (16 bytes) per thread at most
// The prologue's loads are issued unconditionally (past-the-end offsets read
// zero without touching memory), so their count is a compile-time bound.
// Every unneeded load still costs address and TA cycles, which dominate the
// short splits, so the kernel comes in three prologue sizes (FORM 0, 1, 2:
// x pieces kSkXPForm[FORM], (scale, zero) pairs kSkSZForm[FORM] per thread)
// and the launch takes the smallest that covers the block's K range.
constexpr int kSkXPForm[3] = {4, 8, 19};
constexpr int kSc1 = 16;                // cache-policy bit sc1 (device scope)

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

// WPL packed words per lane per group: G / 32 (1, 2, 4, 8 for G = 32 .. 256).
template <int WPL>
struct GroupLoad {
    uint32_t w[2][WPL];     // two column tiles
};

// LDS row of the staged x, in halves: the K range rounded up to 128 plus 8,
// so consecutive rows start 16 bytes apart modulo the 256-byte bank cycle.
__host__ __device__ inline int sk_stride(int krange) { return (krange + 127) / 128 * 128 + 8; }
// LDS row (one column) of the staged (scale, zero) pairs, in 32-bit words:
// odd, so 16 columns read at one group fall in distinct banks.
__host__ __device__ inline int sk_szst(int ngb) { return ngb | 1; }
// LDS bytes of one block: x [16 MB rows][stride] halves + (scale, zero)
// pairs [256 columns][szst] words.
__host__ __device__ inline int sk_lds_bytes(int mb, int krange, int group_size) {
    return 16 * mb * sk_stride(krange) * 2 + kSkBN * sk_szst(krange / group_size) * 4;
}
constexpr int kSkSZ = 32;               // (scale, zero) pairs per thread at most
// weight groups in flight per wave (the ring depth)
__host__ __device__ constexpr int sk_depth(int mb, int wpl) { return (mb <= 2 && wpl <= 4) ? 8 : 4; }
constexpr int kSkSZForm[3] = {4, 8, 32};

// msp = M | splits << 7 | phase_groups << 16 (M < 128, splits < 512,
// phase_groups < 65536): with it every argument the waves need before the
// fixup is within the 14 preloaded argument dwords (the partial and counter
// pointers, used last, follow)
template <int MB, int WPL, int FORM>
__global__ __launch_bounds__(kSkThreads, 1) void skinny_kernel(const half_t* __restrict__ x,
                                                              const uint32_t* __restrict__ qweight,
                                                              const half_t* __restrict__ scales,
                                                              const half_t* __restrict__ zeros,
                                                              half_t* __restrict__ y, int N, int K, uint32_t msp,
                                                              float* __restrict__ partials,
                                                              int* __restrict__ counters) {
    const int M = static_cast<int>(msp & 127u);
    const int splits = static_cast<int>((msp >> 7) & 511u);
    const int phase_groups = static_cast<int>(msp >> 16);
    constexpr int G = WPL * 32;
    constexpr int MP = 16 * MB;                          // padded rows
    constexpr int kSkDepth = sk_depth(MB, WPL);
    constexpr int XPN = kSkXPForm[FORM];
    constexpr int SZN = kSkSZForm[FORM];
    static_assert(kSkXPForm[2] == kSkXP && kSkSZForm[2] == kSkSZ, "the largest form is the bound sk_kmax uses");
    extern __shared__ __attribute__((aligned(16))) half_t xs[];   // [MP][stride], then (s, z) pairs
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
    // The K range is staged in phases of at most phase_groups groups (one
    // phase unless the range exceeds the LDS; then phase_groups is a
    // multiple of the ring depth, so every phase starts on slot 0)
    const int pg = min(phase_groups, g1 - g0);
    const int stride = sk_stride(pg * G);

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
    uint32_t w_off[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int n = n_base + 16 * t + col;
        w_off[t] = n < N ? static_cast<uint32_t>(n) * static_cast<uint32_t>(K / 2) + lg * WPL * 4 : w_bytes;
    }
    auto load_group = [&](GroupLoad<WPL>& gl, int g) {
        const bool ok = g < g1;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t wo = ok ? w_off[t] + static_cast<uint32_t>(g) * (G / 2) : w_bytes;
            if constexpr (WPL == 8) {
                const u32x4 v0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 0, 0));
                const u32x4 v1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 16, 0));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    gl.w[t][j] = v0[j];
                    gl.w[t][4 + j] = v1[j];
                }
            } else if constexpr (WPL == 4) {
                const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 0, 0));
#pragma unroll
                for (int j = 0; j < 4; ++j) gl.w[t][j] = v[j];
            } else if constexpr (WPL == 2) {
                const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rw, wo, 0, 0));
#pragma unroll
                for (int j = 0; j < 2; ++j) gl.w[t][j] = v[j];
            } else {
                gl.w[t][0] = __builtin_amdgcn_raw_buffer_load_b32(rw, wo, 0, 0);
            }
        }
    };

    // ---- the block's (scale, zero) pairs: consecutive lanes read
    //      consecutive groups of one column, so these loads are coalesced
    //      (one 2-byte load per lane and group in the main loop would cost a
    //      cache-line request each) ----
    const int ngb = pg;                                  // groups of the first phase
    const int szst = sk_szst(pg);
    const int nsz = kSkBN * ngb;
    uint32_t* szs = reinterpret_cast<uint32_t*>(xs + MP * stride);
    uint16_t sr[SZN], zr[SZN];
#pragma unroll
    for (int i = 0; i < SZN; ++i) {
        const int e = tid + i * kSkThreads;
        const int c = e / ngb, gi = e - c * ngb;
        const int n = tile * kSkBN + c;
        const uint32_t so = (e < nsz && n < N) ? (static_cast<uint32_t>(n) * ng + g0 + gi) * 2 : sz_bytes;
        sr[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
        zr[i] = __builtin_amdgcn_raw_buffer_load_b16(rz, so, 0, 0);
    }

    // ---- x: the block's whole K range, rows past M as zeros (buffer
    //      loads, no branches) ----
    const uint32_t x_bytes = static_cast<uint32_t>(static_cast<int64_t>(M) * K * 2);
    const auto rx = rsrc(x, x_bytes);
    const int pr = pg * G / 8;                           // pieces per row
    const int pieces = MP * pr;
    uint4 xr[XPN];
#pragma unroll
    for (int i = 0; i < XPN; ++i) {
        const int p = tid + i * kSkThreads;
        const int r = p / pr, c8 = p - r * pr;
        const bool ok = p < pieces && r < M;
        const uint32_t off = ok ? (static_cast<uint32_t>(r) * K + g0 * G + c8 * 8) * 2 : x_bytes;
        xr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < SZN; ++i) {
        const int e = tid + i * kSkThreads;
        if (e < nsz) {
            const int c = e / ngb, gi = e - c * ngb;
            szs[c * szst + gi] = static_cast<uint32_t>(sr[i]) | (static_cast<uint32_t>(zr[i]) << 16);
        }
    }
    // Loads complete in order: the pairs (issued first) were staged without
    // waiting for x; x is staged below without waiting for the weights.
    GroupLoad<WPL> ring[kSkDepth];
    // slot by slot, as the loop refills them: the wait counts at the loop
    // head are the smaller of this order and the loop's own
#pragma unroll
    for (int d = 0; d < kSkDepth; ++d) {
        load_group(ring[d], g0 + d);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < XPN; ++i) {
        const int p = tid + i * kSkThreads;
        if (p < pieces) {
            const int r = p / pr, c8 = p - r * pr;
            *reinterpret_cast<uint4*>(&xs[r * stride + c8 * 8]) = permute8(xr[i]);
        }
    }
    __syncthreads();

    float4_t acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[mb][t] = float4_t{0.f, 0.f, 0.f, 0.f};
    const SkConsts uk = sk_consts();

    // Ring slot d holds group g0 + gb + d. Refills are issued
    // unconditionally at a fixed place, so the compiler's wait counts track
    // the ring exactly; only the compute of groups past the range is skipped.
    const half_t* xcol = &xs[col * stride + 8 * lg * WPL];
    const uint32_t* szcol = &szs[(wave * 32 + col) * szst];
    for (int h0 = 0; h0 < g1 - g0; h0 += pg) {
        const int h1 = min(g1 - g0, h0 + pg);                // this phase: groups g0 + [h0, h1)
        if (h0 > 0) {
            // every wave is done with the previous phase's x and pairs
            __syncthreads();
            const int nsz_h = kSkBN * (h1 - h0), pr_h = (h1 - h0) * G / 8, pieces_h = MP * pr_h;
            for (int e = tid; e < nsz_h; e += kSkThreads) {
                const int c = e / (h1 - h0), gi = e - c * (h1 - h0);
                const int n = tile * kSkBN + c;
                const uint32_t so = n < N ? (static_cast<uint32_t>(n) * ng + g0 + h0 + gi) * 2 : sz_bytes;
                const uint16_t sv = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
                const uint16_t zv = __builtin_amdgcn_raw_buffer_load_b16(rz, so, 0, 0);
                szs[c * szst + gi] = static_cast<uint32_t>(sv) | (static_cast<uint32_t>(zv) << 16);
            }
            for (int pc = tid; pc < pieces_h; pc += kSkThreads) {
                const int r = pc / pr_h, c8 = pc - r * pr_h;
                const uint32_t off = r < M ? (static_cast<uint32_t>(r) * K + (g0 + h0) * G + c8 * 8) * 2 : x_bytes;
                *reinterpret_cast<uint4*>(&xs[r * stride + c8 * 8]) =
                    permute8(__builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0)));
            }
            __syncthreads();
        }
        for (int gb = h0; gb < h1; gb += kSkDepth) {
#pragma unroll
            for (int d = 0; d < kSkDepth; ++d) {
                const int gi = gb + d;                       // group g0 + gi, slot d
                GroupLoad<WPL>& gl = ring[d];
                if (gi < h1) {
                    half8_t bf[2][WPL];
                    float s[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const uint32_t sz = szcol[t * 16 * szst + gi - h0];
                        const half_t z = __builtin_bit_cast(half_t, static_cast<uint16_t>(sz >> 16));
                        const half_t zh = static_cast<half_t>(1024.0f) + z;   // exact
                        const half_t zl = static_cast<half_t>(64.0f) + z;     // exact
#pragma unroll
                        for (int j = 0; j < WPL; ++j)
                            bf[t][j] = unpack8(gl.w[t][j], half2_t{zh, zh}, half2_t{zl, zl}, uk);
                        s[t] = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(sz & 0xFFFFu)));
                    }
                    const half_t* xb = xcol + (gi - h0) * G;
                    float4_t part[MB][2];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int t = 0; t < 2; ++t) part[mb][t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < WPL; ++j) {
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            const half8_t a = *reinterpret_cast<const half8_t*>(xb + 16 * mb * stride + 8 * j);
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
                load_group(gl, g0 + gi + kSkDepth);              // refill the slot
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
    // partial tiles of this column tile, one per split:
    // [split][MB * 2 float4 chunks][512 threads]
    constexpr uint32_t kPartBytes = MB * 2 * kSkThreads * 16;
    const auto prs = rsrc(reinterpret_cast<char*>(partials) +
                              static_cast<int64_t>(tile) * splits * static_cast<int64_t>(kPartBytes),
                          static_cast<uint32_t>(splits) * kPartBytes);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[mb][t]), prs, tid * 16,
                                                   split * kPartBytes + (mb * 2 + t) * kSkThreads * 16, kSc1);
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
    // four splits' loads in flight at a time; splits past the last read
    // zero (past the descriptor's end), and the adds keep split order
    constexpr int kFix = 4;
    for (int sp = 0; sp < splits; sp += kFix) {
        float4_t v[kFix][MB][2];
#pragma unroll
        for (int f = 0; f < kFix; ++f)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    v[f][mb][t] = __builtin_bit_cast(
                        float4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                      prs, tid * 16, (sp + f) * kPartBytes + (mb * 2 + t) * kSkThreads * 16, kSc1));
#pragma unroll
        for (int f = 0; f < kFix; ++f)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < 2; ++t) sum[mb][t] += v[f][mb][t];
    }
    emit(sum);
    if (tid == 0) __hip_atomic_store(&counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int64_t sk_tiles(int64_t N) { return (N + kSkBN - 1) / kSkBN; }

int sk_mb(int64_t M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

// longest K range (whole groups, at most what kSkXP / kSkSZ cover) whose
// staged x and (scale, zero) pairs fit the LDS budget
int64_t sk_kmax(int64_t M, int group_size) {
    const int mb = sk_mb(M);
    const int64_t by_regs = std::min<int64_t>(static_cast<int64_t>(kSkXP) * kSkThreads * 8 / (16 * mb),
                                              static_cast<int64_t>(kSkSZ) * kSkThreads / kSkBN * group_size);
    int64_t kr = by_regs / group_size * group_size;
    while (kr > 0 && sk_lds_bytes(mb, static_cast<int>(kr), group_size) > kSkLds) kr -= group_size;
    return kr;
}

// partial tiles a workspace holds: splits x column tiles never exceed it
int64_t sk_max_parts() { return 3 * static_cast<int64_t>(cu_count()); }

size_t sk_partial_bytes(int64_t M) { return static_cast<size_t>(sk_mb(M)) * 2 * kSkThreads * 16; }

// How a shape runs: K splits across blocks (with a workspace) and, within a
// block, phases of at most `pg` groups staged in LDS one after the other.
// With a workspace, as many splits as fill one block per CU, each keeping
// at least 512 of K (shorter splits cost more in their partial tiles and
// fixup than they add in parallelism: M = 16 on 4096 x 4096 takes 10.4 us
// with 8 splits against 12.1 us with 16), and never fewer than keep each
// split inside the LDS, so every split is one phase. Without one (or with
// more column tiles than the workspace counts), one block per column tile
// walks all of K, in phases of a multiple of the ring depth when K exceeds
// the LDS. false = this shape cannot run here.
bool sk_plan(int64_t M, int64_t N, int64_t K, int group_size, bool have_workspace, int& splits, int& pg) {
    const int64_t tiles = sk_tiles(N);
    const int64_t ng = K / group_size;
    const int64_t gmax = sk_kmax(M, group_size) / group_size;
    if (gmax < 1) return false;
    const int64_t s_min = (ng + gmax - 1) / gmax;
    if (have_workspace && tiles <= split_counter_slots()) {
        int64_t s = std::max<int64_t>(s_min, std::min<int64_t>(cu_count() / tiles, std::max<int64_t>(1, K / 512)));
        while (s > s_min && s * tiles > sk_max_parts()) --s;
        if (s == 1 || s * tiles <= sk_max_parts()) {
            splits = static_cast<int>(s);
            pg = static_cast<int>((ng + s - 1) / s);
            return true;
        }
    }
    splits = 1;
    if (ng <= gmax) {
        pg = static_cast<int>(ng);
        return true;
    }
    const int64_t depth = sk_depth(sk_mb(M), group_size / 32);
    pg = static_cast<int>(gmax / depth * depth);
    return pg >= depth;
}

template <int MB, int WPL, int FORM>
awq_status launch_form(const half_t* x, const uint32_t* qweight, const half_t* scales, const half_t* zeros, int M,
                       int N, int K, half_t* y, int splits, int pg, float* partials, int* counters, size_t lds,
                       hipStream_t stream) {
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&skinny_kernel<MB, WPL, FORM>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kSkLds) != hipSuccess)
            return AWQ_ERR_HIP;
        attr_set = true;
    }
    if (M >= 128 || splits >= 512 || pg >= 65536) return AWQ_ERR_SHAPE;   // the packed msp fields
    const int64_t blocks = sk_tiles(N) * splits;
    hipLaunchKernelGGL((skinny_kernel<MB, WPL, FORM>), dim3(static_cast<unsigned>(blocks)), dim3(kSkThreads), lds,
                       stream, x, qweight, scales, zeros, y, N, K,
                       static_cast<uint32_t>(M) | (static_cast<uint32_t>(splits) << 7) |
                           (static_cast<uint32_t>(pg) << 16),
                       partials, counters);
    return last_launch_status();
}

template <int MB, int WPL>
awq_status launch_cfg(const half_t* x, const uint32_t* qweight, const half_t* scales, const half_t* zeros, int M,
                      int N, int K, half_t* y, void* workspace, hipStream_t stream) {
    int splits = 0, pg = 0;
    if (!sk_plan(M, N, K, WPL * 32, workspace != nullptr, splits, pg)) return AWQ_ERR_CONFIG;
    float* partials = nullptr;
    int* counters = nullptr;
    if (splits > 1) {
        counters = static_cast<int*>(workspace);
        partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + split_counter_bytes());
    }
    // the longest phase sets the LDS
    const size_t lds = static_cast<size_t>(sk_lds_bytes(MB, pg * WPL * 32, WPL * 32));
    // the smallest prologue that stages 16 MB rows of a phase's K range and
    // its (scale, zero) pairs
    auto fits = [&](int form) {
        return 16 * MB * (pg * WPL * 32 / 8) <= kSkXPForm[form] * kSkThreads &&
               kSkBN * pg <= kSkSZForm[form] * kSkThreads;
    };
    if (fits(0))
        return launch_form<MB, WPL, 0>(x, qweight, scales, zeros, M, N, K, y, splits, pg, partials, counters, lds,
                                          stream);
    if (fits(1))
        return launch_form<MB, WPL, 1>(x, qweight, scales, zeros, M, N, K, y, splits, pg, partials, counters, lds,
                                          stream);
    return launch_form<MB, WPL, 2>(x, qweight, scales, zeros, M, N, K, y, splits, pg, partials, counters, lds,
                                      stream);
}

template <int WPL>
awq_status launch_wpl(const half_t* x, const uint32_t* qweight, const half_t* scales, const half_t* zeros, int M,
                      int N, int K, half_t* y, void* workspace, hipStream_t stream) {
    switch (sk_mb(M)) {
        case 1: return launch_cfg<1, WPL>(x, qweight, scales, zeros, M, N, K, y, workspace, stream);
        case 2: return launch_cfg<2, WPL>(x, qweight, scales, zeros, M, N, K, y, workspace, stream);
        default: return launch_cfg<4, WPL>(x, qweight, scales, zeros, M, N, K, y, workspace, stream);
    }
}

}  // namespace

bool skinny_supported(int64_t M, int64_t N, int64_t K, int group_size, bool have_workspace, bool* phased) {
    // buffer offsets are 32-bit: the packed matrix plus one row of slack
    // (the largest offset a zero-reading lane forms), and x, stay below 4 GiB
    // group sizes 32 .. 256 (1 .. 8 packed words per lane and group)
    if (group_size > 256) return false;
    if (M < 1 || M > kSkinnyMaxM || N < 1 || (N + 1) * (K / 2) + 64 >= (int64_t{1} << 32) ||
        M * K * 2 + 64 >= (int64_t{1} << 32))
        return false;
    int splits = 0, pg = 0;
    if (!sk_plan(M, N, K, group_size, have_workspace, splits, pg)) return false;
    if (phased != nullptr) *phased = splits == 1 && pg < K / group_size;
    return true;
}

size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    (void)N;
    (void)K;
    if (M < 1 || M > kSkinnyMaxM) return 0;
    return split_counter_bytes() + static_cast<size_t>(sk_max_parts()) * sk_partial_bytes(M);
}

awq_status launch_skinny(const half_t* x, const uint32_t* qweight, const half_t* scales, const half_t* zeros,
                         int64_t M, int64_t N, int64_t K, int group_size, half_t* y, void* workspace,
                         hipStream_t stream) {
    if (M == 0 || N == 0) return AWQ_OK;
    if (!skinny_supported(M, N, K, group_size, workspace != nullptr)) return AWQ_ERR_CONFIG;
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    switch (group_size) {
        case 32: return launch_wpl<1>(x, qweight, scales, zeros, m, n, k, y, workspace, stream);
        case 64: return launch_wpl<2>(x, qweight, scales, zeros, m, n, k, y, workspace, stream);
        case 128: return launch_wpl<4>(x, qweight, scales, zeros, m, n, k, y, workspace, stream);
        case 256: return launch_wpl<8>(x, qweight, scales, zeros, m, n, k, y, workspace, stream);
        default: return AWQ_ERR_CONFIG;
    }
}

}  // namespace awq
