// HIP kernels for conv2d backward-data on CDNA4 (gfx950).
//
// One launch covers up to 16 stride phases (see dgrad_plan.h). Each workgroup
// owns one BM x BN tile of one phase's GEMM:
//     rows    = BM dx pixels of the phase lattice (h = ph + s*i, w = pw + s*j)
//     columns = BN dx channels
//     reduce  = the phase's taps x K, in BK-wide slices
// The operation is the backward-data convolution of "[CUTLASS] Conv2d dgrad"
// (apache/tvm PR #10110); the tile structure is this file's own, built for
// 64-lane waves, 160 KiB LDS and the 32x32x16 fp16 matrix-core instruction.
//
// Matrix-core mapping. v_mfma_f32_32x32x16_f16 computes a 32x32 fp32 block
// D += A(32x16) * B(16x32); each lane supplies 8 consecutive reduction
// elements of one A row and one B column, and holds 16 results of one D
// column. Here A = filter^T (rows = dx channels) and B = dy^T (columns = dx
// pixels), so every lane ends with 4 consecutive channels of one pixel per
// register group: a single 8-byte NHWC store per group.
//
// Operand staging (per BK slice, double-buffered in LDS, one barrier per slice):
//   dy: each 16-byte vector is 8 consecutive k of one gathered dy row
//       (n, i + dr, j + dt). Rows that fall outside [0,P) x [0,Q) are zero.
//       Written to LDS row = pixel, XOR-swizzled 16-byte chunks.
//   w : read as 8-byte vectors along c (the KRSC filter is c-contiguous),
//       eight k rows per thread, transposed in registers into 16-byte
//       k-contiguous vectors and written to LDS row = channel, swizzled alike.
//   The matrix-core reads are then plain 16-byte LDS reads for both operands.
//
// Epilogue: fp32 accumulator (times g(z) for the fused relu'/hardswish'
// variants) -> fp16 round-to-nearest-even -> 8-byte stores. dx is never read.
// Zero phases (no tap reaches the lattice) store zeros with 16-byte stores
// and never read z.
#include "dgrad_internal.h"

namespace cbw {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resources (V#) for raw, unswizzled 32-bit-format buffer accesses.
// A lane whose offset is at or past the buffer size reads zeros and has its
// store dropped by the hardware range check; kOutOfRange is such an offset
// for every tensor the host admits (all are below 2^31 bytes).
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;

// Byte offset for a buffer access: `off` itself (below 2^31 for an in-range
// lane), or exactly 2^31 when bad == 1. Arithmetic, not a select, so no branch
// is formed around the access. A caller may add up to 2^31 - 1 more bytes to
// a bad offset and still stay out of range without wrapping.
__device__ inline uint32_t out_of_range_if(uint32_t bad, uint32_t off)
{
    return (off & (bad - 1u)) | (bad << 31);
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRawBufferFlags);
}

constexpr int kEpiNone = 0;
constexpr int kEpiDRelu = 1;
constexpr int kEpiDHardswish = 2;

// Hardware dispatch places workgroup b on XCD (b mod 8) as that XCD's
// (b div 8)-th workgroup. Give each XCD whole groups of `g` consecutive
// logical tiles (the channel tiles of one pixel block share their dy rows in
// that XCD's L2), and rotate groups over XCDs so the heavy-first phase order
// stays balanced across XCDs. The tail that does not fill 8 groups keeps the
// identity mapping.
__device__ inline int xcd_group_remap(int b, int total, int g)
{
    const int span = 8 * g;
    const int main_part = (total / span) * span;
    if (b >= main_part)
        return b;
    const int x = b & 7;
    const int l = b >> 3;
    return ((l / g) * 8 + x) * g + (l % g);
}

// Two fp16 of column j (0..3) from two 4-wide rows, packed low/high.
template <int J>
__device__ inline uint32_t pack_column(u32x2 lo, u32x2 hi)
{
    const uint32_t a = (J < 2) ? lo.x : lo.y;
    const uint32_t b = (J < 2) ? hi.x : hi.y;
    if (J & 1)
        return (a >> 16) | (b & 0xffff0000u);
    return (a & 0xffffu) | (b << 16);
}

// g(z) for the fused epilogues, evaluated in fp32 without branches.
// relu'(z) = [z > 0]; hardswish'(z) = 0 below -3, z/3 + 1/2 on the closed
// interval [-3, 3], 1 above 3 (the division is correctly rounded).
__device__ inline float epilogue_factor(int epi, float z)
{
    const float relu = z > 0.0f ? 1.0f : 0.0f;
    const float mid = z / 3.0f + 0.5f;
    const float hsw = z < -3.0f ? 0.0f : (z > 3.0f ? 1.0f : mid);
    return epi == kEpiDRelu ? relu : (epi == kEpiDHardswish ? hsw : 1.0f);
}

// LDS rows are 128 bytes (8 chunks of 16 bytes). Chunk c of row r is stored
// at chunk position c ^ swizzle(r), so that the 16-byte accesses of
// neighbouring lanes (consecutive rows, same logical chunk) fall in distinct
// banks. SWZ 0 spreads each group of 8 consecutive rows over the 8 positions
// (a 128-byte bank window); SWZ 1 gives each pair of rows one position, which
// spreads 16 consecutive rows over a 256-byte window.
template <int SWZ>
__device__ inline int swizzle(int row)
{
    return SWZ == 0 ? (row & 7) : ((row >> 1) & 7);
}

template <int BM, int BN, int BK, int WM, int WN, int SWZ>
__global__ void __launch_bounds__(64 * WM * WN) dgrad_igemm(KernelArgs a)
{
    constexpr int NT = 64 * WM * WN;        // threads
    constexpr int TM = BM / WM;             // pixels per wave
    constexpr int TN = BN / WN;             // channels per wave
    constexpr int FM = TM / 32;             // 32x32 blocks per wave along pixels
    constexpr int FN = TN / 32;             // ... along channels
    constexpr int KCH = BK / 8;             // 16-byte chunks per LDS row
    constexpr int ROWS = BM + BN;           // LDS rows per stage: pixels, then channels
    constexpr int A_PER = BM * KCH / NT;    // dy vectors per thread per stage
    constexpr int A_ROW_STEP = NT / KCH;
    constexpr int B_BLK = KCH * (BN / 4);   // (8 k x 4 c) filter blocks per stage
    constexpr int B_PER = (B_BLK + NT - 1) / NT;
    static_assert(KCH == 8, "the LDS swizzle assumes 8 chunks (64 fp16) per row");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert((BM * KCH) % NT == 0, "dy vectors must divide evenly over threads");
    static_assert(2 * ROWS * KCH * 16 <= 160 * 1024, "LDS budget");

    __shared__ u32x4 lds[2 * ROWS * KCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;

    // ---- which tile of which phase
    const int tile = xcd_group_remap(blockIdx.x, a.total_tiles, a.group);
    int pi = 0;
    for (int i = 1; i < a.nphases; ++i)
        if (tile >= a.ph[i].tile_begin)
            pi = i;
    const PhaseArg ph = a.ph[pi];
    const int local = tile - ph.tile_begin;
    const int tm = local / a.tiles_n;
    const int tn = local - tm * a.tiles_n;
    const int m0 = tm * BM;
    const int c0 = tn * BN;
    const int s = a.stride;
    const int C = a.C;
    const int K = a.K;

    const __amdgpu_buffer_rsrc_t dx_rsrc = make_rsrc(a.dx, a.dx_bytes);

    // ---- zero phase: no tap reaches this lattice; dx is exactly 0 there
    if (ph.nr == 0 || ph.nt == 0) {
        constexpr int ZV = BN / 8;  // 16-byte vectors per pixel in the tile
        const u32x4 zero{0u, 0u, 0u, 0u};
        for (int u = tid; u < BM * ZV; u += NT) {
            const int row = u / ZV;
            const int c = c0 + (u - row * ZV) * 8;
            const int m = m0 + row;
            const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
            const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
            const uint32_t i = fastdiv(rem, ph.div_w);
            const uint32_t j = rem - i * (uint32_t)ph.Wp;
            const uint32_t pix = (n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)i)) * (uint32_t)a.W
                                 + (uint32_t)(ph.pw + s * (int)j);
            const uint32_t bad = (uint32_t)(m >= ph.M) | (uint32_t)(c >= C);
            __builtin_amdgcn_raw_buffer_store_b128(zero, dx_rsrc, out_of_range_if(bad, (pix * (uint32_t)C + (uint32_t)c) * 2u), 0, 0);
        }
        return;
    }

    const __amdgpu_buffer_rsrc_t dy_rsrc = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(a.w, a.w_bytes);

    // ---- the dy rows this thread gathers (fixed for the whole reduction)
    const int a_ch = tid % KCH;
    // Element offsets are kept modulo 2^32: a lattice row i may exceed P, so
    // the base "dy[n, i, j]" can lie outside dy, but every offset used for a
    // load, base + tap offset with 0 <= i + dr < P and 0 <= j + dt < Q, is exact.
    uint32_t a_off[A_PER];   // offset of dy[n, i, j, a_ch*8]
    int a_i[A_PER];
    int a_j[A_PER];
#pragma unroll
    for (int u = 0; u < A_PER; ++u) {
        const int row = tid / KCH + u * A_ROW_STEP;
        const int m = m0 + row;
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        const bool live = m < ph.M;
        a_i[u] = live ? (int)i : -(1 << 24);  // a dead row fails every p >= 0 test
        a_j[u] = (int)j;
        a_off[u] = ((n * (uint32_t)a.P + i) * (uint32_t)a.Q + j) * (uint32_t)K + (uint32_t)(a_ch * 8);
    }

    const int RSC = a.R * a.S * C;
    const int ksteps = (K + BK - 1) / BK;
    const int niter = ph.nr * ph.nt * ksteps;

    // Two register sets: slice it+2 is fetched while slice it+1 (fetched one
    // iteration earlier) is still in flight and slice it is on the matrix cores.
    u32x4 ra0[A_PER], ra1[A_PER];
    u32x2 rb0[B_PER][8], rb1[B_PER][8];

    // Global -> registers for reduction slice (tap ar, tap at, channels k0..k0+BK).
    // Out-of-range lanes use kOutOfRange and receive zeros from the hardware.
    auto load_stage = [&](int ar, int at, int k0, u32x4 (&ra)[A_PER], u32x2 (&rb)[B_PER][8]) {
        const int dr = ph.dr0 - ar;
        const int dt = ph.dt0 - at;
        const uint32_t tap_off = (uint32_t)(dr * a.Q + dt) * (uint32_t)K + (uint32_t)k0;
        const uint32_t k_bad = (uint32_t)(k0 + a_ch * 8 >= K);
#pragma unroll
        for (int u = 0; u < A_PER; ++u) {
            const uint32_t bad = k_bad | (uint32_t)((unsigned)(a_i[u] + dr) >= (unsigned)a.P) |
                                 (uint32_t)((unsigned)(a_j[u] + dt) >= (unsigned)a.Q);
            ra[u] = __builtin_amdgcn_raw_buffer_load_b128(dy_rsrc, out_of_range_if(bad, (a_off[u] + tap_off) * 2u), 0, 0);
        }
        const int r = ph.r0 + ar * s;
        const int t = ph.t0 + at * s;
        const int w_tap = (r * a.S + t) * C;
#pragma unroll
        for (int v = 0; v < B_PER; ++v) {
            const int u = tid + v * NT;
            const int kc = u % KCH;
            const int cq = u / KCH;
            const int k = k0 + kc * 8;
            const int c = c0 + cq * 4;
            const uint32_t bad = (uint32_t)(B_BLK % NT != 0 && u >= B_BLK) | (uint32_t)(k >= K) | (uint32_t)(c >= C);
            const uint32_t off = out_of_range_if(bad, (uint32_t)(k * RSC + w_tap + c) * 2u);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)   // 7*RSC*2 < 2^31 / 8: a bad offset stays in [2^31, 2^32)
                rb[v][kk] = __builtin_amdgcn_raw_buffer_load_b64(w_rsrc, off + (uint32_t)(kk * RSC) * 2u, 0, 0);
        }
    };

    // Registers -> LDS stage `buf` (swizzled; the filter block transposed).
    auto store_stage = [&](int buf, const u32x4 (&ra)[A_PER], const u32x2 (&rb)[B_PER][8]) {
        u32x4* L = lds + buf * (ROWS * KCH);
#pragma unroll
        for (int u = 0; u < A_PER; ++u) {
            const int row = tid / KCH + u * A_ROW_STEP;
            L[row * KCH + (a_ch ^ swizzle<SWZ>(row))] = ra[u];
        }
#pragma unroll
        for (int v = 0; v < B_PER; ++v) {
            const int u = tid + v * NT;
            if (B_BLK % NT == 0 || u < B_BLK) {
                const int kc = u % KCH;
                const int cq = u / KCH;
                const u32x2* b = rb[v];
                const u32x4 col0{pack_column<0>(b[0], b[1]), pack_column<0>(b[2], b[3]),
                                 pack_column<0>(b[4], b[5]), pack_column<0>(b[6], b[7])};
                const u32x4 col1{pack_column<1>(b[0], b[1]), pack_column<1>(b[2], b[3]),
                                 pack_column<1>(b[4], b[5]), pack_column<1>(b[6], b[7])};
                const u32x4 col2{pack_column<2>(b[0], b[1]), pack_column<2>(b[2], b[3]),
                                 pack_column<2>(b[4], b[5]), pack_column<2>(b[6], b[7])};
                const u32x4 col3{pack_column<3>(b[0], b[1]), pack_column<3>(b[2], b[3]),
                                 pack_column<3>(b[4], b[5]), pack_column<3>(b[6], b[7])};
                const int r0 = BM + cq * 4;
                L[(r0 + 0) * KCH + (kc ^ swizzle<SWZ>(r0 + 0))] = col0;
                L[(r0 + 1) * KCH + (kc ^ swizzle<SWZ>(r0 + 1))] = col1;
                L[(r0 + 2) * KCH + (kc ^ swizzle<SWZ>(r0 + 2))] = col2;
                L[(r0 + 3) * KCH + (kc ^ swizzle<SWZ>(r0 + 3))] = col3;
            }
        }
    };

    float16_t acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[fn][fm][e] = 0.0f;

    // One BK slice on the matrix cores. Fragments are double-buffered across
    // the 16-wide sub-steps: the LDS reads for sub-step kk+1 are issued before
    // the MFMAs of sub-step kk, so LDS latency overlaps matrix-core work.
    auto read_frags = [&](const u32x4* L, int kk, half8_t (&af)[FN], half8_t (&bf)[FM]) {
        const int lc = kk * 2 + (lane >> 5);  // this lane's 8-wide k chunk
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int row = BM + wn * TN + fn * 32 + (lane & 31);
            af[fn] = __builtin_bit_cast(half8_t, L[row * KCH + (lc ^ swizzle<SWZ>(row))]);
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int row = wm * TM + fm * 32 + (lane & 31);
            bf[fm] = __builtin_bit_cast(half8_t, L[row * KCH + (lc ^ swizzle<SWZ>(row))]);
        }
    };
    auto mfma_step = [&](const half8_t (&af)[FN], const half8_t (&bf)[FM]) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[fn], bf[fm], acc[fn][fm], 0, 0, 0);
    };
    auto compute_stage = [&](int buf) {
        const u32x4* L = lds + buf * (ROWS * KCH);
        half8_t af0[FN], bf0[FM], af1[FN], bf1[FM];
        static_assert(BK / 16 == 4, "four sub-steps per slice");
        read_frags(L, 0, af0, bf0);
        read_frags(L, 1, af1, bf1);
        mfma_step(af0, bf0);
        read_frags(L, 2, af0, bf0);
        mfma_step(af1, bf1);
        read_frags(L, 3, af1, bf1);
        mfma_step(af0, bf0);
        mfma_step(af1, bf1);
    };

    // ---- main loop. Slice it is consumed from LDS buffer it%2 while slice
    // it+1 (requested one iteration earlier) is in flight and slice it+2 is
    // requested; slice it+1 is then written to the other buffer. Each of the
    // two register sets is a fixed set of VGPRs (the loop is unrolled by two)
    // and the steady state requests unconditionally, so the wait before an
    // LDS write covers only the older batch: loads get two slices to land.
    int ar = 0, at = 0, k0 = 0;   // cursor of the next slice to request
    auto request = [&](u32x4 (&ra)[A_PER], u32x2 (&rb)[B_PER][8]) {
        load_stage(ar, at, k0, ra, rb);
        k0 += BK;
        if (k0 >= K) {
            k0 = 0;
            if (++at == ph.nt) {
                at = 0;
                ++ar;
            }
        }
    };
    request(ra0, rb0);
    store_stage(0, ra0, rb0);
    if (niter > 1)
        request(ra1, rb1);
    __syncthreads();
    int it = 0;
    for (; it + 3 < niter; it += 2) {
        request(ra0, rb0);            // slice it+2
        compute_stage(0);             // slice it
        store_stage(1, ra1, rb1);     // slice it+1
        __syncthreads();
        request(ra1, rb1);            // slice it+3
        compute_stage(1);             // slice it+1
        store_stage(0, ra0, rb0);     // slice it+2
        __syncthreads();
    }
    // 1 to 3 slices remain; slice it is in buffer 0, slice it+1 in register set 1
    if (it + 2 < niter) {
        request(ra0, rb0);
        compute_stage(0);
        store_stage(1, ra1, rb1);
        __syncthreads();
        compute_stage(1);
        store_stage(0, ra0, rb0);
        __syncthreads();
        compute_stage(0);
    } else if (it + 1 < niter) {
        compute_stage(0);
        store_stage(1, ra1, rb1);
        __syncthreads();
        compute_stage(1);
    } else {
        compute_stage(0);
    }

    // ---- epilogue: lane holds channels c..c+3 of pixel m per register group.
    // Out-of-range lanes store to kOutOfRange, which the hardware drops.
    const int epi = a.epi;
    const __amdgpu_buffer_rsrc_t z_rsrc = make_rsrc(epi != kEpiNone ? a.z : a.dx, a.dx_bytes);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm * TM + fm * 32 + (lane & 31);
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        const uint32_t pix = (n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)i)) * (uint32_t)a.W
                             + (uint32_t)(ph.pw + s * (int)j);
        const uint32_t m_bad = (uint32_t)(m >= ph.M);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = c0 + wn * TN + fn * 32 + 8 * g + 4 * (lane >> 5);
                const uint32_t off = out_of_range_if(m_bad | (uint32_t)(c >= C), (pix * (uint32_t)C + (uint32_t)c) * 2u);
                float v0 = acc[fn][fm][4 * g + 0];
                float v1 = acc[fn][fm][4 * g + 1];
                float v2 = acc[fn][fm][4 * g + 2];
                float v3 = acc[fn][fm][4 * g + 3];
                if (epi != kEpiNone) {
                    const half4_t zz = __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(z_rsrc, off, 0, 0));
                    v0 *= epilogue_factor(epi, (float)zz[0]);
                    v1 *= epilogue_factor(epi, (float)zz[1]);
                    v2 *= epilogue_factor(epi, (float)zz[2]);
                    v3 *= epilogue_factor(epi, (float)zz[3]);
                }
                const half4_t o{(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), dx_rsrc, off, 0, 0);
            }
        }
    }
}

// ============================================================================
// Direct-to-LDS variant.
//
// Both operands travel HBM/L2 -> LDS with 16-byte buffer loads that write LDS
// directly (each wave instruction fills a contiguous 1 KiB block, lane l at
// +16*l; out-of-range lanes write zeros), so no staging registers are needed.
// Three LDS stages form a ring: slice it+2 is requested while slice it is on
// the matrix cores. The loads are issued from inline assembly and waited for
// with explicit counts: the compiler's own wait insertion does not tell LDS
// buffers apart and would otherwise wait for every outstanding load before
// any LDS read.
//
// The filter slice is kept as it arrives, one row per k
// (channel-contiguous, as the KRSC layout stores it), and the MFMA operand
// (8 consecutive k of one channel per lane) is formed by the gfx950 LDS
// transpose read: within each group of 16 lanes, lane 4r+q reads row r,
// channels 4q..4q+3, and lane i receives channel i of the four rows. Two such
// reads give the eight k of one 32x16 operand fragment.
//
// LDS layouts (per stage):
//   dy slice: BM rows x 128 bytes (64 k); chunk c of row m at position
//             c ^ ((m >> 1) & 7)  -- conflict-free 16-byte reads for 16 lanes
//   w  slice: 64 rows (k) x 2*BN bytes; 16-byte chunk c of row k at position
//             c ^ (2 * (k & 3))   -- a 16-lane group's four rows hit distinct banks
// ============================================================================

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Buffer descriptor as four dwords (base, stride 0, size, raw 32-bit format).
__device__ inline i32x4 raw_descriptor(const void* base, uint32_t bytes)
{
    const uint64_t p = (uint64_t)base;
    return i32x4{(int)(uint32_t)p, (int)((p >> 32) & 0xffffu), (int)bytes, kRawBufferFlags};
}

// One 16-byte direct-to-LDS load per lane: LDS[lds_base + 16 * lane] <- buffer[voffset].
__device__ inline void dma16(i32x4 desc, uint32_t voffset, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(desc), "s"(lds_base)
                 : "memory", "m0");
}

template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) dgrad_igemm_dma(KernelArgs a)
{
    constexpr int BK = 64;
    constexpr int NW = WM * WN;
    constexpr int NT = 64 * NW;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int A_BYTES = BM * 2 * BK;          // dy slice
    constexpr int B_ROW = BN * 2;                 // one k row of the filter slice
    constexpr int B_BYTES = BK * B_ROW;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int NSTAGE = 3;
    constexpr int A_INSTR = A_BYTES / 1024 / NW;  // 1 KiB blocks per wave per slice
    constexpr int B_INSTR = B_BYTES / 1024 / NW;
    constexpr int LD = A_INSTR + B_INSTR;         // loads per lane per slice
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole 1 KiB blocks per wave");
    static_assert(BN % 64 == 0, "filter rows of at least 8 chunks");
    static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS budget");
    static_assert(2 * LD < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE];
    const uint32_t lds_u32 = (uint32_t)(uintptr_t)((lds_char*)lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;
    const int wn = wave / WM;

    const int tile = xcd_group_remap(blockIdx.x, a.total_tiles, a.group);
    int pi = 0;
    for (int i = 1; i < a.nphases; ++i)
        if (tile >= a.ph[i].tile_begin)
            pi = i;
    const PhaseArg ph = a.ph[pi];
    const int local = tile - ph.tile_begin;
    const int tm = local / a.tiles_n;
    const int tn = local - tm * a.tiles_n;
    const int m0 = tm * BM;
    const int c0 = tn * BN;
    const int s = a.stride;
    const int C = a.C;
    const int K = a.K;

    const __amdgpu_buffer_rsrc_t dx_rsrc = make_rsrc(a.dx, a.dx_bytes);

    if (ph.nr == 0 || ph.nt == 0) {  // zero phase
        constexpr int ZV = BN / 8;
        const u32x4 zero{0u, 0u, 0u, 0u};
        for (int u = tid; u < BM * ZV; u += NT) {
            const int row = u / ZV;
            const int c = c0 + (u - row * ZV) * 8;
            const int m = m0 + row;
            const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
            const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
            const uint32_t i = fastdiv(rem, ph.div_w);
            const uint32_t j = rem - i * (uint32_t)ph.Wp;
            const uint32_t pix = (n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)i)) * (uint32_t)a.W
                                 + (uint32_t)(ph.pw + s * (int)j);
            const uint32_t bad = (uint32_t)(m >= ph.M) | (uint32_t)(c >= C);
            __builtin_amdgcn_raw_buffer_store_b128(zero, dx_rsrc, out_of_range_if(bad, (pix * (uint32_t)C + (uint32_t)c) * 2u), 0, 0);
        }
        return;
    }

    const i32x4 dy_desc = raw_descriptor(a.dy, a.dy_bytes);
    const i32x4 w_desc = raw_descriptor(a.w, a.w_bytes);

    // ---- this lane's dy rows: DMA block b = j*NW + wave covers tile rows 8b..8b+7;
    // lane l fills row 8b + l/8, LDS chunk position l%8, i.e. logical chunk
    // (l%8) ^ swizzle(row).
    uint32_t a_off[A_INSTR];   // element offset of dy[n, i, j, chunk*8], modulo 2^32
    int a_i[A_INSTR], a_j[A_INSTR], a_k[A_INSTR];
#pragma unroll
    for (int jn = 0; jn < A_INSTR; ++jn) {
        const int row = (jn * NW + wave) * 8 + (lane >> 3);
        const int m = m0 + row;
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        a_i[jn] = m < ph.M ? (int)i : -(1 << 24);
        a_j[jn] = (int)j;
        a_k[jn] = ((lane & 7) ^ swizzle<1>(row)) * 8;
        a_off[jn] = ((n * (uint32_t)a.P + i) * (uint32_t)a.Q + j) * (uint32_t)K + (uint32_t)a_k[jn];
    }
    // ---- this lane's filter pieces: block b = j*NW + wave of the filter slice,
    // byte 16*l of it = row k, position p; logical chunk p ^ 2*(k & 3).
    int b_k[B_INSTR], b_c[B_INSTR];
#pragma unroll
    for (int jn = 0; jn < B_INSTR; ++jn) {
        const int byte = (jn * NW + wave) * 1024 + 16 * lane;
        const int k = byte / B_ROW;
        const int pos = (byte % B_ROW) / 16;
        b_k[jn] = k;
        b_c[jn] = (pos ^ (2 * (k & 3))) * 8;
    }

    const int RSC = a.R * a.S * C;
    const int ksteps = (K + BK - 1) / BK;
    const int niter = ph.nr * ph.nt * ksteps;

    int ar = 0, at = 0, k0 = 0;   // cursor of the next slice to request
    auto request = [&](int buf) {
        const int dr = ph.dr0 - ar;
        const int dt = ph.dt0 - at;
        const uint32_t tap_off = (uint32_t)(dr * a.Q + dt) * (uint32_t)K + (uint32_t)k0;
        const uint32_t stage_base = lds_u32 + (uint32_t)(buf * STAGE);
#pragma unroll
        for (int jn = 0; jn < A_INSTR; ++jn) {
            const uint32_t bad = (uint32_t)(k0 + a_k[jn] >= K) | (uint32_t)((unsigned)(a_i[jn] + dr) >= (unsigned)a.P) |
                                 (uint32_t)((unsigned)(a_j[jn] + dt) >= (unsigned)a.Q);
            dma16(dy_desc, out_of_range_if(bad, (a_off[jn] + tap_off) * 2u),
                  stage_base + (uint32_t)((jn * NW + wave) * 1024));
        }
        const int r = ph.r0 + ar * s;
        const int t = ph.t0 + at * s;
        const int w_tap = (r * a.S + t) * C;
#pragma unroll
        for (int jn = 0; jn < B_INSTR; ++jn) {
            const int k = k0 + b_k[jn];
            const int c = c0 + b_c[jn];
            const uint32_t bad = (uint32_t)(k >= K) | (uint32_t)(c >= C);
            dma16(w_desc, out_of_range_if(bad, (uint32_t)(k * RSC + w_tap + c) * 2u),
                  stage_base + (uint32_t)(A_BYTES + (jn * NW + wave) * 1024));
        }
        k0 += BK;
        if (k0 >= K) {
            k0 = 0;
            if (++at == ph.nt) {
                at = 0;
                ++ar;
            }
        }
    };

    // ---- fragment addresses (bytes within a stage, sub-step 0)
    // dy^T operand (B): row m = wm*TM + fm*32 + lane%32, k chunk 2*kk + lane/32.
    const int b_row0 = wm * TM + (lane & 31);
    const int b_sw = swizzle<1>(b_row0);          // same for every fm (fm*32 keeps bits 1..3)
    // filter^T operand (A): group g = lane/16 covers channels +16*(g&1), k +8*(g>>1);
    // within it lane 4r+q reads row r, channels 4q..4q+3.
    const int g = (lane >> 4) & 3;
    const int rr = (lane & 15) >> 2;
    const int qq = lane & 3;
    int a_frag[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int cl = wn * TN + fn * 32 + (g & 1) * 16 + 4 * qq;   // first channel this lane reads
        const int krow = (g >> 1) * 8 + rr;
        a_frag[fn] = A_BYTES + krow * B_ROW + (((cl >> 3) ^ (2 * rr)) * 16) + (cl & 7) * 2;
    }

    float16_t acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[fn][fm][e] = 0.0f;

    auto read_frags = [&](int sb, int kk, half8_t (&af)[FN], half8_t (&bf)[FM]) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const lds_char* p = (lds_char*)lds + sb + a_frag[fn] + kk * 16 * B_ROW;
            const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)p);
            const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p + 4 * B_ROW));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
            af[fn] = __builtin_bit_cast(half8_t, u32x4{l2.x, l2.y, h2.x, h2.y});
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int off = sb + (b_row0 + fm * 32) * 128 + (((kk * 2 + (lane >> 5)) ^ b_sw) * 16);
            bf[fm] = __builtin_bit_cast(half8_t, *(const u32x4*)(lds + off));
        }
    };
    auto mfma_step = [&](const half8_t (&af)[FN], const half8_t (&bf)[FM]) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[fn], bf[fm], acc[fn][fm], 0, 0, 0);
    };
    auto compute = [&](int buf) {
        const int sb = buf * STAGE;
        half8_t af0[FN], bf0[FM], af1[FN], bf1[FM];
        read_frags(sb, 0, af0, bf0);
        read_frags(sb, 1, af1, bf1);
        mfma_step(af0, bf0);
        read_frags(sb, 2, af0, bf0);
        mfma_step(af1, bf1);
        read_frags(sb, 3, af1, bf1);
        mfma_step(af0, bf0);
        mfma_step(af1, bf1);
    };

    // ---- main loop over a ring of three LDS stages
    request(0);
    if (niter > 1)
        request(1);
    int buf = 0;
    for (int it = 0; it < niter; ++it) {
        if (it + 1 < niter)
            wait_vmcnt<LD>();        // slice it landed (slice it+1 may still fly)
        else
            wait_vmcnt<0>();
        __syncthreads();             // every wave's part of slice it is in LDS, and
                                     // every wave is done with slice it-1's buffer
        if (it + 2 < niter)
            request(buf == 0 ? 2 : buf - 1);   // buffer (it+2) % 3
        compute(buf);
        buf = buf == 2 ? 0 : buf + 1;
    }

    // ---- epilogue (as in the register-staged kernel)
    const int epi = a.epi;
    const __amdgpu_buffer_rsrc_t z_rsrc = make_rsrc(epi != kEpiNone ? a.z : a.dx, a.dx_bytes);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm * TM + fm * 32 + (lane & 31);
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        const uint32_t pix = (n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)i)) * (uint32_t)a.W
                             + (uint32_t)(ph.pw + s * (int)j);
        const uint32_t m_bad = (uint32_t)(m >= ph.M);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int c = c0 + wn * TN + fn * 32 + 8 * gq + 4 * (lane >> 5);
                const uint32_t off = out_of_range_if(m_bad | (uint32_t)(c >= C), (pix * (uint32_t)C + (uint32_t)c) * 2u);
                float v0 = acc[fn][fm][4 * gq + 0];
                float v1 = acc[fn][fm][4 * gq + 1];
                float v2 = acc[fn][fm][4 * gq + 2];
                float v3 = acc[fn][fm][4 * gq + 3];
                if (epi != kEpiNone) {
                    const half4_t zz = __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(z_rsrc, off, 0, 0));
                    v0 *= epilogue_factor(epi, (float)zz[0]);
                    v1 *= epilogue_factor(epi, (float)zz[1]);
                    v2 *= epilogue_factor(epi, (float)zz[2]);
                    v3 *= epilogue_factor(epi, (float)zz[3]);
                }
                const half4_t o{(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), dx_rsrc, off, 0, 0);
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_dma(const KernelArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((dgrad_igemm_dma<BM, BN, WM, WN>), dim3(a.total_tiles), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

#define CBW_CONFIG(BM, BN, BK, WM, WN, SWZ) \
    {BM, BN, BK, WM, WN, #BM "x" #BN "x" #BK "/" #WM "x" #WN "/s" #SWZ, 2 * (BM + BN) * BK * 2}
#define CBW_DMA_CONFIG(BM, BN, WM, WN) \
    {BM, BN, 64, WM, WN, #BM "x" #BN "x64/" #WM "x" #WN "/d", 3 * (BM + BN) * 64 * 2}

const TileConfig kConfigs[] = {
    CBW_CONFIG(128, 128, 64, 2, 2, 0),
    CBW_CONFIG(256, 128, 64, 2, 2, 0),
    CBW_CONFIG(128, 64, 64, 2, 2, 0),
    CBW_CONFIG(64, 64, 64, 2, 2, 0),
    CBW_CONFIG(128, 256, 64, 2, 2, 0),
    CBW_CONFIG(256, 64, 64, 4, 1, 0),
    CBW_CONFIG(128, 128, 64, 2, 2, 1),
    CBW_CONFIG(256, 128, 64, 2, 2, 1),
    CBW_CONFIG(128, 64, 64, 2, 2, 1),
    CBW_CONFIG(64, 64, 64, 2, 2, 1),
    CBW_CONFIG(128, 256, 64, 2, 2, 1),
    CBW_CONFIG(256, 64, 64, 4, 1, 1),
    CBW_DMA_CONFIG(256, 128, 2, 2),
    CBW_DMA_CONFIG(128, 128, 2, 2),
    CBW_DMA_CONFIG(128, 256, 2, 2),
    CBW_DMA_CONFIG(256, 64, 4, 1),
    CBW_DMA_CONFIG(128, 64, 2, 2),
    CBW_DMA_CONFIG(64, 64, 2, 2),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

template <int BM, int BN, int BK, int WM, int WN, int SWZ>
hipError_t launch(const KernelArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((dgrad_igemm<BM, BN, BK, WM, WN, SWZ>), dim3(a.total_tiles), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int num_tile_configs() { return kNumConfigs; }

const TileConfig& tile_config(int id) { return kConfigs[id]; }

hipError_t launch_tile_config(int id, const KernelArgs& a, hipStream_t stream)
{
    switch (id) {
    case 0: return launch<128, 128, 64, 2, 2, 0>(a, stream);
    case 1: return launch<256, 128, 64, 2, 2, 0>(a, stream);
    case 2: return launch<128, 64, 64, 2, 2, 0>(a, stream);
    case 3: return launch<64, 64, 64, 2, 2, 0>(a, stream);
    case 4: return launch<128, 256, 64, 2, 2, 0>(a, stream);
    case 5: return launch<256, 64, 64, 4, 1, 0>(a, stream);
    case 6: return launch<128, 128, 64, 2, 2, 1>(a, stream);
    case 7: return launch<256, 128, 64, 2, 2, 1>(a, stream);
    case 8: return launch<128, 64, 64, 2, 2, 1>(a, stream);
    case 9: return launch<64, 64, 64, 2, 2, 1>(a, stream);
    case 10: return launch<128, 256, 64, 2, 2, 1>(a, stream);
    case 11: return launch<256, 64, 64, 4, 1, 1>(a, stream);
    case 12: return launch_dma<256, 128, 2, 2>(a, stream);
    case 13: return launch_dma<128, 128, 2, 2>(a, stream);
    case 14: return launch_dma<128, 256, 2, 2>(a, stream);
    case 15: return launch_dma<256, 64, 4, 1>(a, stream);
    case 16: return launch_dma<128, 64, 2, 2>(a, stream);
    case 17: return launch_dma<64, 64, 2, 2>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace cbw
