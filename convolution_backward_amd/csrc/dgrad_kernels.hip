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

__device__ inline float epilogue_factor(int epi, float z)
{
    if (epi == kEpiDRelu)
        return z > 0.0f ? 1.0f : 0.0f;
    if (epi == kEpiDHardswish)  // 0 below -3, z/3 + 1/2 on the closed interval [-3, 3], 1 above 3
        return z < -3.0f ? 0.0f : (z > 3.0f ? 1.0f : z / 3.0f + 0.5f);
    return 1.0f;
}

template <int BM, int BN, int BK, int WM, int WN>
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

    // ---- zero phase: no tap reaches this lattice; dx is exactly 0 there
    if (ph.nr == 0 || ph.nt == 0) {
        constexpr int ZV = BN / 8;  // 16-byte vectors per pixel in the tile
        for (int u = tid; u < BM * ZV; u += NT) {
            const int row = u / ZV;
            const int c = c0 + (u - row * ZV) * 8;
            const int m = m0 + row;
            if (m < ph.M && c < C) {
                const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
                const uint32_t rem = (uint32_t)m - n * (uint32_t)(ph.div_hw.d);
                const uint32_t i = fastdiv(rem, ph.div_w);
                const uint32_t j = rem - i * (uint32_t)ph.Wp;
                const int h = ph.ph + s * (int)i;
                const int x = ph.pw + s * (int)j;
                const int pix = (((int)n * a.H + h) * a.W + x) * C;
                *reinterpret_cast<u32x4*>(a.dx + pix + c) = u32x4{0u, 0u, 0u, 0u};
            }
        }
        return;
    }

    // ---- the dy rows this thread gathers (fixed for the whole reduction)
    const int a_ch = tid % KCH;
    // Offsets are kept modulo 2^32: a lattice row i may exceed P, so the base
    // of "dy[n, i, j]" can lie outside dy, but every offset actually loaded,
    // base + tap offset with 0 <= i + dr < P and 0 <= j + dt < Q, is exact.
    uint32_t a_off[A_PER];   // offset of dy[n, i, j, a_ch*8]
    int a_i[A_PER];
    int a_j[A_PER];
#pragma unroll
    for (int u = 0; u < A_PER; ++u) {
        const int row = tid / KCH + u * A_ROW_STEP;
        const int m = m0 + row;
        if (m < ph.M) {
            const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
            const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
            const uint32_t i = fastdiv(rem, ph.div_w);
            const uint32_t j = rem - i * (uint32_t)ph.Wp;
            a_i[u] = (int)i;
            a_j[u] = (int)j;
            a_off[u] = ((n * (uint32_t)a.P + i) * (uint32_t)a.Q + j) * (uint32_t)K + (uint32_t)(a_ch * 8);
        } else {
            a_i[u] = -(1 << 24);  // every tap then lands at p < 0: never loaded
            a_j[u] = 0;
            a_off[u] = 0u;
        }
    }

    const int RSC = a.R * a.S * C;
    const int ksteps = (K + BK - 1) / BK;
    const int niter = ph.nr * ph.nt * ksteps;

    u32x4 ra[A_PER];
    u32x2 rb[B_PER][8];

    // Global -> registers for reduction slice (tap ar, tap at, channels k0..k0+BK).
    auto load_stage = [&](int ar, int at, int k0) {
        const int dr = ph.dr0 - ar;
        const int dt = ph.dt0 - at;
        const uint32_t tap_off = (uint32_t)(dr * a.Q + dt) * (uint32_t)K + (uint32_t)k0;
        const bool k_ok = k0 + a_ch * 8 < K;
#pragma unroll
        for (int u = 0; u < A_PER; ++u) {
            const int p = a_i[u] + dr;
            const int q = a_j[u] + dt;
            if (k_ok && (unsigned)p < (unsigned)a.P && (unsigned)q < (unsigned)a.Q)
                ra[u] = *reinterpret_cast<const u32x4*>(a.dy + (a_off[u] + tap_off));
            else
                ra[u] = u32x4{0u, 0u, 0u, 0u};
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
            const bool ok = (B_BLK % NT == 0 || u < B_BLK) && k < K && c < C;
            const uint16_t* src = a.w + k * RSC + w_tap + c;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                rb[v][kk] = ok ? *reinterpret_cast<const u32x2*>(src + kk * RSC) : u32x2{0u, 0u};
        }
    };

    // Registers -> LDS stage `buf` (swizzled; the filter block transposed).
    auto store_stage = [&](int buf) {
        u32x4* L = lds + buf * (ROWS * KCH);
#pragma unroll
        for (int u = 0; u < A_PER; ++u) {
            const int row = tid / KCH + u * A_ROW_STEP;
            L[row * KCH + (a_ch ^ (row & 7))] = ra[u];
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
                L[(r0 + 0) * KCH + (kc ^ ((r0 + 0) & 7))] = col0;
                L[(r0 + 1) * KCH + (kc ^ ((r0 + 1) & 7))] = col1;
                L[(r0 + 2) * KCH + (kc ^ ((r0 + 2) & 7))] = col2;
                L[(r0 + 3) * KCH + (kc ^ ((r0 + 3) & 7))] = col3;
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

    auto compute_stage = [&](int buf) {
        const u32x4* L = lds + buf * (ROWS * KCH);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int lc = kk * 2 + (lane >> 5);  // this lane's 8-wide k chunk
            half8_t af[FN];
            half8_t bf[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int row = BM + wn * TN + fn * 32 + (lane & 31);
                af[fn] = __builtin_bit_cast(half8_t, L[row * KCH + (lc ^ (row & 7))]);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = wm * TM + fm * 32 + (lane & 31);
                bf[fm] = __builtin_bit_cast(half8_t, L[row * KCH + (lc ^ (row & 7))]);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[fn], bf[fm], acc[fn][fm], 0, 0, 0);
        }
    };

    // ---- main loop: prefetch slice it+1 into registers while the matrix
    // cores consume slice it from LDS; one barrier per slice.
    int ar = 0, at = 0, k0 = 0;
    load_stage(ar, at, k0);
    store_stage(0);
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
        const bool more = it + 1 < niter;
        if (more) {
            k0 += BK;
            if (k0 >= K) {
                k0 = 0;
                if (++at == ph.nt) {
                    at = 0;
                    ++ar;
                }
            }
            load_stage(ar, at, k0);
        }
        compute_stage(it & 1);
        if (more)
            store_stage((it + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds channels c..c+3 of pixel m per register group
    const int epi = a.epi;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm * TM + fm * 32 + (lane & 31);
        if (m >= ph.M)
            continue;
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        const int h = ph.ph + s * (int)i;
        const int x = ph.pw + s * (int)j;
        const int pix = (((int)n * a.H + h) * a.W + x) * C;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = c0 + wn * TN + fn * 32 + 8 * g + 4 * (lane >> 5);
                if (c >= C)
                    continue;
                float v0 = acc[fn][fm][4 * g + 0];
                float v1 = acc[fn][fm][4 * g + 1];
                float v2 = acc[fn][fm][4 * g + 2];
                float v3 = acc[fn][fm][4 * g + 3];
                if (epi != kEpiNone) {
                    const half4_t zz = __builtin_bit_cast(half4_t, *reinterpret_cast<const u32x2*>(a.z + pix + c));
                    v0 *= epilogue_factor(epi, (float)zz[0]);
                    v1 *= epilogue_factor(epi, (float)zz[1]);
                    v2 *= epilogue_factor(epi, (float)zz[2]);
                    v3 *= epilogue_factor(epi, (float)zz[3]);
                }
                const half4_t o{(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
                *reinterpret_cast<u32x2*>(a.dx + pix + c) = __builtin_bit_cast(u32x2, o);
            }
        }
    }
}

#define CBW_CONFIG(BM, BN, BK, WM, WN) \
    {BM, BN, BK, WM, WN, #BM "x" #BN "x" #BK "/" #WM "x" #WN, 2 * (BM + BN) * BK * 2}

const TileConfig kConfigs[] = {
    CBW_CONFIG(128, 128, 64, 2, 2),
    CBW_CONFIG(256, 128, 64, 2, 2),
    CBW_CONFIG(128, 64, 64, 2, 2),
    CBW_CONFIG(64, 64, 64, 2, 2),
    CBW_CONFIG(128, 256, 64, 2, 2),
    CBW_CONFIG(256, 64, 64, 4, 1),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

template <int BM, int BN, int BK, int WM, int WN>
hipError_t launch(const KernelArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((dgrad_igemm<BM, BN, BK, WM, WN>), dim3(a.total_tiles), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int num_tile_configs() { return kNumConfigs; }

const TileConfig& tile_config(int id) { return kConfigs[id]; }

hipError_t launch_tile_config(int id, const KernelArgs& a, hipStream_t stream)
{
    switch (id) {
    case 0: return launch<128, 128, 64, 2, 2>(a, stream);
    case 1: return launch<256, 128, 64, 2, 2>(a, stream);
    case 2: return launch<128, 64, 64, 2, 2>(a, stream);
    case 3: return launch<64, 64, 64, 2, 2>(a, stream);
    case 4: return launch<128, 256, 64, 2, 2>(a, stream);
    case 5: return launch<256, 64, 64, 4, 1>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace cbw
