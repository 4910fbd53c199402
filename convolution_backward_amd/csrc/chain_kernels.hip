// Two dgrad steps of a bottleneck in one kernel: persistent kernel fusion in
// the sense of the Bolt paper notes (KuangjuX/Paper-reading #28, "Persistent
// kernel (GEMM/Conv) fusion"): the first convolution's output tile never
// leaves the workgroup that made it, and the second convolution reads it from
// LDS instead of HBM.
//
// The chain (NHWC fp16, fp32 accumulation):
//   t[m, c]   = fp16( g(z[m, c]) * sum over taps (r, s) and k of
//                     dy[n, h + pad - r, w + pad - s, k] * w1[k, r, s, c] )
//   dx[m, ci] = fp16( sum over c of t[m, c] * w2[c, ci] )
// for dx pixel m = (n, h, w): the stride-1 dgrad of an RxS convolution with
// Cm input channels, its activation derivative g(z) (relu' or hardswish' of
// the saved pre-activation z), then the dgrad of the 1x1 convolution in front
// of it (C -> Cm, filter w2 = [Cm][1][1][C]). t is rounded to fp16 once, as
// the two separate kernels would store it.
//
// Threadblock residence (the notes' key property: the first GEMM's tile
// spans all of its output channels, ThreadBlock_N = GEMM_N): a workgroup owns
// 128 dx pixels and all Cm (<= 128) intermediate channels, so the second GEMM
// (pixels x C, reduction over Cm) finds its whole input in the workgroup.
// The intermediate tile is held in LDS between the two GEMMs (the notes'
// shared-memory-resident variant: both GEMMs spread their output over eight
// waves, so each wave needs fragments another wave produced).
//
// MI355X mapping:
//   * 512 threads = 8 waves as 2 (channels) x 4 (pixel groups of 32), for
//     both GEMMs; v_mfma_f32_32x32x16_f16 with A = filter^T (rows channels,
//     read with ds_read_b64_tr_b16 from filter rows in LDS) and B = the pixel
//     rows (dy, later t) read with 16-byte LDS reads.
//   * Slices of 64 reduction elements, double-buffered in LDS through
//     registers: the next slice's 16-byte buffer loads are in flight while the
//     current slice is on the matrix cores; one barrier per slice.
//   * Stage 1 walks taps x ceil(K/64) slices; stage 2 walks ceil(C/128)
//     output-channel chunks x Cm/64 slices, each chunk finished by an
//     LDS-staged epilogue that stores whole 128-byte pieces of dx rows.
//   * Tiles go to XCDs in contiguous eighths, so neighbouring pixel tiles
//     (which share dy halo rows) share an L2.
// Out-of-range accesses (padding taps, dead pixels past N*H*W, ragged K, Cm
// or C) use the buffer range check: loads read zeros and stores are dropped.
#include "dgrad_internal.h"
#include "kernel_common.h"

namespace cbw {
namespace {

constexpr int kBM = 128;       // dx pixels per workgroup
constexpr int kThreads = 512;  // 8 waves
constexpr int kBN2 = 128;      // input channels per stage-2 chunk

template <int CM>
struct ChainLayout {
    static constexpr int DY_BYTES = kBM * 128;            // 128 pixel rows x 64 k
    static constexpr int W1_ROW = 2 * CM;                  // filter row: CM channels
    static constexpr int W1_BYTES = 64 * W1_ROW;
    static constexpr int STAGE1 = DY_BYTES + W1_BYTES;
    static constexpr int W2_ROW = 2 * kBN2;                // 256 bytes
    static constexpr int W2_BYTES = 64 * W2_ROW;
    static constexpr int STAGING = 8 * 32 * 128;           // per wave 32 pixels x 64 channels
    static constexpr int RING = (2 * STAGE1 > 2 * W2_BYTES + STAGING) ? 2 * STAGE1 : 2 * W2_BYTES + STAGING;
    static constexpr int T_ROW = 2 * CM;
    static constexpr int T_OFF = RING;
    static constexpr int TOTAL = RING + kBM * T_ROW;
};

// NS1 > 0: stage 1 has exactly NS1 slices (taps x k steps), known at compile
// time, and runs fully unrolled with a deeper prefetch; 0: any count.
template <int CM, int E, int NS1>
__global__ __launch_bounds__(kThreads) void chain_igemm(ChainArgs a)
{
    using L = ChainLayout<CM>;
    constexpr int FN1 = CM / 64;        // 32-channel blocks per wave in stage 1 (each wave: CM/2 channels)
    constexpr int W1_LD = CM / 64;      // 16-byte filter chunks per thread per stage-1 slice
    constexpr int KS2 = CM / 64;        // stage-2 slices per output-channel chunk
    __shared__ __attribute__((aligned(1024))) char lds[L::TOTAL];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1;            // channel half
    const int wm = wave >> 1;           // pixel group of 32
    const int tile = xcd_remap(blockIdx.x, a.tiles, 1, 1);   // each XCD a contiguous eighth of the tiles
    const int m0 = tile * kBM;

    const __amdgpu_buffer_rsrc_t dy_r = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t w1_r = make_rsrc(a.w1, a.w1_bytes);
    const __amdgpu_buffer_rsrc_t w2_r = make_rsrc(a.w2, a.w2_bytes);
    const __amdgpu_buffer_rsrc_t dx_r = make_rsrc(a.dx, a.dx_bytes);

    // ---- stage-1 loader: dy chunks tid + 512*j, j < 2 (row tid/8 + 64*j, chunk tid%8)
    const int ld_chunk = tid & 7;
    int ld_hp[2], ld_wp[2];             // h + pad, w + pad of the row's pixel (-2^24: dead row)
    uint32_t ld_base[2];                // element offset of dy[n, h+pad, w+pad, 8*chunk] (mod 2^32)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = m0 + (tid >> 3) + 64 * j;
        const uint32_t n = fastdiv((uint32_t)m, a.div_hw);
        const uint32_t rem = (uint32_t)m - n * a.div_hw.d;
        const uint32_t h = fastdiv(rem, a.div_w);
        const uint32_t w = rem - h * (uint32_t)a.W;
        const bool live = m < a.M;
        ld_hp[j] = live ? (int)h + a.pad : -(1 << 24);
        ld_wp[j] = (int)w + a.pad;
        ld_base[j] = ((n * (uint32_t)a.P + h + (uint32_t)a.pad) * (uint32_t)a.Q + w + (uint32_t)a.pad) * (uint32_t)a.K +
                     (uint32_t)(ld_chunk * 8);
    }
    // Register sets of prefetched stage-1 slices: slice j is loaded into set
    // j % DEPTH. With a known slice count the walk is unrolled, so the
    // compiler tracks each set's loads exactly and waits only for the slice
    // it stores next, DEPTH - 1 slices of loads staying in flight.
    constexpr int DEPTH = NS1 > 0 ? 3 : 1;
    u32x4 rdy[DEPTH][2], rw1[DEPTH][W1_LD];
    auto load1 = [&](u32x4 (&ldy)[2], u32x4 (&lw1)[W1_LD], int r, int s, int k0) {
        const uint32_t tapoff = ((uint32_t)r * (uint32_t)a.Q + (uint32_t)s) * (uint32_t)a.K;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int p = ld_hp[j] - r, q = ld_wp[j] - s;
            const uint32_t bad = (uint32_t)!(((unsigned)p < (unsigned)a.P) & ((unsigned)q < (unsigned)a.Q) &
                                             (k0 + ld_chunk * 8 < a.K));
            ldy[j] = __builtin_amdgcn_raw_buffer_load_b128(dy_r, out_of_range_if(bad, (ld_base[j] - tapoff + (uint32_t)k0) * 2u), 0, 0);
        }
#pragma unroll
        for (int j = 0; j < W1_LD; ++j) {
            const int i = tid + kThreads * j;
            const int krow = i / (CM / 8), cc = i % (CM / 8);
            const int k = k0 + krow, c = cc * 8;
            const uint32_t bad = (uint32_t)((k >= a.K) | (c >= a.Cm));
            const uint32_t off = ((((uint32_t)k * (uint32_t)a.R + (uint32_t)r) * (uint32_t)a.S + (uint32_t)s) * (uint32_t)a.Cm + (uint32_t)c) * 2u;
            lw1[j] = __builtin_amdgcn_raw_buffer_load_b128(w1_r, out_of_range_if(bad, off), 0, 0);
        }
    };
    auto store1 = [&](const u32x4 (&ldy)[2], const u32x4 (&lw1)[W1_LD], int buf) {
        char* st = lds + buf * L::STAGE1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = (tid >> 3) + 64 * j;
            *(u32x4*)(st + row * 128 + ((ld_chunk ^ dy_swizzle(row)) * 16)) = ldy[j];
        }
#pragma unroll
        for (int j = 0; j < W1_LD; ++j) {
            const int i = tid + kThreads * j;
            const int krow = i / (CM / 8), cc = i % (CM / 8);
            *(u32x4*)(st + L::DY_BYTES + krow * L::W1_ROW + ((cc ^ w_swizzle<L::W1_ROW>(krow)) * 16)) = lw1[j];
        }
    };

    // ---- fragment addresses. Filter^T operand (A): lane group g = lane/16
    // covers channels +16*(g&1) and k +8*(g>>1); in it lane 4*rr+qq reads
    // row rr, channels 4*qq..4*qq+3 (two transpose reads, rows +0 and +4).
    const int g = (lane >> 4) & 3;
    const int rr = (lane & 15) >> 2;
    const int qq = lane & 3;
    const int krow_a = (g >> 1) * 8 + rr;
    // Pixel-row operand (B): row wm*32 + lane%32, k chunk 2*kk + lane/32.
    const int prow = wm * 32 + (lane & 31);
    const int psw = dy_swizzle(prow);

    auto tr_pair = [&](const char* p, int row_bytes) -> half8_t {
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(lds_char*)p);
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(lds_char*)(p + 4 * row_bytes));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(half8_t, u32x4{l2.x, l2.y, h2.x, h2.y});
    };

    // ================= stage 1: D1[c][m] over taps x k
    int a1_off[FN1];
#pragma unroll
    for (int fn = 0; fn < FN1; ++fn) {
        const int cl = wn * (CM / 2) + fn * 32 + (g & 1) * 16 + 4 * qq;
        a1_off[fn] = L::DY_BYTES + krow_a * L::W1_ROW + (((cl >> 3) ^ w_swizzle<L::W1_ROW>(krow_a)) * 16) + (cl & 7) * 2;
    }
    float16_t acc1[FN1];
#pragma unroll
    for (int fn = 0; fn < FN1; ++fn)
        acc1[fn] = float16_t{};
    auto compute1 = [&](int buf) {
        const char* st = lds + buf * L::STAGE1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const half8_t bf = *(const half8_t*)(st + prow * 128 + (((kk * 2 + (lane >> 5)) ^ psw) * 16));
#pragma unroll
            for (int fn = 0; fn < FN1; ++fn) {
                const half8_t af = tr_pair(st + a1_off[fn] + kk * 16 * L::W1_ROW, L::W1_ROW);
                acc1[fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf, acc1[fn], 0, 0, 0);
            }
        }
    };

    // ================= stage-2 loader (w2 slices of 64 rows x 128 channels)
    u32x4 rw2[2];
    auto load2 = [&](int u) {
        const int ch = u / KS2, ks = u - (u / KS2) * KS2;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int i = tid + kThreads * j;
            const int row = i >> 4, cc = i & 15;
            const int cm = ks * 64 + row, ci = ch * kBN2 + cc * 8;
            const uint32_t bad = (uint32_t)((cm >= a.Cm) | (ci >= a.C));
            rw2[j] = __builtin_amdgcn_raw_buffer_load_b128(w2_r, out_of_range_if(bad, ((uint32_t)cm * (uint32_t)a.C + (uint32_t)ci) * 2u), 0, 0);
        }
    };
    auto store2 = [&](int buf) {
        char* st = lds + buf * L::W2_BYTES;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int i = tid + kThreads * j;
            const int row = i >> 4, cc = i & 15;
            *(u32x4*)(st + row * L::W2_ROW + ((cc ^ w_swizzle<L::W2_ROW>(row)) * 16)) = rw2[j];
        }
    };
    const int nch = (a.C + kBN2 - 1) / kBN2;
    const int ns2 = nch * KS2;
    // The tile's z values (epilogue 1): fp16 in the accumulator layout.
    u32x2 zr[FN1][4];
    auto load_z = [&]() {
        if constexpr (E != 0) {
            const __amdgpu_buffer_rsrc_t z_r = make_rsrc(a.z, a.z_bytes);
            const int m = m0 + prow;
#pragma unroll
            for (int fn = 0; fn < FN1; ++fn)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int c = wn * (CM / 2) + fn * 32 + 8 * gq + 4 * (lane >> 5);
                    const uint32_t bad = (uint32_t)((m >= a.M) | (c >= a.Cm));
                    zr[fn][gq] = __builtin_amdgcn_raw_buffer_load_b64(z_r, out_of_range_if(bad, ((uint32_t)m * (uint32_t)a.Cm + (uint32_t)c) * 2u), 0, 0);
                }
        }
    };

    const int ksteps = (a.K + 63) / 64;
    const int ns1 = a.R * a.S * ksteps;
    {
        int r = 0, s = 0, k0 = 0;       // cursor of the slice being loaded
        auto advance = [&]() {
            k0 += 64;
            if (k0 >= a.K) {
                k0 = 0;
                if (++s == a.S) {
                    s = 0;
                    ++r;
                }
            }
        };
        if constexpr (NS1 > 0) {
#pragma unroll
            for (int j = 0; j < DEPTH && j < NS1; ++j) {
                load1(rdy[j], rw1[j], r, s, k0);
                advance();
            }
            store1(rdy[0], rw1[0], 0);
            __syncthreads();
            // slice it: refill set it % DEPTH (its slice is in LDS) with slice
            // it + DEPTH, compute slice it, store slice it + 1 into the other buffer
#pragma unroll
            for (int it = 0; it < NS1; ++it) {
                if (it + DEPTH < NS1) {
                    load1(rdy[it % DEPTH], rw1[it % DEPTH], r, s, k0);
                    advance();
                }
                if (it == (NS1 > DEPTH ? NS1 - DEPTH : 0)) {
                    // the last slice is requested: z and the first w2 slice
                    // take the registers its sets free
                    load_z();
                    load2(0);
                }
                compute1(it & 1);
                if (it + 1 < NS1)
                    store1(rdy[(it + 1) % DEPTH], rw1[(it + 1) % DEPTH], (it + 1) & 1);
                __syncthreads();
            }
        } else {
            load1(rdy[0], rw1[0], r, s, k0);
            advance();
            store1(rdy[0], rw1[0], 0);
            __syncthreads();
            for (int it = 0; it < ns1; ++it) {
                const bool more = it + 1 < ns1;
                if (more) {
                    load1(rdy[0], rw1[0], r, s, k0);
                    advance();
                }
                compute1(it & 1);
                if (more)
                    store1(rdy[0], rw1[0], (it + 1) & 1);
                __syncthreads();
            }
            load2(0);
        }
    }


    // ================= epilogue 1: t = fp16(D1 * g(z)) into the resident tile
    {
        const int px = prow;             // this lane's pixel within the tile
        half4_t tv[FN1][4];
        if constexpr (E != 0) {
            if constexpr (NS1 == 0)
                load_z();
#pragma unroll
            for (int fn = 0; fn < FN1; ++fn)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const half4_t zh = __builtin_bit_cast(half4_t, zr[fn][gq]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        tv[fn][gq][i] = (_Float16)(acc1[fn][4 * gq + i] * epilogue_factor<E>((float)zh[i]));
                }
        } else {
#pragma unroll
            for (int fn = 0; fn < FN1; ++fn)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        tv[fn][gq][i] = (_Float16)acc1[fn][4 * gq + i];
        }
#pragma unroll
        for (int fn = 0; fn < FN1; ++fn)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int c = wn * (CM / 2) + fn * 32 + 8 * gq + 4 * (lane >> 5);
                *(half4_t*)(lds + L::T_OFF + px * L::T_ROW + (((c >> 3) ^ dy_swizzle(px)) * 16) + (c & 7) * 2) = tv[fn][gq];
            }
    }
    store2(0);
    __syncthreads();

    // ================= stage 2: D2[ci][m] per 128-channel chunk, reduction over Cm
    int a2_off[2];
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
        const int cl = wn * 64 + fn * 32 + (g & 1) * 16 + 4 * qq;
        a2_off[fn] = krow_a * L::W2_ROW + (((cl >> 3) ^ w_swizzle<L::W2_ROW>(krow_a)) * 16) + (cl & 7) * 2;
    }
    float16_t acc2[2];
    acc2[0] = float16_t{};
    acc2[1] = float16_t{};
    auto compute2 = [&](int buf, int ks) {
        const char* st = lds + buf * L::W2_BYTES;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int chunk = ks * 8 + kk * 2 + (lane >> 5);
            const half8_t bf = *(const half8_t*)(lds + L::T_OFF + prow * L::T_ROW + ((chunk ^ psw) * 16));
#pragma unroll
            for (int fn = 0; fn < 2; ++fn) {
                const half8_t af = tr_pair(st + a2_off[fn] + kk * 16 * L::W2_ROW, L::W2_ROW);
                acc2[fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf, acc2[fn], 0, 0, 0);
            }
        }
    };
    // Epilogue 2 of chunk ch: the wave's 64 channels x 32 pixels go through its
    // own LDS block (rows of 128 bytes, chunk c of pixel row p at c ^ (p & 7))
    // and leave as 16-byte stores, eight lanes per 128-byte piece of a dx row.
    char* stg = lds + 2 * L::W2_BYTES + wave * (32 * 128);
    auto epilogue2 = [&](int ch) {
        const int pl = lane & 31;
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int cl = fn * 32 + 8 * gq + 4 * (lane >> 5);
                half4_t hv;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    hv[i] = (_Float16)acc2[fn][4 * gq + i];
                *(half4_t*)(stg + pl * 128 + (((cl >> 3) ^ (pl & 7)) * 16) + (cl & 7) * 2) = hv;
            }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = lane + 64 * u;
            const int row = idx >> 3, cc = idx & 7;
            const u32x4 v = *(const u32x4*)(stg + row * 128 + ((cc ^ (row & 7)) * 16));
            const int m = m0 + wm * 32 + row;
            const int ci = ch * kBN2 + wn * 64 + cc * 8;
            const uint32_t bad = (uint32_t)((m >= a.M) | (ci >= a.C));
            __builtin_amdgcn_raw_buffer_store_b128(v, dx_r, out_of_range_if(bad, ((uint32_t)m * (uint32_t)a.C + (uint32_t)ci) * 2u), 0, kStoreNT);
        }
    };
    for (int u = 0; u < ns2; ++u) {
        const bool more = u + 1 < ns2;
        if (more)
            load2(u + 1);
        const int ks = u - (u / KS2) * KS2;
        compute2(u & 1, ks);
        if (ks == KS2 - 1) {
            epilogue2(u / KS2);
            acc2[0] = float16_t{};
            acc2[1] = float16_t{};
        }
        if (more)
            store2((u + 1) & 1);
        __syncthreads();
    }
}

template <int CM, int E, int NS1>
hipError_t chain_launch_t(const ChainArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((chain_igemm<CM, E, NS1>), dim3(a.tiles), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int CM, int E, int NS1>
int chain_private_t()
{
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(chain_igemm<CM, E, NS1>)) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return (int)attr.localSizeBytes;
}

// Stage-1 slice counts with an unrolled kernel: 3x3 taps at K <= 64 (nine
// slices) and at 64 < K <= 128 (eighteen).
constexpr int kChainUnrolled[2] = {9, 18};

using ChainLaunchFn = hipError_t (*)(const ChainArgs&, hipStream_t);
// [variant: any count, 9 slices, 18 slices][CM == 128][epilogue]
const ChainLaunchFn kChainLaunch[3][2][3] = {
    {{&chain_launch_t<64, 0, 0>, &chain_launch_t<64, 1, 0>, &chain_launch_t<64, 2, 0>},
     {&chain_launch_t<128, 0, 0>, &chain_launch_t<128, 1, 0>, &chain_launch_t<128, 2, 0>}},
    {{&chain_launch_t<64, 0, 9>, &chain_launch_t<64, 1, 9>, &chain_launch_t<64, 2, 9>},
     {&chain_launch_t<128, 0, 9>, &chain_launch_t<128, 1, 9>, &chain_launch_t<128, 2, 9>}},
    {{&chain_launch_t<64, 0, 18>, &chain_launch_t<64, 1, 18>, &chain_launch_t<64, 2, 18>},
     {&chain_launch_t<128, 0, 18>, &chain_launch_t<128, 1, 18>, &chain_launch_t<128, 2, 18>}},
};
int (*const kChainPrivate[3][2][3])() = {
    {{&chain_private_t<64, 0, 0>, &chain_private_t<64, 1, 0>, &chain_private_t<64, 2, 0>},
     {&chain_private_t<128, 0, 0>, &chain_private_t<128, 1, 0>, &chain_private_t<128, 2, 0>}},
    {{&chain_private_t<64, 0, 9>, &chain_private_t<64, 1, 9>, &chain_private_t<64, 2, 9>},
     {&chain_private_t<128, 0, 9>, &chain_private_t<128, 1, 9>, &chain_private_t<128, 2, 9>}},
    {{&chain_private_t<64, 0, 18>, &chain_private_t<64, 1, 18>, &chain_private_t<64, 2, 18>},
     {&chain_private_t<128, 0, 18>, &chain_private_t<128, 1, 18>, &chain_private_t<128, 2, 18>}},
};

// The kernel variant for a problem: 1 + the index of its unrolled slice
// count, or 0 (any count).
inline int chain_variant(const ChainArgs& a)
{
    const int ns1 = a.R * a.S * ((a.K + 63) / 64);
    for (int v = 0; v < 2; ++v)
        if (ns1 == kChainUnrolled[v])
            return v + 1;
    return 0;
}

}  // namespace

hipError_t launch_chain(const ChainArgs& a, hipStream_t stream)
{
    if (a.Cm < 1 || a.Cm > 128 || a.epi < 0 || a.epi > 2)
        return hipErrorInvalidValue;
    return kChainLaunch[chain_variant(a)][a.Cm > 64][a.epi](a, stream);
}

int chain_private_bytes(int Cm, int epi)
{
    if (Cm < 1 || Cm > 128 || epi < 0 || epi > 2)
        return -1;
    int most = 0;
    for (int v = 0; v < 3; ++v) {
        const int b = kChainPrivate[v][Cm > 64][epi]();
        if (b < 0)
            return -1;
        most = b > most ? b : most;
    }
    return most;
}

int chain_lds_bytes(int Cm)
{
    return Cm <= 64 ? ChainLayout<64>::TOTAL : ChainLayout<128>::TOTAL;
}

}  // namespace cbw
