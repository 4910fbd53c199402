// A fifth dgrad kernel, for 3x3 stride-1 layers whose dx and dy images have
// the same extent (pad 1, P = H, Q = W) and at most 64 dy channels: the
// whole reduction is one 64-wide k chunk, so everything a tile needs fits in
// LDS at once.
//
// The operation is that of the other kernels (the backward-data convolution
// of "[CUTLASS] Conv2d dgrad", apache/tvm PR #10110, as an implicit GEMM);
// the tap shifts are those of dgrad_halo: output pixel m (linear in n, h, w)
// takes tap (r, t) from dy pixel m + d, d = (1 - r) * W + (1 - t), when the
// shifted row and column stay inside the image, so a tile of BM pixels
// reads only dy pixels [m0 - D, m0 + BM + D), D = W + 1.
//
// Such layers are small (the ResNet-50 stage-2 layer at batch 8: 1.85
// GFLOP, 6.5 MB) and their time is latency: a kernel that streams nine
// slices through a ring waits for a load round trip about every slice. Here
// each workgroup issues all its loads at once (the dy halo, 16-byte rows of
// 144 bytes as in dgrad_halo, and the nine filter taps, 72 KiB for 64
// channels), and runs its 72 matrix-core operations per wave back to back,
// fragments read from LDS one step ahead, waiting only where a group of
// three taps begins for that group's filter to have landed. One tile per
// workgroup, four waves of 64 x 32.
#include "dgrad_internal.h"
#include "kernel_common.h"

namespace cbw {
namespace {

template <int BM, int BN, int WM, int WN>
struct Halo1Shape {
    static constexpr int NW = WM * WN;
    static constexpr int TAPS = 9;
    static constexpr int FSTAGE = 64 * BN * 2;    // one tap of the filter (bytes)
    static constexpr int FILT = TAPS * FSTAGE;
    static constexpr int ROW = 9 * 16;            // bytes per halo row
    static constexpr int RPL = 7 * NW;            // halo rows one load of every wave fills
    static constexpr int HL = 12;                 // halo loads per wave
    static constexpr int HR = HL * RPL;           // halo rows the buffer holds
    static constexpr int HBUF = (HR + 1) * ROW;   // and the row the last load's last lane writes
    static constexpr int Z0 = FILT;               // 512 bytes of zeros
    static constexpr int B0 = Z0 + 512;           // the halo buffer
    static constexpr int LDS_USED = B0 + HBUF;
};

// Halo rows for shift bound D: the tile and D on each side, rounded up to
// whole loads.
__host__ __device__ constexpr int halo1_rows(int BM, int rows_per_load, int D)
{
    return (BM + 2 * D + rows_per_load - 1) / rows_per_load * rows_per_load;
}

template <int BM, int BN, int WM, int WN, bool SPLIT>
__global__ void __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(1, 1)))
dgrad_halo1(KernelArgs a)
{
    using Sh = Halo1Shape<BM, BN, WM, WN>;
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int B_ROW = BN * 2;                 // one k row of a filter tap
    constexpr int FSTAGE = Sh::FSTAGE;
    constexpr int TAPS = Sh::TAPS, ROW = Sh::ROW, RPL = Sh::RPL, HL = Sh::HL;
    constexpr int Z0 = Sh::Z0, B0 = Sh::B0;
    constexpr int FB = FSTAGE / 1024;             // 1 KiB blocks per tap
    constexpr int F_INSTR = Sh::FILT / 1024 / NW; // filter loads per wave
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BN % 64 == 0 && FB % NW == 0, "a tap is whole loads of every wave");
    static_assert(Z0 % 256 == 0, "zeros: a bank window");
    static_assert(Sh::LDS_USED <= 160 * 1024, "LDS budget");
    static_assert(HL + F_INSTR < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char lds[Sh::LDS_USED];
    const uint32_t lds_u32 = (uint32_t)(uintptr_t)((lds_char*)lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int C = pin(a.C);
    const int K = pin(a.K);
    const int P = pin(a.P);
    const int Q = pin(a.Q);
    const int RSC = pin(9 * C);                   // filter elements per k

    // ---- this workgroup's tile and k chunk (one phase; the grid is the tile
    // count, times the chunk count when the chunks are split: workgroup
    // chunk*tiles + tile)
    const int ntile = pin(a.gemm_tiles);
    const int nchunk = SPLIT ? pin(a.sk_maxseg) : 1;
    const int bid = SPLIT ? (int)blockIdx.x % ntile : (int)blockIdx.x;
    const int chunk = SPLIT ? pin((int)blockIdx.x / ntile) : 0;
    const int tile = xcd_remap(bid, ntile, a.group, a.xcd_mode);
    const int kc0 = chunk * 64;                   // the chunk's first dy channel
    const PhaseArg& ph = a.ph[0];
    int tm, tn;
    if (a.order != 1) {    // channel tiles of one pixel block are consecutive
        tm = tile / a.tiles_n;
        tn = tile - tm * a.tiles_n;
    } else {               // pixel blocks of one channel tile are consecutive
        tn = tile / ph.tiles_m;
        tm = tile - tn * ph.tiles_m;
    }
    const int m0 = pin(tm * BM);
    const int c0 = pin(tn * BN);
    const int M = pin(ph.M);
    const int D = pin(Q + 1);                     // buffer row x holds dy pixel m0 - D + x
    const int HB = pin(halo1_rows(BM, RPL, D) / RPL);   // halo loads per wave that carry rows

    const i32x4 dy_desc = raw_descriptor(a.dy, a.dy_bytes);
    const i32x4 w_desc = raw_descriptor(a.w, a.w_bytes);

    // ---- zeros for the taps that leave the image
    if (wave == 0 && lane < 32)
        *(__attribute__((address_space(3))) u32x4*)((lds_char*)lds + Z0 + lane * 16) = u32x4{0u, 0u, 0u, 0u};

    // ---- the halo, as in dgrad_halo: load j of wave v fills block
    // b = j*NW + v, units 63b .. 63b + 63 of the buffer; lane l writes unit
    // 63b + l = row 7b + l/9, unit l%9, from dy pixel m0 - D + 7b + l/9 at k
    // 8*(l%9) (lane 63 writes the first unit of row 7b + 7, which block b + 1
    // writes with the same bytes). Lanes that load nothing (their units read
    // as zeros): the unused unit of each row, units past K, and every lane of
    // a load past the halo. Rows outside the image hold what the range check
    // gives; only taps that leave the image would read them, and those read
    // the zeros instead.
    {
        const int hq = lane / 9;
        const int hr = lane - 9 * hq;
        const uint32_t hoff0 = (uint32_t)(m0 - D + 7 * wave + hq) * (uint32_t)(2 * K) + (uint32_t)(16 * hr);
        const bool skip = hr == 8 || kc0 + 8 * hr >= K;
        const uint32_t vstep = pin((uint32_t)(RPL * 2 * K));
        const uint32_t h_wave = pin(lds_u32 + (uint32_t)(B0 + wave * 63 * 16));
        static_for<0, HL>([&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            const bool off = skip || J >= HB;
            dma16_at<(uint32_t)(J * NW * 63 * 16)>(dy_desc, off ? 0x80000000u : hoff0 + (uint32_t)J * vstep,
                                                   pin((uint32_t)(2 * kc0)), h_wave);
        });
    }

    // ---- the filter: tap T (= 3r + t) in bytes T*FSTAGE.., row k of 64 at
    // k*B_ROW, channel chunk p at position p ^ w_swizzle(k) (as in the other
    // kernels). Load X of wave v fills block X*NW + v, tap X*NW / FB; byte
    // 16*l of the block is row k = 8*((X*NW + v) % FB) + l/8, position l%8:
    // w[k, r, t, c0 + 8*chunk] at element k*9C + T*C + c0 + 8*chunk (the
    // tap and c0 in the scalar offset). Rows past K and channels past C load
    // zeros.
    {
        const uint32_t dma_base = pin(lds_u32 + (uint32_t)(wave * 1024));
        static_for<0, F_INSTR>([&](auto x_c) {
            constexpr int X = decltype(x_c)::value;
            constexpr int T = X * NW / FB;
            const int b = (X * NW + wave) % FB;
            const int k = 8 * b + (lane >> 3);
            const int cc = ((lane & 7) ^ w_swizzle<B_ROW>(k)) * 8;
            const uint32_t vo = (kc0 + k >= K || c0 + cc >= C) ? 0x80000000u : (uint32_t)(k * RSC + cc) * 2u;
            dma16_at<(uint32_t)(X * NW * 1024)>(w_desc, vo, pin((uint32_t)(kc0 * RSC + T * C + c0) * 2u), dma_base);
        });
    }

    // ---- fragment addresses. dy^T (B): tile pixel p = wm*TM + fm*32 +
    // lane%32 at k chunk 2*kk + lane/32 is halo row p + D + d for tap shift
    // d, at byte 144*(p + D + d) + 16*(2*kk + lane/32); where the tap leaves
    // the image, the zero block's byte at the same offset within a 256-byte
    // bank window. Filter^T (A): group g = lane/16 covers channels +16*(g&1),
    // k +8*(g>>1); within it lane 4r+q reads row r, channels 4q..4q+3
    // (transpose reads).
    uint32_t b_off[TAPS][FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int pr = wm * TM + fm * 32 + (lane & 31);
        const int m = m0 + pr;
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const int i = (int)fastdiv(rem, ph.div_w);
        const int jj = (int)(rem - (uint32_t)i * (uint32_t)ph.Wp);
        const uint32_t base = (uint32_t)(B0 + ROW * (pr + D) + 16 * (lane >> 5));
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const bool ok = (m < M) & ((unsigned)(i + 1 - r) < (unsigned)P) & ((unsigned)(jj + 1 - t) < (unsigned)Q);
                const uint32_t ad = base + (uint32_t)(ROW * ((1 - r) * Q + (1 - t)));
                b_off[3 * r + t][fm] = ok ? ad : ((ad & 255u) | (uint32_t)Z0);
            }
    }
    const int g4 = (lane >> 4) & 3;
    const int rr = (lane & 15) >> 2;
    const int qq = lane & 3;
    int a_frag[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int cl = wn * TN + fn * 32 + (g4 & 1) * 16 + 4 * qq;
        const int krow = (g4 >> 1) * 8 + rr;
        a_frag[fn] = krow * B_ROW + (((cl >> 3) ^ w_swizzle<B_ROW>(krow)) * 16) + (cl & 7) * 2;
    }

    // ---- the 36 sub-steps (9 taps x 4) back to back, each on fragments
    // read one sub-step ahead. The loads went out as the halo, then the
    // filter tap after tap (FPG loads per wave for each group of three
    // taps): before a group's first fragments are read, the wave waits for
    // its loads up to that group (the later groups may stay in flight) and
    // meets the other waves, so the first taps' operations run while the
    // rest of the filter lands.
    constexpr int FPG = 3 * FB / NW;
    static_assert(F_INSTR == 3 * FPG, "three groups of three taps");
    auto wait_group = [&](auto g_c) __attribute__((always_inline)) {
        constexpr int G = decltype(g_c)::value;
        wait_vmcnt<(2 - G) * FPG>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
    };
    wait_group(IC<0>{});

    float16_t acc[FN][FM];
    half8_t af[2][FN], bf[2][FM];
    auto read_frags = [&](auto s_c, auto set_c) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        constexpr int SET = decltype(set_c)::value;
        constexpr int T = S / 4, KK = S % 4;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const lds_char* p = (lds_char*)lds + T * FSTAGE + a_frag[fn] + KK * 16 * B_ROW;
            const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)p);
            const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p + 4 * B_ROW));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
            af[SET][fn] = __builtin_bit_cast(half8_t, u32x4{l2.x, l2.y, h2.x, h2.y});
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            bf[SET][fm] = __builtin_bit_cast(half8_t, *(const __attribute__((address_space(3))) u32x4*)(
                                                          (lds_char*)lds + b_off[T][fm] + KK * 32));
    };
    read_frags(IC<0>{}, IC<0>{});
    static_for<0, 4 * TAPS>([&](auto s_c) {
        constexpr int S = decltype(s_c)::value;
        if constexpr (S + 1 < 4 * TAPS) {
            if constexpr ((S + 1) % 12 == 0)
                wait_group(IC<(S + 1) / 12>{});
            read_frags(IC<S + 1>{}, IC<(S + 1) & 1>{});
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                if constexpr (S == 0)
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[0][fn], bf[0][fm], float16_t{}, 0, 0, 0);
                else
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[S & 1][fn], bf[S & 1][fm], acc[fn][fm], 0, 0, 0);
            }
    });

    // ---- split chunks: the partial sums of the tile's chunks meet. As the
    // stream-K fix-up of dgrad_igemm: workgroup (tile, chunk) leaves its fp32
    // sums in workspace slot [tile][chunk] (16-byte group q of thread tid at
    // float offset (q*NT + tid)*4) and arrives on the tile's counter; the
    // last to arrive (no workgroup waits for another) adds the chunks in
    // chunk order, its own from registers, resets the counter and runs the
    // epilogue; the others end here. A workgroup that finds every other
    // chunk arrived is the last without writing its own sums. Every
    // workspace access is system-scope (sc0 sc1), so no L2 writeback or
    // invalidate is needed across the XCDs' caches: a workgroup's sums have
    // reached memory once its vmcnt drains, which precedes its arrival.
    if constexpr (SPLIT) {
        constexpr int NT = 64 * NW;
        constexpr int NQ = FN * FM * 4;           // 16-byte groups of accumulators per thread
        constexpr uint32_t kSegBytes = (uint32_t)BM * BN * 4;
        constexpr int kSys = 17;                  // cache policy sc0 sc1
        int* const count = a.sk_count + tile;
        const __amdgpu_buffer_rsrc_t ws =
            make_rsrc(a.sk_part + (size_t)tile * (size_t)nchunk * (size_t)(BM * BN), (uint32_t)nchunk * kSegBytes);
        const uint32_t lane_off = (uint32_t)tid * 16u;
        __attribute__((address_space(3))) int* flag = (__attribute__((address_space(3))) int*)((lds_char*)lds + Z0);
        __syncthreads();                          // every wave is done reading the zeros
        if (tid == 0)
            *flag = __hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nchunk - 1 ? 1 : 0;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(*flag) == 0) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int g = (fn * FM + fm) * 4 + q;
                        const float4_t v{acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2], acc[fn][fm][4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ws,
                                                               (uint32_t)chunk * kSegBytes + (uint32_t)(g * NT) * 16u + lane_off, 0, kSys);
                    }
            wait_vmcnt<0>();                      // this wave's sums are in memory
            __syncthreads();                      // ... and every wave's; every wave has read the flag
            if (tid == 0) {
                const int old = __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                *flag = old == nchunk - 1 ? 1 : 0;
            }
            __syncthreads();
            if (__builtin_amdgcn_readfirstlane(*flag) == 0)
                return;
        }
        // chunk by chunk, all NQ groups of a chunk in flight at once
        float4_t sum[NQ];
#pragma unroll
        for (int g = 0; g < NQ; ++g)
            sum[g] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int sg = 0; sg < nchunk; ++sg) {
            float4_t v[NQ];
            if (sg == chunk) {
#pragma unroll
                for (int g = 0; g < NQ; ++g) {
                    const int fn = g / (FM * 4), fm = (g / 4) % FM, q = g % 4;
                    v[g] = float4_t{acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2], acc[fn][fm][4 * q + 3]};
                }
            } else {
#pragma unroll
                for (int g = 0; g < NQ; ++g)
                    v[g] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                            ws, (uint32_t)sg * kSegBytes + (uint32_t)(g * NT) * 16u + lane_off, 0, kSys));
            }
#pragma unroll
            for (int g = 0; g < NQ; ++g)
                sum[g] += v[g];
        }
#pragma unroll
        for (int g = 0; g < NQ; ++g) {
            const int fn = g / (FM * 4), fm = (g / 4) % FM, q = g % 4;
            acc[fn][fm][4 * q] = sum[g][0];
            acc[fn][fm][4 * q + 1] = sum[g][1];
            acc[fn][fm][4 * q + 2] = sum[g][2];
            acc[fn][fm][4 * q + 3] = sum[g][3];
        }
        if (tid == 0)
            __hip_atomic_store(count, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: fp32 -> fp16 (RNE), staged through the first filter tap
    // (every wave is done reading the filter after the barrier) and stored
    // as whole pixel rows. With P = H and stride 1, dx pixel m is lattice row
    // m, at element m*C.
    constexpr int CH = TN / 8;            // 16-byte chunks per staged pixel row
    constexpr int EROW = TN * 2;          // bytes per staged pixel row
    constexpr int EBLK = 32 * EROW;       // bytes per wave per pixel group
    constexpr int PPI = 64 / CH;          // pixels per store instruction
    constexpr int EST = 32 / PPI;         // store instructions per pixel group
    static_assert(CH >= 2 && CH <= 64 && 64 % CH == 0, "whole pixel rows per store");
    static_assert(NW * EBLK <= FSTAGE, "the staging blocks fit in one tap");
    __syncthreads();
    const __amdgpu_buffer_rsrc_t e_dx = make_rsrc(a.dx, a.dx_bytes);
    lds_char* blk = (lds_char*)lds + wave * EBLK;
    const int cw = c0 + wn * TN;
    const int pw = lane & 31;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const half4_t o{(_Float16)acc[fn][fm][4 * gq + 0], (_Float16)acc[fn][fm][4 * gq + 1],
                                (_Float16)acc[fn][fm][4 * gq + 2], (_Float16)acc[fn][fm][4 * gq + 3]};
                const int q = fn * 4 + gq;
                *(__attribute__((address_space(3))) u32x2*)(blk + pw * EROW + ((q ^ ((pw >> 1) % CH)) * 16) + (lane >> 5) * 8) =
                    __builtin_bit_cast(u32x2, o);
            }
#pragma unroll
        for (int e = 0; e < EST; ++e) {
            const int pr = e * PPI + lane / CH;
            const int q = lane % CH;
            const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(blk + pr * EROW + ((q ^ ((pr >> 1) % CH)) * 16));
            const int m = m0 + wm * TM + fm * 32 + pr;
            const int c = cw + q * 8;
            const uint32_t bad = (uint32_t)(m >= M) | (uint32_t)(c >= C);
            __builtin_amdgcn_raw_buffer_store_b128(v, e_dx, out_of_range_if(bad, ((uint32_t)m * (uint32_t)C + (uint32_t)c) * 2u),
                                                   0, kStoreNT);
        }
    }
}

// The layers this kernel runs: 3x3, stride 1, pad 1, P = H and Q = W, no
// fused epilogue factor, a halo of at most the rows the buffer holds, and at
// most 64 dy channels, or up to kHalo1MaxChunks chunks of 64 when the chunks
// are split over workgroups (which needs a workspace; the host runs such a
// layer on the plain kernel of the same tile without one).
template <int BM, int BN, int WM, int WN>
bool halo1_fits(int R, int S, int stride, int pad, int H, int W, int P, int Q, int K, int epi)
{
    using Sh = Halo1Shape<BM, BN, WM, WN>;
    if (stride != 1 || R != 3 || S != 3 || pad != 1 || P != H || Q != W || K < 1 || K > 64 * kHalo1MaxChunks ||
        epi != kEpiNone || Q > Sh::HR)
        return false;
    return halo1_rows(BM, Sh::RPL, Q + 1) <= Sh::HR;
}

// Whether the planned launch is one this kernel runs: that one phase (taps
// from (0, 0), dy offsets of the first tap = 1) in GEMM tiles only, one per
// workgroup, either whole (K <= 64) or split into its k chunks (one
// workgroup per tile and chunk, partial sums in the workspace).
template <int BM, int BN, int WM, int WN>
bool halo1_runs(const KernelArgs& a)
{
    const PhaseArg& ph = a.ph[0];
    if (a.nzphases > 0 || a.ncomp > 0 || a.zstripes > 0 || a.nphases != 1 || a.total_tiles != a.gemm_tiles ||
        ph.nr != 3 || ph.nt != 3 || ph.r0 != 0 || ph.t0 != 0 || ph.dr0 != 1 || ph.dt0 != 1 || ph.ph != 0 || ph.pw != 0 ||
        ph.Wp != a.W || ph.div_hw.d != (uint32_t)(a.H * a.W) ||
        !halo1_fits<BM, BN, WM, WN>(a.R, a.S, a.stride, 1, a.H, a.W, a.P, a.Q, a.K, a.epi))
        return false;
    const int chunks = (a.K + 63) / 64;
    if (!a.sk)
        return chunks == 1 && a.grid == a.gemm_tiles;
    return chunks > 1 && a.sk_maxseg == chunks && (int64_t)a.grid == (int64_t)a.gemm_tiles * chunks &&
           a.sk_part != nullptr && a.sk_count != nullptr;
}

template <int BM, int BN, int WM, int WN>
hipError_t halo1_launch(const KernelArgs& a, hipStream_t stream)
{
    if (!halo1_runs<BM, BN, WM, WN>(a))
        return hipErrorInvalidValue;
    if (a.sk)
        hipLaunchKernelGGL((dgrad_halo1<BM, BN, WM, WN, true>), dim3(a.grid), dim3(64 * WM * WN), 0, stream, a);
    else
        hipLaunchKernelGGL((dgrad_halo1<BM, BN, WM, WN, false>), dim3(a.grid), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
int halo1_resident(void)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(dgrad_halo1<BM, BN, WM, WN, false>),
                                                     64 * WM * WN, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    return n > 0 ? n : 1;
}

template <int BM, int BN, int WM, int WN>
int halo1_private(void)
{
    int most = 0;
    for (const void* f : {reinterpret_cast<const void*>(dgrad_halo1<BM, BN, WM, WN, false>),
                          reinterpret_cast<const void*>(dgrad_halo1<BM, BN, WM, WN, true>)}) {
        hipFuncAttributes attr;
        if (hipFuncGetAttributes(&attr, f) != hipSuccess) {
            (void)hipGetLastError();
            return -1;
        }
        most = (int)attr.localSizeBytes > most ? (int)attr.localSizeBytes : most;
    }
    return most;
}

// The compiled configurations of this kernel: (BM, BN, WM, WN).
#define CBW_HALO1_CONFIGS(X) \
    X(128, 64, 2, 2)

#define CBW_HALO1_ENTRY(BM, BN, WM, WN) \
    {BM, BN, 64, WM, WN, #BM "x" #BN "x64/" #WM "x" #WN "s", Halo1Shape<BM, BN, WM, WN>::LDS_USED, true, false, true, true, true},
const TileConfig kHalo1Configs[] = {CBW_HALO1_CONFIGS(CBW_HALO1_ENTRY)};
constexpr int kNumHalo1 = sizeof(kHalo1Configs) / sizeof(kHalo1Configs[0]);

using Halo1LaunchFn = hipError_t (*)(const KernelArgs&, hipStream_t);
using Halo1RunsFn = bool (*)(const KernelArgs&);
using Halo1FitsFn = bool (*)(int, int, int, int, int, int, int, int, int, int);
#define CBW_HALO1_LAUNCH(BM, BN, WM, WN) &halo1_launch<BM, BN, WM, WN>,
#define CBW_HALO1_FITS(BM, BN, WM, WN) &halo1_fits<BM, BN, WM, WN>,
#define CBW_HALO1_RUNS(BM, BN, WM, WN) &halo1_runs<BM, BN, WM, WN>,
#define CBW_HALO1_RESIDENT(BM, BN, WM, WN) &halo1_resident<BM, BN, WM, WN>,
#define CBW_HALO1_PRIVATE(BM, BN, WM, WN) &halo1_private<BM, BN, WM, WN>,
const Halo1LaunchFn kHalo1Launch[] = {CBW_HALO1_CONFIGS(CBW_HALO1_LAUNCH)};
const Halo1FitsFn kHalo1Fits[] = {CBW_HALO1_CONFIGS(CBW_HALO1_FITS)};
const Halo1RunsFn kHalo1Runs[] = {CBW_HALO1_CONFIGS(CBW_HALO1_RUNS)};
int (*const kHalo1Resident[])(void) = {CBW_HALO1_CONFIGS(CBW_HALO1_RESIDENT)};
int (*const kHalo1Private[])(void) = {CBW_HALO1_CONFIGS(CBW_HALO1_PRIVATE)};

}  // namespace

int halo1_num_configs() { return kNumHalo1; }

const TileConfig& halo1_config(int i) { return kHalo1Configs[i]; }

bool halo1_admits(int i, int R, int S, int stride, int pad, int H, int W, int P, int Q, int K, int epi)
{
    return i >= 0 && i < kNumHalo1 && kHalo1Fits[i](R, S, stride, pad, H, W, P, Q, K, epi);
}

bool halo1_runs_launch(int i, const KernelArgs& a) { return i >= 0 && i < kNumHalo1 && kHalo1Runs[i](a); }

hipError_t launch_halo1(int i, const KernelArgs& a, hipStream_t stream)
{
    if (i < 0 || i >= kNumHalo1)
        return hipErrorInvalidValue;
    return kHalo1Launch[i](a, stream);
}

int halo1_blocks_per_cu(int i) { return (i >= 0 && i < kNumHalo1) ? kHalo1Resident[i]() : 1; }

int halo1_private_bytes(int i) { return (i >= 0 && i < kNumHalo1) ? kHalo1Private[i]() : -1; }

}  // namespace cbw
