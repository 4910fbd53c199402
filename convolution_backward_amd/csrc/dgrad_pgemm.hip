// A fourth dgrad kernel, for 1x1 stride-1 layers without padding: there the
// backward-data convolution of "[CUTLASS] Conv2d dgrad" (apache/tvm PR
// #10110) is one plain GEMM, dx[m, c] = sum over k of dy[m, k] * w[k, c],
// with m the linear pixel index of both images (P = H, Q = W).
//
// Such layers have short reductions (K / 64 slices per tile) and many tiles,
// so what happens between tiles decides the time. This kernel is persistent
// with four waves of 128 x 64 (as in dgrad_wide, one wave per SIMD): each
// workgroup walks tiles slot, slot + G, slot + 2G, ... (G workgroups, one
// per CU), and the direct-to-LDS loads of its 3-stage ring run two slices
// ahead across tile boundaries, so the first slices of the next tile are in
// LDS when a tile ends. Since dx and dy share the pixel index, a lane's
// load and store offsets are linear in the row: no index division.
//
// A tile's epilogue (fp32 -> fp16, staged through a block of the wave's own
// past the ring, stored as whole pixel rows) runs right after its last
// slice; the next tile's first slice lets those stores stay in flight, its
// second waits for them. (Draining the epilogue one group per slice under
// the next tile's operations instead, with two accumulator sets, was faster
// with dx in cache but not when dx streams to HBM: every slice then waits
// for stores issued about a slice and a half earlier.)
#include "dgrad_internal.h"
#include "kernel_common.h"

namespace cbw {
namespace {

template <int BM, int BN, int WM, int WN>
struct PgemmShape {
    static constexpr int NW = WM * WN;
    static constexpr int BK = 64;
    static constexpr int A_BYTES = BM * 2 * BK;
    static constexpr int B_BYTES = BK * BN * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int STG0 = 3 * STAGE;                  // the staging blocks
    static constexpr int EBLK = 32 * (BN / WN) * 2;         // one wave's block
    static constexpr int LDS_USED = STG0 + NW * EBLK;
    static constexpr int FM = BM / WM / 32;                 // epilogue groups per tile
};

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(1, 1)))
dgrad_pgemm(KernelArgs a)
{
    using Sh = PgemmShape<BM, BN, WM, WN>;
    constexpr int BK = 64;
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int A_BYTES = Sh::A_BYTES;
    constexpr int B_ROW = BN * 2;
    constexpr int STAGE = Sh::STAGE;
    constexpr int A_INSTR = A_BYTES / 1024 / NW;
    constexpr int B_INSTR = Sh::B_BYTES / 1024 / NW;
    constexpr int LD = A_INSTR + B_INSTR;         // loads per wave per slice
    constexpr int CH = TN / 8;                    // 16-byte chunks per staged pixel row
    constexpr int EROW = TN * 2;                  // bytes per staged pixel row
    constexpr int EBLK = Sh::EBLK;
    constexpr int PPI = 64 / CH;                  // pixels per store instruction
    constexpr int EST = 32 / PPI;                 // stores per epilogue group
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_BYTES % (1024 * NW) == 0 && Sh::B_BYTES % (1024 * NW) == 0, "whole 1 KiB blocks per wave");
    static_assert(BN % 64 == 0, "filter rows of at least 8 chunks");
    static_assert(Sh::LDS_USED <= 160 * 1024, "LDS budget");
    static_assert(CH >= 2 && CH <= 64 && 64 % CH == 0, "whole pixel rows per store");
    static_assert(LD + FM * EST < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char lds[Sh::LDS_USED];
    const uint32_t lds_u32 = (uint32_t)(uintptr_t)((lds_char*)lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int C = pin(a.C);
    const int K = pin(a.K);
    const int M = pin(a.ph[0].M);
    const int ksteps = pin(K / BK);               // the host admits K a multiple of 64
    const int tiles_n = pin(a.tiles_n);
    const int tiles_m = pin(a.ph[0].tiles_m);
    const int ntiles = pin(a.gemm_tiles);
    const int G = gridDim.x;
    const int slot = xcd_remap(blockIdx.x, G, a.group, a.xcd_mode);
    const int mytiles = pin(slot < ntiles ? (ntiles - 1 - slot) / G + 1 : 0);
    const int niter = pin(mytiles * ksteps);      // slices of this workgroup
    const bool order1 = a.order == 1;

    const i32x4 dy_desc = raw_descriptor(a.dy, a.dy_bytes);
    const i32x4 w_desc = raw_descriptor(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t e_dx = make_rsrc(a.dx, a.dx_bytes);

    // local tile u of this workgroup: its first pixel and channel
    auto tile_origin = [&](int u, int& m0, int& c0) __attribute__((always_inline)) {
        const int tile = slot + u * G;
        int tm, tn;
        if (!order1) {
            tm = tile / tiles_n;
            tn = tile - tm * tiles_n;
        } else {
            tn = tile / tiles_m;
            tm = tile - tn * tiles_m;
        }
        m0 = tm * BM;
        c0 = tn * BN;
    };

    // ---- request side. DMA block b = jn*NW + wave of a dy slice covers tile
    // rows 8b..8b+7; lane l fills row 8b + l/8 at chunk position l%8, holding
    // logical chunk (l%8) ^ dy_swizzle(row): dy[m0 + row, k0 + chunk*8], at
    // byte ((m0 + row)*K + k0 + chunk*8)*2 (the pixel index is the same in dy
    // and dx). Byte 16*l of block jn*NW + wave of a filter slice is row k,
    // position p, holding logical chunk p ^ w_swizzle(k): w[k0 + k, c0 + 8*chunk].
    uint32_t dy_vo[A_INSTR], w_vo[B_INSTR];
#pragma unroll
    for (int jn = 0; jn < A_INSTR; ++jn)
        dy_vo[jn] = 0x80000000u;
#pragma unroll
    for (int jn = 0; jn < B_INSTR; ++jn)
        w_vo[jn] = 0x80000000u;
    // the lanes' offsets within a tile's slice, formed when the stream enters the tile
    auto set_lanes = [&](int m0, int c0) __attribute__((always_inline)) {
#pragma unroll
        for (int jn = 0; jn < A_INSTR; ++jn) {
            const int row = (jn * NW + wave) * 8 + (lane >> 3);
            const int ak = ((lane & 7) ^ dy_swizzle(row)) * 8;
            dy_vo[jn] = m0 + row < M ? (uint32_t)(row * K + ak) * 2u : 0x80000000u;
        }
#pragma unroll
        for (int jn = 0; jn < B_INSTR; ++jn) {
            const int byte = (jn * NW + wave) * 1024 + 16 * lane;
            const int k = byte / B_ROW;
            const int cc = (((byte % B_ROW) / 16) ^ w_swizzle<B_ROW>(k)) * 8;
            w_vo[jn] = c0 + cc < C ? (uint32_t)(k * C + cc) * 2u : 0x80000000u;
        }
    };
    int item = 0;                 // the next item (slice) to request
    int rq_u = 0, rq_k = 0;       // its local tile and k step
    int rq_m0 = 0, rq_c0 = 0;
    uint32_t so_a = 0, so_b = 0;
    const uint32_t dma_base = pin(lds_u32 + (uint32_t)(wave * 1024));
    // the offsets of item `item` (past the last slice: every lane out of range)
    auto prepare = [&]() __attribute__((always_inline)) {
        if (item < niter) {
            if (rq_k == 0) {      // a new tile: lane offsets and masks for its pixels and channels
                tile_origin(rq_u, rq_m0, rq_c0);
                rq_m0 = pin(rq_m0);
                rq_c0 = pin(rq_c0);
                set_lanes(rq_m0, rq_c0);
            }
            so_a = pin((uint32_t)(rq_m0 * K + rq_k * BK) * 2u);
            so_b = pin((uint32_t)(rq_k * BK * C + rq_c0) * 2u);
        } else {
#pragma unroll
            for (int jn = 0; jn < A_INSTR; ++jn)
                dy_vo[jn] = 0x80000000u;
#pragma unroll
            for (int jn = 0; jn < B_INSTR; ++jn)
                w_vo[jn] = 0x80000000u;
            so_a = 0;
            so_b = 0;
        }
    };
    // load X of the prepared item into the stage at LDS address sbase (+ the wave's block)
    auto issue_one = [&](auto x_c, uint32_t sbase) __attribute__((always_inline)) {
        constexpr int X = decltype(x_c)::value;
        if constexpr (X < A_INSTR)
            dma16_at<(uint32_t)(X * NW * 1024)>(dy_desc, dy_vo[X], so_a, sbase);
        else
            dma16_at<(uint32_t)(A_BYTES + (X - A_INSTR) * NW * 1024)>(w_desc, w_vo[X - A_INSTR], so_b, sbase);
    };
    auto advance = [&]() __attribute__((always_inline)) {
        ++item;
        if (++rq_k == ksteps) {
            rq_k = 0;
            ++rq_u;
        }
    };

    // ---- fragment addresses (bytes within a stage, sub-step 0), as in dgrad_wide
    const int b_row0 = wm * TM + (lane & 31);
    const int b_sw = dy_swizzle(b_row0);
    const int g4 = (lane >> 4) & 3;
    const int rr = (lane & 15) >> 2;
    const int qq = lane & 3;
    int a_frag[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int cl = wn * TN + fn * 32 + (g4 & 1) * 16 + 4 * qq;
        const int krow = (g4 >> 1) * 8 + rr;
        a_frag[fn] = A_BYTES + krow * B_ROW + (((cl >> 3) ^ w_swizzle<B_ROW>(krow)) * 16) + (cl & 7) * 2;
    }
    // fragments of sub-step KK of the slice in the stage at byte sb
    auto read_frags = [&](uint32_t sb, auto kk_c, half8_t (&af)[FN], half8_t (&bf)[FM]) __attribute__((always_inline)) {
        constexpr int KK = decltype(kk_c)::value;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const lds_char* p = (lds_char*)lds + sb + a_frag[fn] + KK * 16 * B_ROW;
            const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)p);
            const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p + 4 * B_ROW));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
            af[fn] = __builtin_bit_cast(half8_t, u32x4{l2.x, l2.y, h2.x, h2.y});
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const lds_char* p = (lds_char*)lds + sb + (b_row0 + fm * 32) * 128 + (((KK * 2 + (lane >> 5)) ^ b_sw) * 16);
            bf[fm] = __builtin_bit_cast(half8_t, *(const __attribute__((address_space(3))) u32x4*)p);
        }
    };

    // ---- epilogue groups (after the tile's last slice). Group fm: pixels
    // wm*TM + fm*32 .. +31 of the wave's block, all TN channels, staged
    // through the wave's own block past the ring and stored as whole rows.
    lds_char* blk = (lds_char*)lds + Sh::STG0 + wave * EBLK;
    float16_t acc[FN][FM];
    auto stage_group = [&](auto fm_c) __attribute__((always_inline)) {
        constexpr int FMG = decltype(fm_c)::value;
        const int pw = lane & 31;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const half4_t o{(_Float16)acc[fn][FMG][4 * gq + 0], (_Float16)acc[fn][FMG][4 * gq + 1],
                                (_Float16)acc[fn][FMG][4 * gq + 2], (_Float16)acc[fn][FMG][4 * gq + 3]};
                const int q = fn * 4 + gq;
                *(__attribute__((address_space(3))) u32x2*)(blk + pw * EROW + ((q ^ ((pw >> 1) % CH)) * 16) + (lane >> 5) * 8) =
                    __builtin_bit_cast(u32x2, o);
            }
    };
    u32x4 ev[EST];
    auto read_group = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < EST; ++e) {
            const int pr = e * PPI + lane / CH;
            const int q = lane % CH;
            ev[e] = *(const __attribute__((address_space(3))) u32x4*)(blk + pr * EROW + ((q ^ ((pr >> 1) % CH)) * 16));
        }
    };
    const uint32_t e_lane = (uint32_t)((wm * TM + lane / CH) * C + wn * TN + (lane % CH) * 8) * 2u;
    const int e_row = wm * TM + lane / CH;
    const int e_col = wn * TN + (lane % CH) * 8;
    const uint32_t e_step = pin((uint32_t)(PPI * C * 2));
    auto store_group = [&](int fmg, int m0, int c0) __attribute__((always_inline)) {
        const uint32_t base = pin((uint32_t)((m0 + fmg * 32) * C + c0) * 2u);
        const int lim = M - m0 - fmg * 32;
        const bool col_ok = e_col < C - c0;
#pragma unroll
        for (int e = 0; e < EST; ++e) {
            const bool ok = col_ok & (e_row + e * PPI < lim);
            __builtin_amdgcn_raw_buffer_store_b128(ev[e], e_dx, ok ? e_lane + base + (uint32_t)e * e_step : 0x80000000u,
                                                   0, kStoreNT);
        }
    };

    // ---- the slices. Slice it of the walk lives in stage it % 3 (a run-time
    // index: its LDS base is a scalar). As in dgrad_wide, sub-steps 0 and 2
    // run on fragment set 0, 1 and 3 on set 1; the barrier sits after
    // sub-step 2's operations, then the next slice's first fragments are read
    // under sub-step 3. The LD loads of item it + 2 go out between the
    // operations of sub-steps 0-2 (past the last slice, every lane out of
    // range). The wait lets those loads stay in flight, plus, in a tile's
    // first slice after an epilogue, that epilogue's FM*EST stores: they were
    // issued after the loads of slice it + 1, which it waits for.
    constexpr int OPS = FM * FN;
    half8_t af[2][FN], bf[2][FM];
    int st = 0;
    auto slice = [&](auto first_c, bool after_epi, int it) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first_c)::value;
        const uint32_t sb = (uint32_t)(st * STAGE);
        const int rst = st == 0 ? 2 : st - 1;
        const uint32_t rbase = pin(dma_base + (uint32_t)(rst * STAGE));
        prepare();
        auto ops = [&](auto kk_c, int f, auto issue_c) __attribute__((always_inline)) {
            constexpr int KK = decltype(kk_c)::value;
            static_for<0, OPS>([&](auto j_c) {
                constexpr int J = decltype(j_c)::value;
                constexpr int fm = J / FN, fn = J % FN;
                if constexpr (FIRST && KK == 0)
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[f][fn], bf[f][fm], float16_t{}, 0, 0, 0);
                else
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[f][fn], bf[f][fm], acc[fn][fm], 0, 0, 0);
                if constexpr (decltype(issue_c)::value) {
                    static_for<0, LD>([&](auto x_c) {
                        if constexpr (decltype(x_c)::value * 3 * OPS / LD == KK * OPS + J)
                            issue_one(x_c, rbase);
                    });
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        ops(IC<0>{}, 0, IC<1>{});
        read_frags(sb, IC<2>{}, af[0], bf[0]);
        ops(IC<1>{}, 1, IC<1>{});
        read_frags(sb, IC<3>{}, af[1], bf[1]);
        ops(IC<2>{}, 0, IC<1>{});
        const bool has_next = it + 1 < niter;
        if (has_next) {
            if (FIRST && after_epi)
                wait_vmcnt<LD + FM * EST>();
            else
                wait_vmcnt<LD>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
            const uint32_t nsb = (uint32_t)((st == 2 ? 0 : st + 1) * STAGE);
            read_frags(nsb, IC<0>{}, af[0], bf[0]);
        }
        ops(IC<3>{}, 1, IC<0>{});
        if (has_next) {
            const uint32_t nsb = (uint32_t)((st == 2 ? 0 : st + 1) * STAGE);
            read_frags(nsb, IC<1>{}, af[1], bf[1]);
        }
        advance();
        st = st == 2 ? 0 : st + 1;
    };

    // ---- prologue: items 0 and 1
    prepare();
    static_for<0, LD>([&](auto x_c) { issue_one(x_c, dma_base); });
    advance();
    prepare();
    static_for<0, LD>([&](auto x_c) { issue_one(x_c, pin(dma_base + (uint32_t)STAGE)); });
    advance();
    wait_vmcnt<LD>();
    __syncthreads();
    read_frags(0u, IC<0>{}, af[0], bf[0]);
    read_frags(0u, IC<1>{}, af[1], bf[1]);
    int it = 0;
    for (int u = 0; u < mytiles; ++u) {
        slice(IC<true>{}, u > 0, it++);
        for (int k = 1; k < ksteps; ++k)
            slice(IC<false>{}, false, it++);
        int m0, c0;
        tile_origin(u, m0, c0);
        m0 = pin(m0);
        c0 = pin(c0);
        static_for<0, FM>([&](auto f_c) {
            stage_group(f_c);
            read_group();
            store_group(decltype(f_c)::value, m0, c0);
        });
    }
    wait_vmcnt<0>();   // the loads past the last slice have written LDS before the workgroup ends
}

// The layers this kernel runs: 1x1, stride 1, no padding (dx and dy share
// the pixel index), no fused epilogue factor, K a multiple of 64.
template <int BM, int BN, int WM, int WN>
bool pgemm_fits(int R, int S, int stride, int pad, int K, int epi)
{
    return R == 1 && S == 1 && stride == 1 && pad == 0 && epi == kEpiNone && K % 64 == 0 && K > 0;
}

template <int BM, int BN, int WM, int WN>
hipError_t pgemm_launch(const KernelArgs& a, hipStream_t stream)
{
    const PhaseArg& ph = a.ph[0];
    if (a.sk || a.nzphases > 0 || a.ncomp > 0 || a.zstripes > 0 || a.nphases != 1 || a.total_tiles != a.gemm_tiles ||
        a.grid < 1 || a.grid > a.gemm_tiles || ph.nr != 1 || ph.nt != 1 || ph.r0 != 0 || ph.t0 != 0 || ph.dr0 != 0 ||
        ph.dt0 != 0 || ph.ph != 0 || ph.pw != 0 || ph.Wp != a.W || ph.div_hw.d != (uint32_t)(a.H * a.W) ||
        a.P != a.H || a.Q != a.W || a.order == 2 || !pgemm_fits<BM, BN, WM, WN>(a.R, a.S, a.stride, 0, a.K, a.epi))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((dgrad_pgemm<BM, BN, WM, WN>), dim3(a.grid), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
int pgemm_resident(void)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(dgrad_pgemm<BM, BN, WM, WN>),
                                                     64 * WM * WN, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    return n > 0 ? n : 1;
}

template <int BM, int BN, int WM, int WN>
int pgemm_private(void)
{
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(dgrad_pgemm<BM, BN, WM, WN>)) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return (int)attr.localSizeBytes;
}

// The compiled configurations of this kernel: (BM, BN, WM, WN).
#define CBW_PGEMM_CONFIGS(X) \
    X(256, 128, 2, 2)

#define CBW_PGEMM_ENTRY(BM, BN, WM, WN) \
    {BM, BN, 64, WM, WN, #BM "x" #BN "x64/" #WM "x" #WN "p", PgemmShape<BM, BN, WM, WN>::LDS_USED, false, false, false, true},
const TileConfig kPgemmConfigs[] = {CBW_PGEMM_CONFIGS(CBW_PGEMM_ENTRY)};
constexpr int kNumPgemm = sizeof(kPgemmConfigs) / sizeof(kPgemmConfigs[0]);

using PgemmLaunchFn = hipError_t (*)(const KernelArgs&, hipStream_t);
using PgemmFitsFn = bool (*)(int, int, int, int, int, int);
#define CBW_PGEMM_LAUNCH(BM, BN, WM, WN) &pgemm_launch<BM, BN, WM, WN>,
#define CBW_PGEMM_FITS(BM, BN, WM, WN) &pgemm_fits<BM, BN, WM, WN>,
#define CBW_PGEMM_RESIDENT(BM, BN, WM, WN) &pgemm_resident<BM, BN, WM, WN>,
#define CBW_PGEMM_PRIVATE(BM, BN, WM, WN) &pgemm_private<BM, BN, WM, WN>,
const PgemmLaunchFn kPgemmLaunch[] = {CBW_PGEMM_CONFIGS(CBW_PGEMM_LAUNCH)};
const PgemmFitsFn kPgemmFits[] = {CBW_PGEMM_CONFIGS(CBW_PGEMM_FITS)};
int (*const kPgemmResident[])(void) = {CBW_PGEMM_CONFIGS(CBW_PGEMM_RESIDENT)};
int (*const kPgemmPrivate[])(void) = {CBW_PGEMM_CONFIGS(CBW_PGEMM_PRIVATE)};

}  // namespace

int pgemm_num_configs() { return kNumPgemm; }

const TileConfig& pgemm_config(int i) { return kPgemmConfigs[i]; }

bool pgemm_admits(int i, int R, int S, int stride, int pad, int K, int epi)
{
    return i >= 0 && i < kNumPgemm && kPgemmFits[i](R, S, stride, pad, K, epi);
}

hipError_t launch_pgemm(int i, const KernelArgs& a, hipStream_t stream)
{
    if (i < 0 || i >= kNumPgemm)
        return hipErrorInvalidValue;
    return kPgemmLaunch[i](a, stream);
}

int pgemm_blocks_per_cu(int i) { return (i >= 0 && i < kNumPgemm) ? kPgemmResident[i]() : 1; }

int pgemm_private_bytes(int i) { return (i >= 0 && i < kNumPgemm) ? kPgemmPrivate[i]() : -1; }

}  // namespace cbw
