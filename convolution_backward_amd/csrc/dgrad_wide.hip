// A second dgrad kernel for launches made only of GEMM tiles (no zero
// phases, no split reduction): fewer, larger wave tiles.
//
// The operation and the operand path are those of dgrad_igemm in
// dgrad_kernels.hip (the backward-data convolution of "[CUTLASS] Conv2d
// dgrad", apache/tvm PR #10110, as an implicit GEMM per stride phase): 64-wide
// reduction slices (taps outermost, then k) travel HBM/L2 -> LDS with 16-byte
// direct-to-LDS buffer loads in a ring of three stages, two slices ahead, with
// the same XOR-permuted LDS layouts, and v_mfma_f32_32x32x16_f16 takes A =
// filter^T (transpose reads) and B = dy^T (16-byte reads).
//
// What differs is the work per wave. A 256x128 tile is split over four waves
// of 128 pixels x 64 channels (instead of eight of 64x64): per 64-wide slice a
// wave issues 32 matrix-core operations (1024 cycles, one wave per SIMD) for
// 16 KiB of dy and 8 KiB of filter fragments, so the CU reads 96 KiB of LDS
// per slice instead of 128 KiB, and only four waves meet at each barrier.
// Each workgroup owns one tile (the grid is the tile count, one workgroup per
// CU at a time for LDS reasons), which keeps the wave-uniform state small
// enough for the scalar register file.
#include "dgrad_internal.h"
#include "kernel_common.h"

namespace cbw {
namespace {

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(1, 1)))
dgrad_wide(KernelArgs a)
{
    constexpr int BK = 64;
    constexpr int NW = WM * WN;
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
    static_assert(LD < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE];
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
    const int SC = pin(a.S * C);          // filter elements per tap row
    const int RSC = pin(a.R * SC);        // filter elements per k
    const int ksteps = (K + BK - 1) / BK;

    // ---- this workgroup's tile (the grid is the tile count)
    const int tile = xcd_remap(blockIdx.x, gridDim.x, a.group, a.xcd_mode);
    int pi = 0;
    for (int i = 1; i < a.nphases; ++i)
        if (tile >= a.ph[i].tile_begin)
            pi = i;
    const PhaseArg& ph = a.ph[pi];
    const int local = tile - ph.tile_begin;
    int tm, tn;
    if (a.order != 1) {    // channel tiles of one pixel block are consecutive
        tm = local / a.tiles_n;
        tn = local - tm * a.tiles_n;
    } else {               // pixel blocks of one channel tile are consecutive
        tn = local / ph.tiles_m;
        tm = local - tn * ph.tiles_m;
    }
    const int m0 = pin(tm * BM);
    const int c0 = pin(tn * BN);
    const int niter = pin(ph.nr * ph.nt * ksteps);
    const int s = pin(a.stride);
    const int dr0 = pin(ph.dr0), dt0 = pin(ph.dt0), ntap = pin(ph.nt);
    const int wt0 = pin(ph.r0 * SC + ph.t0 * C + c0);

    const i32x4 dy_desc = raw_descriptor(a.dy, a.dy_bytes);
    const i32x4 w_desc = raw_descriptor(a.w, a.w_bytes);

    // ---- request side. DMA block b = jn*NW + wave of a dy slice covers tile
    // rows 8b..8b+7; lane l fills row 8b + l/8 at chunk position l%8, holding
    // logical chunk (l%8) ^ dy_swizzle(row). Byte 16*l of block jn*NW + wave
    // of a filter slice is row k, position p, holding logical chunk
    // p ^ w_swizzle(k). A lane's dy offset changes only at tap boundaries:
    // per tap it is a byte offset (or 2^31 for a padding tap or a dead row)
    // plus the wave-uniform 2*k0 in the load's scalar offset.
    int a_k[A_INSTR], b_k[B_INSTR];
    uint32_t a_off[A_INSTR];   // byte offset of dy[n, i, j, chunk*8], modulo 2^32 (exact where loaded)
    int a_i[A_INSTR], a_j[A_INSTR];
    uint32_t dy_vo[A_INSTR];   // the lane's dy byte offset for the current tap and k step
    uint32_t w_vt[B_INSTR];    // the lane's filter byte offset in the tile (2^31: channel past C)
    uint32_t w_vo[B_INSTR];    // ... for the current k step
#pragma unroll
    for (int jn = 0; jn < A_INSTR; ++jn) {
        const int row = (jn * NW + wave) * 8 + (lane >> 3);
        a_k[jn] = ((lane & 7) ^ dy_swizzle(row)) * 8;
        const int m = m0 + row;
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        a_i[jn] = m < ph.M ? (int)i : -(1 << 24);   // a dead row fails every p >= 0 test
        a_j[jn] = (int)j;
        a_off[jn] = (((n * (uint32_t)P + i) * (uint32_t)Q + j) * (uint32_t)K + (uint32_t)a_k[jn]) * 2u;
    }
#pragma unroll
    for (int jn = 0; jn < B_INSTR; ++jn) {
        const int byte = (jn * NW + wave) * 1024 + 16 * lane;
        const int k = byte / B_ROW;
        const int pos = (byte % B_ROW) / 16;
        const int cc = (pos ^ w_swizzle<B_ROW>(k)) * 8;
        b_k[jn] = k;
        w_vt[jn] = c0 + cc >= C ? 0x80000000u : (uint32_t)(k * RSC + cc) * 2u;
    }
    int ar = 0, at = 0, k0 = 0;   // request cursor: row tap, column tap, k step
    bool new_tap = true;
    uint32_t q_wtap = 0;          // filter byte offset of the current tap (wave-uniform)
    uint32_t q_base = 0;          // LDS address of the stage being filled
    auto prepare = [&](int buf) {
        if (new_tap) {            // once per tap: padding checks and dy offsets
            new_tap = false;
            const int dr = dr0 - ar;
            const int dt = dt0 - at;
            const uint32_t tapoff = (uint32_t)((dr * Q + dt) * K) * 2u;
#pragma unroll
            for (int jn = 0; jn < A_INSTR; ++jn) {
                const bool ok = ((unsigned)(a_i[jn] + dr) < (unsigned)P) & ((unsigned)(a_j[jn] + dt) < (unsigned)Q);
                dy_vo[jn] = ok ? a_off[jn] + tapoff : 0x80000000u;
            }
#pragma unroll
            for (int jn = 0; jn < B_INSTR; ++jn)
                w_vo[jn] = w_vt[jn];
            q_wtap = (uint32_t)(wt0 + ar * s * SC + at * s * C) * 2u;
        }
        if (k0 + BK > K) {        // ragged last k step of a tap: mask the lanes past K
#pragma unroll
            for (int jn = 0; jn < A_INSTR; ++jn)
                dy_vo[jn] = k0 + a_k[jn] >= K ? 0x80000000u : dy_vo[jn];
#pragma unroll
            for (int jn = 0; jn < B_INSTR; ++jn)
                w_vo[jn] = k0 + b_k[jn] >= K ? 0x80000000u : w_vo[jn];
        }
        q_base = lds_u32 + (uint32_t)(buf * STAGE);
    };
    // Issue load number x of the prepared slice (dy blocks first, then
    // filter blocks).
    auto issue_one = [&](int x) {
        if (x < A_INSTR) {
            dma16(dy_desc, dy_vo[x], (uint32_t)k0 * 2u, q_base + (uint32_t)((x * NW + wave) * 1024));
        } else {
            const int jn = x - A_INSTR;
            dma16(w_desc, w_vo[jn], q_wtap + (uint32_t)(k0 * RSC) * 2u,
                  q_base + (uint32_t)(A_BYTES + (jn * NW + wave) * 1024));
        }
    };
    auto advance = [&]() {        // the cursor past the issued slice: k innermost, then taps
        k0 += BK;
        if (k0 >= K) {
            k0 = 0;
            new_tap = true;
            if (++at == ntap) {
                at = 0;
                ++ar;
            }
        }
    };

    // ---- fragment addresses (bytes within a stage, sub-step 0)
    // dy^T operand (B): row m = wm*TM + fm*32 + lane%32, k chunk 2*kk + lane/32.
    const int b_row0 = wm * TM + (lane & 31);
    const int b_sw = dy_swizzle(b_row0);          // the same for every fm (fm*32 keeps bits 1..3)
    // filter^T operand (A): group g = lane/16 covers channels +16*(g&1), k +8*(g>>1);
    // within it lane 4r+q reads row r, channels 4q..4q+3.
    const int g = (lane >> 4) & 3;
    const int rr = (lane & 15) >> 2;
    const int qq = lane & 3;
    int a_frag[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int cl = wn * TN + fn * 32 + (g & 1) * 16 + 4 * qq;
        const int krow = (g >> 1) * 8 + rr;
        a_frag[fn] = A_BYTES + krow * B_ROW + (((cl >> 3) ^ w_swizzle<B_ROW>(krow)) * 16) + (cl & 7) * 2;
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
    // ---- the slice loop. Slice it lives in stage it % 3; its loads were
    // issued during slice it - 2. The slice's four 16-wide sub-steps run on
    // fragments in two register sets: sub-steps 0 and 2 in set 0, 1 and 3 in
    // set 1, each set refilled right after the sub-step that used it.
    //
    // One barrier per slice, in its middle: after the operations of sub-step 2
    // are issued, the wave waits for its loads of slice it + 1 (its loads of
    // slice it + 2, issued since, may stay in flight) and for its own
    // fragment reads of slice it, then meets the other waves. Past that
    // barrier (a) slice it + 1 is in LDS and (b) no wave reads slice it's
    // stage any more, so set 0 is refilled with sub-step 0 of slice it + 1
    // while sub-step 3 runs, set 1 with its sub-step 1 after, and slice it +
    // 1's loads of slice it + 3 may overwrite stage it % 3. The next slice
    // then starts on fragments already in registers, and the operations in
    // flight keep the matrix core busy while the wave waits at the barrier.
    //
    // The LD loads of slice it + 2 go out one at a time between the
    // operations of sub-steps 0-2 (with one wave per SIMD, a load whose issue
    // waits for the address unit then holds up no operation: the one just
    // issued keeps the matrix core busy). The scheduling barriers keep that
    // order.
    constexpr int OPS = FM * FN;          // operations per sub-step
    half8_t af[2][FN], bf[2][FM];
    auto ops = [&](int f, int kk, bool issue) {
#pragma unroll
        for (int j = 0; j < OPS; ++j) {
            const int fm = j / FN, fn = j % FN;
            acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[f][fn], bf[f][fm], acc[fn][fm], 0, 0, 0);
            const int op = kk * OPS + j;
#pragma unroll
            for (int x = 0; x < LD; ++x)
                if (x * 3 * OPS / LD == op && issue)
                    issue_one(x);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    prepare(0);
#pragma unroll
    for (int x = 0; x < LD; ++x)
        issue_one(x);
    advance();
    if (niter > 1) {
        prepare(1);
#pragma unroll
        for (int x = 0; x < LD; ++x)
            issue_one(x);
        advance();
        wait_vmcnt<LD>();
    } else {
        wait_vmcnt<0>();
    }
    __syncthreads();                      // slice 0 is in LDS
    read_frags(0, 0, af[0], bf[0]);
    read_frags(0, 1, af[1], bf[1]);
    int cbuf = 0, rbuf = 2;
    for (int it = 0; it < niter; ++it) {
        const int sb = cbuf * STAGE;
        const bool more = it + 2 < niter;   // loads of slice it + 2 go out during this slice
        if (more)
            prepare(rbuf);
        ops(0, 0, more);
        read_frags(sb, 2, af[0], bf[0]);
        ops(1, 1, more);
        read_frags(sb, 3, af[1], bf[1]);
        ops(0, 2, more);
        const int nbuf = cbuf == 2 ? 0 : cbuf + 1;
        if (it + 1 < niter) {
            if (more)
                wait_vmcnt<LD>();
            else
                wait_vmcnt<0>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
            read_frags(nbuf * STAGE, 0, af[0], bf[0]);
        }
        ops(1, 3, false);
        if (it + 1 < niter)
            read_frags(nbuf * STAGE, 1, af[1], bf[1]);
        if (more) {
            advance();
            rbuf = rbuf == 2 ? 0 : rbuf + 1;
        }
        cbuf = nbuf;
    }

    // ---- epilogue: acc x g(z) -> fp16 (RNE), staged through the stage of
    // the last slice and stored as whole pixel rows (see dgrad_igemm). The
    // lane holds channels 8*gq + 4*(lane/32) .. +3 of block fn, pixel lane%32
    // of pixel group fm. No load is in flight: the last slice's wait was for
    // all of them.
    const int sdone = cbuf == 0 ? 2 : cbuf - 1;
    constexpr int CH = TN / 8;            // 16-byte chunks per staged pixel row
    constexpr int EROW = TN * 2;          // bytes per staged pixel row
    constexpr int EBLK = 32 * EROW;       // bytes per wave per pixel group
    constexpr int PPI = 64 / CH;          // pixels per store instruction
    constexpr int EST = 32 / PPI;         // store instructions per pixel group
    static_assert(NW * EBLK <= STAGE, "the staging blocks fit in one stage");
    static_assert(CH >= 2 && CH <= 64 && 64 % CH == 0, "whole pixel rows per store");
    auto pixel_offset = [&](int m) -> uint32_t {   // dx element offset of lattice row m
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        const uint32_t pix = (n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)i)) * (uint32_t)a.W
                             + (uint32_t)(ph.pw + s * (int)j);
        return pix * (uint32_t)C;
    };
    auto epilogue = [&](auto tag) {
        constexpr int E = decltype(tag)::value;
        const __amdgpu_buffer_rsrc_t e_dx = make_rsrc(a.dx, a.dx_bytes);
        const __amdgpu_buffer_rsrc_t z_rsrc = make_rsrc(E != kEpiNone ? a.z : a.dx, a.dx_bytes);
        const int cw = c0 + wn * TN;      // first channel of this wave's block
        u32x2 zr[FM][FN][4];      // every z of the wave's block, loaded before the first use
        if constexpr (E != kEpiNone) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int m = m0 + wm * TM + fm * 32 + (lane & 31);
                const uint32_t pix = pixel_offset(m);
                const uint32_t m_bad = (uint32_t)(m >= ph.M);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int c = cw + fn * 32 + 8 * gq + 4 * (lane >> 5);
                        zr[fm][fn][gq] = __builtin_amdgcn_raw_buffer_load_b64(
                            z_rsrc, out_of_range_if(m_bad | (uint32_t)(c >= C), (pix + (uint32_t)c) * 2u), 0, 0);
                    }
            }
        }
        lds_char* blk = (lds_char*)lds + sdone * STAGE + wave * EBLK;
        __syncthreads();   // every wave is done reading the stage's operands
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int pw = lane & 31;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    float v0 = acc[fn][fm][4 * gq + 0];
                    float v1 = acc[fn][fm][4 * gq + 1];
                    float v2 = acc[fn][fm][4 * gq + 2];
                    float v3 = acc[fn][fm][4 * gq + 3];
                    if constexpr (E != kEpiNone) {
                        const half4_t zz = __builtin_bit_cast(half4_t, zr[fm][fn][gq]);
                        v0 *= epilogue_factor<E>((float)zz[0]);
                        v1 *= epilogue_factor<E>((float)zz[1]);
                        v2 *= epilogue_factor<E>((float)zz[2]);
                        v3 *= epilogue_factor<E>((float)zz[3]);
                    }
                    const half4_t o{(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
                    const int q = fn * 4 + gq;
                    *(__attribute__((address_space(3))) u32x2*)(blk + pw * EROW + ((q ^ ((pw >> 1) % CH)) * 16) + (lane >> 5) * 8) =
                        __builtin_bit_cast(u32x2, o);
                }
            }
            // read back whole chunks: instruction e covers pixels e*PPI .. e*PPI+PPI-1
#pragma unroll
            for (int e = 0; e < EST; ++e) {
                const int pr = e * PPI + lane / CH;
                const int q = lane % CH;
                const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(blk + pr * EROW + ((q ^ ((pr >> 1) % CH)) * 16));
                const int m = m0 + wm * TM + fm * 32 + pr;
                const int c = cw + q * 8;
                const uint32_t bad = (uint32_t)(m >= ph.M) | (uint32_t)(c >= C);
                __builtin_amdgcn_raw_buffer_store_b128(v, e_dx, out_of_range_if(bad, (pixel_offset(m) + (uint32_t)c) * 2u),
                                                       0, kStoreNT);
            }
        }
    };
    switch (a.epi) {
    case kEpiDRelu: epilogue(EpiTag<kEpiDRelu>{}); break;
    case kEpiDHardswish: epilogue(EpiTag<kEpiDHardswish>{}); break;
    default: epilogue(EpiTag<kEpiNone>{}); break;
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t wide_launch(const KernelArgs& a, hipStream_t stream)
{
    if (a.sk || a.nzphases > 0 || a.ncomp > 0 || a.zstripes > 0 || a.total_tiles != a.gemm_tiles ||
        a.grid != a.gemm_tiles)
        return hipErrorInvalidValue;   // the host plans only GEMM tiles, one per workgroup, for this kernel
    hipLaunchKernelGGL((dgrad_wide<BM, BN, WM, WN>), dim3(a.grid), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
int wide_resident(void)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(dgrad_wide<BM, BN, WM, WN>),
                                                     64 * WM * WN, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    return n > 0 ? n : 1;
}

template <int BM, int BN, int WM, int WN>
int wide_private(void)
{
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(dgrad_wide<BM, BN, WM, WN>)) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return (int)attr.localSizeBytes;
}

// The compiled configurations of this kernel: (BM, BN, WM, WN).
#define CBW_WIDE_CONFIGS(X) \
    X(256, 128, 2, 2)

#define CBW_WIDE_ENTRY(BM, BN, WM, WN) \
    {BM, BN, 64, WM, WN, #BM "x" #BN "x64/" #WM "x" #WN "w", 3 * (BM + BN) * 64 * 2, false, false, true},
const TileConfig kWideConfigs[] = {CBW_WIDE_CONFIGS(CBW_WIDE_ENTRY)};
constexpr int kNumWide = sizeof(kWideConfigs) / sizeof(kWideConfigs[0]);

using WideLaunchFn = hipError_t (*)(const KernelArgs&, hipStream_t);
#define CBW_WIDE_LAUNCH(BM, BN, WM, WN) &wide_launch<BM, BN, WM, WN>,
#define CBW_WIDE_RESIDENT(BM, BN, WM, WN) &wide_resident<BM, BN, WM, WN>,
#define CBW_WIDE_PRIVATE(BM, BN, WM, WN) &wide_private<BM, BN, WM, WN>,
const WideLaunchFn kWideLaunch[] = {CBW_WIDE_CONFIGS(CBW_WIDE_LAUNCH)};
int (*const kWideResident[])(void) = {CBW_WIDE_CONFIGS(CBW_WIDE_RESIDENT)};
int (*const kWidePrivate[])(void) = {CBW_WIDE_CONFIGS(CBW_WIDE_PRIVATE)};

}  // namespace

int wide_num_configs() { return kNumWide; }

const TileConfig& wide_config(int i) { return kWideConfigs[i]; }

hipError_t launch_wide(int i, const KernelArgs& a, hipStream_t stream)
{
    if (i < 0 || i >= kNumWide)
        return hipErrorInvalidValue;
    return kWideLaunch[i](a, stream);
}

int wide_blocks_per_cu(int i) { return (i >= 0 && i < kNumWide) ? kWideResident[i]() : 1; }

int wide_private_bytes(int i) { return (i >= 0 && i < kNumWide) ? kWidePrivate[i]() : -1; }

}  // namespace cbw
