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
//
// The fused epilogues' z tile (BM pixels x BN channels, fp16) travels to LDS
// during the last two slices, into the stages that no slice needs any more,
// so its load latency hides behind matrix-core work instead of opening the
// epilogue.
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
    auto pixel_offset = [&](int m) __attribute__((always_inline)) -> uint32_t {   // dx element offset of lattice row m
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        const uint32_t pix = (n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)i)) * (uint32_t)a.W
                             + (uint32_t)(ph.pw + s * (int)j);
        return pix * (uint32_t)C;
    };

    // ---- the request stream: items 0..niter-1 are the slices; items niter
    // and niter + 1 carry the fused epilogue's z tile (BM pixels x BN
    // channels), each as one slice's worth of loads. Item j goes to stage
    // j mod 3 like a slice, so z lands in the two stages no slice needs any
    // more while the last two slices run, and its latency hides behind them.
    // Without z (or past its end) the lanes are out of range and write zeros.
    // Load X of an item fills this wave's block X*NW + wave of the stage
    // (blocks 0..A_INSTR*NW-1 are the dy rows of a slice, the rest its filter
    // rows). In the z items, 1 KiB block b holds z rows ZRPB*b.., row p's
    // chunk c at position c ^ (p % ZCH); item niter holds blocks
    // 0..LD*NW-1, item niter + 1 the rest.
    constexpr int ZROW = BN * 2;
    constexpr int ZCH = ZROW / 16;                   // chunks per z row
    constexpr int ZRPB = 1024 / ZROW;                // rows per 1 KiB block
    constexpr int ZX = BM * ZROW / 1024 / NW;        // z blocks per wave
    constexpr int ZA_ROWS = LD * NW * ZRPB;          // rows in item niter
    static_assert(ZROW <= 1024 && 1024 % ZROW == 0 && 64 % ZCH == 0, "whole z rows per block");
    static_assert((BM * ZROW / 1024) % NW == 0, "whole z blocks per wave");
    static_assert(ZX > LD && ZX <= 2 * LD, "the z tile spans the two items");
    static_assert(A_BYTES == A_INSTR * NW * 1024, "block X of a stage at X*NW KiB");
    const bool zpre = a.epi != kEpiNone;
    const int zstage_a = niter % 3, zstage_b = (niter + 1) % 3;
    const i32x4 z_desc = raw_descriptor(zpre ? a.z : a.dx, a.dx_bytes);
    auto z_offset = [&](int x) __attribute__((always_inline)) -> uint32_t {          // this lane's z byte offset in block x*NW + wave
        const int row = (x * NW + wave) * ZRPB + lane / ZCH;
        const int c = ((lane % ZCH) ^ (row % ZCH)) * 8;
        const int m = m0 + row;
        const uint32_t bad = (uint32_t)(!zpre) | (uint32_t)(x >= ZX) | (uint32_t)(m >= ph.M) | (uint32_t)(c0 + c >= C);
        const uint32_t off = bad ? 0u : (pixel_offset(m) + (uint32_t)(c0 + c)) * 2u;
        return out_of_range_if(bad, off);
    };
    auto z_row_lds = [&](int p) __attribute__((always_inline)) -> int {            // LDS byte offset of z row p
        return p < ZA_ROWS ? zstage_a * STAGE + p * ZROW : zstage_b * STAGE + (p - ZA_ROWS) * ZROW;
    };

    int item = 0;                 // the next item to prepare
    int ar = 0, at = 0, k0 = 0;   // slice cursor: row tap, column tap, k step
    bool new_tap = true;
    uint32_t q_wtap = 0;          // filter byte offset of the current tap (wave-uniform)
    // the prepared item's descriptors and scalar offsets: dy-block loads (a)
    // and filter-block loads (b)
    i32x4 desc_a = dy_desc, desc_b = w_desc;
    uint32_t so_a = 0, so_b = 0;
    // LDS address of this wave's first block; block X of stage st lies a
    // compile-time distance further (m0 is formed with one add)
    const uint32_t dma_base = pin(lds_u32 + (uint32_t)(wave * 1024));
    auto prepare = [&]() __attribute__((always_inline)) {
        if (item < niter) {
            if (new_tap) {        // once per tap: padding checks and dy offsets
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
            if (k0 + BK > K) {    // ragged last k step of a tap: mask the lanes past K
#pragma unroll
                for (int jn = 0; jn < A_INSTR; ++jn)
                    dy_vo[jn] = k0 + a_k[jn] >= K ? 0x80000000u : dy_vo[jn];
#pragma unroll
                for (int jn = 0; jn < B_INSTR; ++jn)
                    w_vo[jn] = k0 + b_k[jn] >= K ? 0x80000000u : w_vo[jn];
            }
            so_a = pin((uint32_t)k0 * 2u);
            so_b = pin(q_wtap + (uint32_t)(k0 * RSC) * 2u);
        } else {                  // a z item
            const int x0 = (item - niter) * LD;
#pragma unroll
            for (int jn = 0; jn < A_INSTR; ++jn)
                dy_vo[jn] = z_offset(x0 + jn);
#pragma unroll
            for (int jn = 0; jn < B_INSTR; ++jn)
                w_vo[jn] = z_offset(x0 + A_INSTR + jn);
            desc_a = z_desc;
            desc_b = z_desc;
            so_a = 0;
            so_b = 0;
        }
    };
    // Issue load X of the prepared item into stage ST.
    auto issue_one = [&](auto st_c, auto x_c) __attribute__((always_inline)) {
        constexpr int ST = decltype(st_c)::value;
        constexpr int X = decltype(x_c)::value;
        if constexpr (X < A_INSTR)
            dma16_at<(uint32_t)(ST * STAGE + X * NW * 1024)>(desc_a, dy_vo[X], so_a, dma_base);
        else
            dma16_at<(uint32_t)(ST * STAGE + X * NW * 1024)>(desc_b, w_vo[X - A_INSTR], so_b, dma_base);
    };
    auto advance = [&]() __attribute__((always_inline)) {        // past the issued item; for a slice: k innermost, then taps
        ++item;
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
    auto read_frags = [&](auto st_c, int kk, half8_t (&af)[FN], half8_t (&bf)[FM]) __attribute__((always_inline)) {
        constexpr int sb = decltype(st_c)::value * STAGE;
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
    // item it + 2, issued since, may stay in flight) and for its own
    // fragment reads of slice it, then meets the other waves. Past that
    // barrier (a) slice it + 1 is in LDS and (b) no wave reads slice it's
    // stage any more, so set 0 is refilled with sub-step 0 of slice it + 1
    // while sub-step 3 runs, set 1 with its sub-step 1 after, and slice it +
    // 1's loads of item it + 3 may overwrite stage it % 3. The next slice
    // then starts on fragments already in registers, and the operations in
    // flight keep the matrix core busy while the wave waits at the barrier.
    // Every slice has the same instruction stream (the z items stand in for
    // the missing slices it + 2 at the end), which keeps branches out of it.
    //
    // The LD loads of item it + 2 go out one at a time between the
    // operations of sub-steps 0-2 (with one wave per SIMD, a load whose issue
    // waits for the address unit then holds up no operation: the one just
    // issued keeps the matrix core busy). The scheduling barriers keep that
    // order.
    constexpr int OPS = FM * FN;          // operations per sub-step
    half8_t af[2][FN], bf[2][FM];
    auto ops = [&](auto st_c, int f, auto kk_c, auto issue_c) __attribute__((always_inline)) {
        constexpr int KK = decltype(kk_c)::value;
        static_for<0, OPS>([&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            constexpr int fm = J / FN, fn = J % FN;
            acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[f][fn], bf[f][fm], acc[fn][fm], 0, 0, 0);
            if constexpr (decltype(issue_c)::value) {
                static_for<0, LD>([&](auto x_c) {
                    if constexpr (decltype(x_c)::value * 3 * OPS / LD == KK * OPS + J)
                        issue_one(st_c, x_c);
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // Slice it in stage ST (= it % 3); item it + 2 (a slice or a z item)
    // goes out during it into stage (ST + 2) % 3.
    auto slice = [&](auto st_c, int it) __attribute__((always_inline)) {
        constexpr IC<(decltype(st_c)::value + 1) % 3> next_c{};
        constexpr IC<(decltype(st_c)::value + 2) % 3> req_c{};
        prepare();
        ops(req_c, 0, IC<0>{}, IC<1>{});
        read_frags(st_c, 2, af[0], bf[0]);
        ops(req_c, 1, IC<1>{}, IC<1>{});
        read_frags(st_c, 3, af[1], bf[1]);
        ops(req_c, 0, IC<2>{}, IC<1>{});
        const bool has_next = it + 1 < niter;
        if (has_next) {
            // slice it + 1's loads went out before item it + 2's, which may
            // stay in flight
            wait_vmcnt<LD>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
            read_frags(next_c, 0, af[0], bf[0]);
        }
        ops(req_c, 1, IC<3>{}, IC<0>{});
        if (has_next)
            read_frags(next_c, 1, af[1], bf[1]);
        advance();
    };

    // items 0 and 1 (slice 1, or the first z item when niter is 1)
    prepare();
    static_for<0, LD>([&](auto x_c) { issue_one(IC<0>{}, x_c); });
    advance();
    prepare();
    static_for<0, LD>([&](auto x_c) { issue_one(IC<1>{}, x_c); });
    advance();
    wait_vmcnt<LD>();
    __syncthreads();                      // slice 0 is in LDS
    read_frags(IC<0>{}, 0, af[0], bf[0]);
    read_frags(IC<0>{}, 1, af[1], bf[1]);
    // three slices per pass, so every stage index is a compile-time constant
    // (one exit, so the accumulators keep their registers through the loop)
    for (int it = 0; it < niter;) {
        slice(IC<0>{}, it);
        ++it;
        if (it < niter) {
            slice(IC<1>{}, it);
            ++it;
        }
        if (it < niter) {
            slice(IC<2>{}, it);
            ++it;
        }
    }

    // ---- epilogue: acc x g(z) -> fp16 (RNE), staged through the stage of
    // the last slice and stored as whole pixel rows (see dgrad_igemm). The
    // lane holds channels 8*gq + 4*(lane/32) .. +3 of block fn, pixel lane%32
    // of pixel group fm. The two z items may still be in flight: every
    // wave waits for its loads before the barrier that opens the epilogue.
    const int sdone = (niter - 1) % 3;
    constexpr int CH = TN / 8;            // 16-byte chunks per staged pixel row
    constexpr int EROW = TN * 2;          // bytes per staged pixel row
    constexpr int EBLK = 32 * EROW;       // bytes per wave per pixel group
    constexpr int PPI = 64 / CH;          // pixels per store instruction
    constexpr int EST = 32 / PPI;         // store instructions per pixel group
    static_assert(NW * EBLK <= STAGE, "the staging blocks fit in one stage");
    static_assert(CH >= 2 && CH <= 64 && 64 % CH == 0, "whole pixel rows per store");
    auto epilogue = [&](auto tag) __attribute__((always_inline)) {
        constexpr int E = decltype(tag)::value;
        const __amdgpu_buffer_rsrc_t e_dx = make_rsrc(a.dx, a.dx_bytes);
        const int cw = c0 + wn * TN;      // first channel of this wave's block
        lds_char* blk = (lds_char*)lds + sdone * STAGE + wave * EBLK;
        wait_vmcnt<0>();   // this wave's part of the z tile is in LDS (and no load writes LDS after the end)
        __syncthreads();   // every wave is done reading the stage's operands, and the z tile is whole
        const int pw = lane & 31;
        // z of pixel group fm (the lane's 4 channels of each 8-channel chunk),
        // read from LDS one group ahead, before the staging writes of the
        // group in hand, so the reads overlap the arithmetic
        u32x2 zr[2][FN][4];
        auto read_z = [&](int fm, u32x2 (&zz)[FN][4]) __attribute__((always_inline)) {
            const int p = wm * TM + fm * 32 + pw;                  // z row in the tile
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int cz = wn * TN + fn * 32 + 8 * gq;     // first channel of the chunk
                    zz[fn][gq] = *(const __attribute__((address_space(3))) u32x2*)(
                        (lds_char*)lds + z_row_lds(p) + ((((cz >> 3) ^ (p % ZCH)) * 16)) + (lane >> 5) * 8);
                }
        };
        if constexpr (E != kEpiNone)
            read_z(0, zr[0]);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if constexpr (E != kEpiNone) {
                if (fm + 1 < FM)
                    read_z(fm + 1, zr[(fm + 1) & 1]);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    float v0 = acc[fn][fm][4 * gq + 0];
                    float v1 = acc[fn][fm][4 * gq + 1];
                    float v2 = acc[fn][fm][4 * gq + 2];
                    float v3 = acc[fn][fm][4 * gq + 3];
                    if constexpr (E != kEpiNone) {
                        const half4_t zz = __builtin_bit_cast(half4_t, zr[fm & 1][fn][gq]);
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
    {BM, BN, 64, WM, WN, #BM "x" #BN "x64/" #WM "x" #WN "w", 3 * (BM + BN) * 64 * 2, false, false, true, false},
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
