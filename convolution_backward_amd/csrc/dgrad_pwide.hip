// A persistent form of dgrad_wide for strided layers whose phases all have
// taps (3x3 stride 2, say): many tiles with short reductions (1-4 taps of a
// phase, 2-8 slices), where what happens between tiles decides the time.
//
// The operation and the operand path are those of dgrad_wide: the
// backward-data convolution of "[CUTLASS] Conv2d dgrad" (apache/tvm PR
// #10110) as an implicit GEMM per stride phase, 64-wide reduction slices
// (taps outermost, then k) carried HBM/L2 -> LDS by 16-byte direct-to-LDS
// loads into a ring of three stages, two slices ahead, four waves of 128
// pixels x 64 channels, v_mfma_f32_32x32x16_f16 with A = filter^T
// (transpose reads) and B = dy^T.
//
// What differs: each workgroup walks tiles slot, slot + G, slot + 2G, ...
// (G workgroups, one per CU), and the stream of slice requests runs on
// across tile (and phase) boundaries, so the first slices of the next tile
// are in LDS when a tile ends. A tile's epilogue (fp32 -> fp16, staged
// through a block of the wave's own past the ring, stored as whole pixel
// rows) runs right after its last slice; the next tile's first slice lets
// those stores stay in flight, its second waits for them. No fused epilogue
// factor and no zero phases: such layers go to dgrad_igemm.
#include "dgrad_internal.h"
#include "kernel_common.h"

namespace cbw {
namespace {

template <int BM, int BN, int WM, int WN>
struct PwideShape {
    static constexpr int NW = WM * WN;
    static constexpr int BK = 64;
    static constexpr int A_BYTES = BM * 2 * BK;
    static constexpr int B_BYTES = BK * BN * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int STG0 = 3 * STAGE;                  // the staging blocks
    static constexpr int EBLK = 32 * (BN / WN) * 2;         // one wave's block
    static constexpr int LDS_USED = STG0 + NW * EBLK;
};

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(1, 1)))
dgrad_pwide(KernelArgs a)
{
    using Sh = PwideShape<BM, BN, WM, WN>;
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
    constexpr int EST = 32 / PPI;                 // stores per pixel group
    constexpr int EPI_STORES = FM * EST;          // GEMM stores of one epilogue (per wave)
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_BYTES % (1024 * NW) == 0 && Sh::B_BYTES % (1024 * NW) == 0, "whole 1 KiB blocks per wave");
    static_assert(BN % 64 == 0, "filter rows of at least 8 chunks");
    static_assert(Sh::LDS_USED <= 160 * 1024, "LDS budget");
    static_assert(CH >= 2 && CH <= 64 && 64 % CH == 0, "whole pixel rows per store");
    static_assert(LD + EPI_STORES < 64, "vmcnt range");

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
    const int SC = pin(a.S * C);          // filter elements per tap row
    const int RSC = pin(a.R * SC);        // filter elements per k
    const int s = pin(a.stride);
    const int ksteps = (K + BK - 1) / BK;
    const int ntiles = pin(a.gemm_tiles);
    const int G = gridDim.x;
    const int slot = xcd_remap(blockIdx.x, G, a.group, a.xcd_mode);
    const int mytiles = pin(slot < ntiles ? (ntiles - 1 - slot) / G + 1 : 0);

    const i32x4 dy_desc = raw_descriptor(a.dy, a.dy_bytes);
    const i32x4 w_desc = raw_descriptor(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t e_dx = make_rsrc(a.dx, a.dx_bytes);

    // local tile u of this workgroup: its phase, first lattice row and channel
    auto decode = [&](int u, int& pi, int& m0, int& c0) __attribute__((always_inline)) {
        const int tile = slot + u * G;
        int local;
        if (a.order == 2) {    // the phases of one pixel block side by side, rotating with the round
            // (every phase has the same tiles and G is a multiple of the phase
            // count, so this is a bijection onto the phase-major numbering)
            const int np = a.nphases;
            const int blk = tile / np;
            const int j = tile - blk * np;
            pi = (j + u) % np;
            local = blk;
        } else {
            pi = 0;
            for (int i = 1; i < a.nphases; ++i)
                if (tile >= a.ph[i].tile_begin)
                    pi = i;
            local = tile - a.ph[pi].tile_begin;
        }
        int tm, tn;
        if (a.order != 1) {    // channel tiles of one pixel block are consecutive
            tm = local / a.tiles_n;
            tn = local - tm * a.tiles_n;
        } else {               // pixel blocks of one channel tile are consecutive
            tn = local / a.ph[pi].tiles_m;
            tm = local - tn * a.ph[pi].tiles_m;
        }
        m0 = tm * BM;
        c0 = tn * BN;
    };

    // ---- request side: a cursor over this workgroup's slices, tile after
    // tile. DMA block b = wave*A_INSTR + jn of a dy slice covers tile rows
    // 8b..8b+7 (a wave's blocks are consecutive, so its lane's rows step by 8
    // from load to load), lane l fills row 8b + l/8 at chunk position l%8,
    // holding logical chunk (l%8) ^ dy_swizzle(row); byte 16*l of block
    // jn*NW + wave of a filter slice is row k, position p, holding logical
    // chunk p ^ w_swizzle(k) (as in dgrad_wide). A lane's dy offset changes
    // only at tap boundaries (2^31 for a padding tap or a dead row), the k
    // step rides in the load's scalar offset.
    int a_k[A_INSTR], b_k[B_INSTR];
    uint32_t a_off[A_INSTR];   // byte offset of dy[n, i, j, chunk*8], modulo 2^32 (exact where loaded)
    int a_i[A_INSTR], a_j[A_INSTR];
    uint32_t dy_vo[A_INSTR];   // the lane's dy byte offset for the current tap
    uint32_t w_vt[B_INSTR];    // the lane's filter byte offset in the tile (2^31: channel past C)
    uint32_t w_vo[B_INSTR];    // ... for the current k step
#pragma unroll
    for (int jn = 0; jn < A_INSTR; ++jn) {
        const int row = (wave * A_INSTR + jn) * 8 + (lane >> 3);
        a_k[jn] = ((lane & 7) ^ dy_swizzle(row)) * 8;
        a_off[jn] = 0;
        a_i[jn] = 0;
        a_j[jn] = 0;
        dy_vo[jn] = 0x80000000u;
    }
#pragma unroll
    for (int jn = 0; jn < B_INSTR; ++jn) {
        const int byte = (jn * NW + wave) * 1024 + 16 * lane;
        b_k[jn] = byte / B_ROW;
        w_vt[jn] = 0x80000000u;
        w_vo[jn] = 0x80000000u;
    }
    int rq_u = 0, rq_k = 0, rq_niter = 0;   // the next item's local tile, its slice in the tile, the tile's slices
    int ar = 0, at = 0, k0 = 0;             // ... its row tap, column tap, k step
    bool new_tap = true;
    int dr0 = 0, dt0 = 0, ntap = 1, wt0 = 0;
    uint32_t q_wtap = 0;                    // filter byte offset of the current tap (wave-uniform)
    uint32_t so_a = 0, so_b = 0;
    const uint32_t dma_base = pin(lds_u32 + (uint32_t)(wave * 1024));              // the wave's first filter block
    const uint32_t dma_base_a = pin(lds_u32 + (uint32_t)(wave * A_INSTR * 1024));  // ... and dy block
    // the cursor enters local tile rq_u: the phase's taps and the lanes' rows
    auto enter_tile = [&]() __attribute__((always_inline)) {
        int pi, m0, c0;
        decode(rq_u, pi, m0, c0);
        const PhaseArg& ph = a.ph[pi];
        m0 = pin(m0);
        c0 = pin(c0);
        rq_niter = pin(ph.nr * ph.nt * ksteps);
        dr0 = pin(ph.dr0);
        dt0 = pin(ph.dt0);
        ntap = pin(ph.nt);
        wt0 = pin(ph.r0 * SC + ph.t0 * C + c0);
        ar = 0;
        at = 0;
        k0 = 0;
        new_tap = true;
        // the lane's rows m, m + 8, ..., lattice coordinates (n, i, j) with
        // m = (n*Hp + i)*Wp + j: the first by division, the next by carries
        // (one at most each when Wp >= 8), offsets in the P x Q grid of dy
        const uint32_t Wp = (uint32_t)ph.Wp;
        const uint32_t Hp = fastdiv(ph.div_hw.d, ph.div_w);
        const bool stepwise = Wp >= 8u;
        const uint32_t d_step = (uint32_t)(8 * K * 2);
        const uint32_t d_row = (uint32_t)(Q * K * 2) - Wp * (uint32_t)(K * 2);
        const uint32_t d_img = (uint32_t)(P * Q * K * 2) - Hp * (uint32_t)(Q * K * 2);
        auto row_at = [&](int jn, uint32_t n, uint32_t i, uint32_t j, uint32_t base) __attribute__((always_inline)) {
            const int m = m0 + (wave * A_INSTR + jn) * 8 + (lane >> 3);
            a_i[jn] = m < ph.M ? (int)i : -(1 << 24);   // a dead row fails every p >= 0 test
            a_j[jn] = (int)j;
            a_off[jn] = base + (uint32_t)a_k[jn] * 2u;   // byte offset of dy[n, i, j, chunk*8], modulo 2^32
        };
        auto divide = [&](int jn, uint32_t& n, uint32_t& i, uint32_t& j, uint32_t& base) __attribute__((always_inline)) {
            const int m = m0 + (wave * A_INSTR + jn) * 8 + (lane >> 3);
            n = fastdiv((uint32_t)m, ph.div_hw);
            const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
            i = fastdiv(rem, ph.div_w);
            j = rem - i * Wp;
            base = (((n * (uint32_t)P + i) * (uint32_t)Q + j) * (uint32_t)K) * 2u;
        };
        if (stepwise) {
            uint32_t n, i, j, base;
            divide(0, n, i, j, base);
            row_at(0, n, i, j, base);
#pragma unroll
            for (int jn = 1; jn < A_INSTR; ++jn) {
                j += 8u;
                base += d_step;
                const bool wrap = j >= Wp;
                j = wrap ? j - Wp : j;
                i = wrap ? i + 1u : i;
                base = wrap ? base + d_row : base;
                const bool next = i >= Hp;
                i = next ? i - Hp : i;
                base = next ? base + d_img : base;
                row_at(jn, n, i, j, base);
            }
        } else {
#pragma unroll
            for (int jn = 0; jn < A_INSTR; ++jn) {
                uint32_t n, i, j, base;
                divide(jn, n, i, j, base);
                row_at(jn, n, i, j, base);
            }
        }
#pragma unroll
        for (int jn = 0; jn < B_INSTR; ++jn) {
            const int byte = (jn * NW + wave) * 1024 + 16 * lane;
            const int pos = (byte % B_ROW) / 16;
            const int cc = (pos ^ w_swizzle<B_ROW>(b_k[jn])) * 8;
            w_vt[jn] = c0 + cc >= C ? 0x80000000u : (uint32_t)(b_k[jn] * RSC + cc) * 2u;
        }
    };
    // the offsets of the next item (past the last slice: every lane out of range)
    auto prepare = [&]() __attribute__((always_inline)) {
        if (rq_u < mytiles) {
            if (rq_k == 0)
                enter_tile();
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
    // load X of the prepared item into the stage at byte offset soff (to the wave's blocks)
    auto issue_one = [&](auto x_c, uint32_t soff) __attribute__((always_inline)) {
        constexpr int X = decltype(x_c)::value;
        if constexpr (X < A_INSTR)
            dma16_at<(uint32_t)(X * 1024)>(dy_desc, dy_vo[X], so_a, dma_base_a + soff);
        else
            dma16_at<(uint32_t)(A_BYTES + (X - A_INSTR) * NW * 1024)>(w_desc, w_vo[X - A_INSTR], so_b, dma_base + soff);
    };
    // past the issued item: k innermost, then column taps, then row taps, then tiles
    auto advance = [&]() __attribute__((always_inline)) {
        k0 += BK;
        if (k0 >= K) {
            k0 = 0;
            new_tap = true;
            if (++at == ntap) {
                at = 0;
                ++ar;
            }
        }
        if (++rq_k == rq_niter) {
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

    // ---- epilogue. Pixel group fm: lattice rows wm*TM + fm*32 .. +31 of the
    // tile, the wave's TN channels. The lane holds channels 8*gq + 4*(lane/32)
    // .. +3 of block fn, row lane%32; it writes them to the wave's staging
    // block (chunk q of row p at position q ^ ((p >> 1) % CH)) and reads back
    // whole chunks: store e of group fm covers rows fm*32 + e*PPI + lane/CH.
    // The block belongs to the wave alone, so no barrier guards it.
    //
    // The lane's rows step by PPI from store to store. Its dx pixel is
    // (n*H + ph + s*i)*W + pw + s*j for lattice row m = (n*Hp + i)*Wp + j:
    // the first row is decomposed by division, the next ones follow by adding
    // PPI to j and carrying into i and n (one carry at most each when
    // Wp >= PPI; narrower lattices divide every row), so that each store's
    // offset costs adds and selects instead of integer multiplies.
    lds_char* blk = (lds_char*)lds + Sh::STG0 + wave * EBLK;
    float16_t acc[FN][FM];
    auto epilogue = [&](int pi, int m0, int c0) __attribute__((always_inline)) {
        const PhaseArg& ph = a.ph[pi];
        const int cw = c0 + wn * TN;          // first channel of this wave's block
        const int pw = lane & 31;
        const int Mp = ph.M;
        const uint32_t Wp = (uint32_t)ph.Wp;
        const uint32_t Hp = fastdiv(ph.div_hw.d, ph.div_w);
        const bool stepwise = Wp >= (uint32_t)PPI;
        // element-offset steps (multiples of C): PPI along j, a wrap into the
        // next lattice row, a wrap into the next image
        const uint32_t d_step = (uint32_t)(s * PPI * C);
        const uint32_t d_row = (uint32_t)(s * a.W * C) - (uint32_t)(s * C) * Wp;
        const uint32_t d_img = (uint32_t)(a.H * a.W * C) - (uint32_t)(s * a.W * C) * Hp;
        const int mlane = m0 + wm * TM + lane / CH;   // the lane's row in store 0 of group 0
        const int c = cw + (lane % CH) * 8;
        constexpr int NR = FM * EST;                  // rows of the lane, PPI apart
        uint32_t rowoff[NR];                          // their pixel * C
        auto divide = [&](int r) __attribute__((always_inline)) -> uint32_t {
            const uint32_t m = (uint32_t)(mlane + r * PPI);
            const uint32_t n = fastdiv(m, ph.div_hw);
            const uint32_t rem = m - n * ph.div_hw.d;
            const uint32_t i = fastdiv(rem, ph.div_w);
            const uint32_t j = rem - i * Wp;
            return ((n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)i)) * (uint32_t)a.W + (uint32_t)(ph.pw + s * (int)j)) *
                   (uint32_t)C;
        };
        if (stepwise) {
            const uint32_t m = (uint32_t)mlane;
            const uint32_t n = fastdiv(m, ph.div_hw);
            const uint32_t rem = m - n * ph.div_hw.d;
            uint32_t ii = fastdiv(rem, ph.div_w);
            uint32_t ji = rem - ii * Wp;
            uint32_t pix_c = ((n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)ii)) * (uint32_t)a.W + (uint32_t)(ph.pw + s * (int)ji)) *
                             (uint32_t)C;
            rowoff[0] = pix_c;
#pragma unroll
            for (int r = 1; r < NR; ++r) {
                ji += (uint32_t)PPI;
                pix_c += d_step;
                const bool wrap = ji >= Wp;
                ji = wrap ? ji - Wp : ji;
                ii = wrap ? ii + 1u : ii;
                pix_c = wrap ? pix_c + d_row : pix_c;
                const bool next = ii >= Hp;
                ii = next ? ii - Hp : ii;
                pix_c = next ? pix_c + d_img : pix_c;
                rowoff[r] = pix_c;
            }
        } else {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                rowoff[r] = divide(r);
        }
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
                const int m = mlane + (fm * EST + e) * PPI;
                const uint32_t bad = (uint32_t)(m >= Mp) | (uint32_t)(c >= C);
                const uint32_t off = (rowoff[fm * EST + e] + (uint32_t)c) * 2u;
                __builtin_amdgcn_raw_buffer_store_b128(v, e_dx, out_of_range_if(bad, off), 0, kStoreNT);
            }
        }
    };

    // ---- the slices. Slice it of the walk lives in stage it % 3 (a run-time
    // index: its LDS base is a scalar). Sub-steps 0 and 2 run on fragment set
    // 0, 1 and 3 on set 1; the barrier sits after sub-step 2's operations,
    // then the next slice's first fragments are read under sub-step 3. The LD
    // loads of item it + 2 go out between the operations of sub-steps 0-2.
    // The wait lets those loads stay in flight, and in a tile's first slice
    // after an epilogue also that epilogue's stores: they were issued after
    // the loads of this slice's successor, which it waits for.
    constexpr int OPS = FM * FN;
    half8_t af[2][FN], bf[2][FM];
    int st = 0;                   // stage of the slice in hand
    auto slice = [&](auto first_c, bool after_epi, bool has_next) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first_c)::value;    // the tile's first slice: the sums start from zero
        const uint32_t sb = (uint32_t)(st * STAGE);
        const int rst = st == 0 ? 2 : st - 1;               // stage of item it + 2
        const uint32_t rbase = pin((uint32_t)(rst * STAGE));
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
        if (has_next) {
            if (FIRST && after_epi)
                wait_vmcnt<LD + EPI_STORES>();
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

    // ---- prologue: items 0 and 1 (item 1 may already be past the last slice)
    prepare();
    static_for<0, LD>([&](auto x_c) { issue_one(x_c, 0u); });
    advance();
    prepare();
    static_for<0, LD>([&](auto x_c) { issue_one(x_c, (uint32_t)STAGE); });
    advance();
    wait_vmcnt<LD>();
    __syncthreads();
    read_frags(0u, IC<0>{}, af[0], bf[0]);
    read_frags(0u, IC<1>{}, af[1], bf[1]);
    for (int u = 0; u < mytiles; ++u) {
        int pi, m0, c0;
        decode(u, pi, m0, c0);
        pi = pin(pi);
        m0 = pin(m0);
        c0 = pin(c0);
        const int niter = pin(a.ph[pi].nr * a.ph[pi].nt * ksteps);
        const bool last_tile = u + 1 == mytiles;
        slice(IC<true>{}, u > 0, niter > 1 || !last_tile);
        for (int k = 1; k < niter; ++k)
            slice(IC<false>{}, false, k + 1 < niter || !last_tile);
        epilogue(pi, m0, c0);
    }
    wait_vmcnt<0>();   // the loads past the last slice have written LDS before the workgroup ends
}

// The layers this kernel runs: stride at least 2 (so several phases share a
// launch), a filter at least as wide and tall as the stride (so every phase
// has taps: phase p's taps are those r = p + pad mod s, one exists for every
// p when R >= s), no fused epilogue factor.
bool pwide_fits(int R, int S, int stride, int epi) { return stride >= 2 && R >= stride && S >= stride && epi == kEpiNone; }

// The launches this kernel runs: GEMM tiles only (no zero phase: those go to
// dgrad_igemm), no split, the grid no larger than the tiles; the
// phase-interleaved order only with a grid that is a multiple of the phases.
bool pwide_runs(const KernelArgs& a)
{
    return !a.sk && a.nzphases == 0 && a.zstripes == 0 && a.ncomp == 0 && a.total_tiles == a.gemm_tiles &&
           pwide_fits(a.R, a.S, a.stride, a.epi) && a.grid >= 1 && a.grid <= a.gemm_tiles &&
           (a.order != 2 || a.grid % a.nphases == 0);
}

template <int BM, int BN, int WM, int WN>
hipError_t pwide_launch(const KernelArgs& a, hipStream_t stream)
{
    if (!pwide_runs(a))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((dgrad_pwide<BM, BN, WM, WN>), dim3(a.grid), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
int pwide_resident(void)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(dgrad_pwide<BM, BN, WM, WN>),
                                                     64 * WM * WN, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    return n > 0 ? n : 1;
}

template <int BM, int BN, int WM, int WN>
int pwide_private(void)
{
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(dgrad_pwide<BM, BN, WM, WN>)) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return (int)attr.localSizeBytes;
}

// The compiled configurations of this kernel: (BM, BN, WM, WN).
#define CBW_PWIDE_CONFIGS(X) \
    X(256, 128, 2, 2)

#define CBW_PWIDE_ENTRY(BM, BN, WM, WN) \
    {BM, BN, 64, WM, WN, #BM "x" #BN "x64/" #WM "x" #WN "q", PwideShape<BM, BN, WM, WN>::LDS_USED, false, true, false, true},
const TileConfig kPwideConfigs[] = {CBW_PWIDE_CONFIGS(CBW_PWIDE_ENTRY)};
constexpr int kNumPwide = sizeof(kPwideConfigs) / sizeof(kPwideConfigs[0]);

using PwideLaunchFn = hipError_t (*)(const KernelArgs&, hipStream_t);
#define CBW_PWIDE_LAUNCH(BM, BN, WM, WN) &pwide_launch<BM, BN, WM, WN>,
#define CBW_PWIDE_RESIDENT(BM, BN, WM, WN) &pwide_resident<BM, BN, WM, WN>,
#define CBW_PWIDE_PRIVATE(BM, BN, WM, WN) &pwide_private<BM, BN, WM, WN>,
const PwideLaunchFn kPwideLaunch[] = {CBW_PWIDE_CONFIGS(CBW_PWIDE_LAUNCH)};
int (*const kPwideResident[])(void) = {CBW_PWIDE_CONFIGS(CBW_PWIDE_RESIDENT)};
int (*const kPwidePrivate[])(void) = {CBW_PWIDE_CONFIGS(CBW_PWIDE_PRIVATE)};

}  // namespace

int pwide_num_configs() { return kNumPwide; }

const TileConfig& pwide_config(int i) { return kPwideConfigs[i]; }

bool pwide_admits(int i, int R, int S, int stride, int epi) { return i >= 0 && i < kNumPwide && pwide_fits(R, S, stride, epi); }

bool pwide_runs_launch(int i, const KernelArgs& a) { return i >= 0 && i < kNumPwide && pwide_runs(a); }

hipError_t launch_pwide(int i, const KernelArgs& a, hipStream_t stream)
{
    if (i < 0 || i >= kNumPwide)
        return hipErrorInvalidValue;
    return kPwideLaunch[i](a, stream);
}

int pwide_blocks_per_cu(int i) { return (i >= 0 && i < kNumPwide) ? kPwideResident[i]() : 1; }

int pwide_private_bytes(int i) { return (i >= 0 && i < kNumPwide) ? kPwidePrivate[i]() : -1; }

}  // namespace cbw
