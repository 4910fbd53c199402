// A third dgrad kernel, for 3x3 stride-1 layers whose dx and dy images have
// the same extent (pad 1, P = H, Q = W): per 64-wide k chunk, the dy rows a
// tile needs for all nine taps are loaded into LDS once, with the halo the
// taps reach, and every tap reads its shifted rows from there.
//
// The operation is that of dgrad_igemm and dgrad_wide (the backward-data
// convolution of "[CUTLASS] Conv2d dgrad", apache/tvm PR #10110, as an
// implicit GEMM). With stride 1, pad 1 and P = H, Q = W, output pixel m
// (linear in n, h, w) takes tap (r, t) from dy pixel m + d, with the constant
// shift d = (1 - r) * W + (1 - t), when the shifted row and column stay
// inside the image. So the BM pixels of a tile read, per k chunk and for all
// nine taps, only the dy pixels [m0 - D, m0 + BM + D) with D = W + 1, where
// dgrad_wide loads BM rows per tap. With a 256 x 128 tile that cuts what a
// slice brings into LDS from 48 KiB to about 20 KiB.
//
// Layout and walk (one tile per workgroup, four waves of 128 x 64 as in
// dgrad_wide):
//   * LDS: a ring of three filter stages (64 k rows x BN channels, as in
//     dgrad_wide), then two halo buffers, each after 512 bytes of zeros. A
//     halo row is one dy pixel's 64-wide k chunk in eight 16-byte units plus
//     one unused unit (144 bytes), so row x starts 9x units into its buffer:
//     16 consecutive rows start in 16 distinct 16-byte bank groups of the
//     256-byte bank window, whatever the first row, and a fragment read
//     needs no per-lane permutation. One 16-byte load per lane fills 63 units
//     (seven rows) and one more that the next load fills with the same bytes.
//   * Chunks run one after the other, the nine taps of a chunk as nine
//     slices, unrolled: tap, filter stage and halo buffer of every slice are
//     compile-time constants (nine slices per chunk keep the stage of tap t
//     at t mod 3), so the loop carries almost no scalar work.
//   * Each slice issues one filter slice, two ahead; the first seven slices
//     of a chunk also issue two halo loads per wave of the next chunk's halo
//     (fourteen per wave: 392 rows, the most a buffer holds), into the buffer
//     the previous chunk used; loads past the halo load nothing. In the last
//     chunk those loads, and the filter loads of its tap 7, bring the fused
//     epilogue's z tile into LDS instead.
//   * Fragments: the filter^T operand as in dgrad_wide (transpose reads);
//     the dy^T fragment of tile pixel p for tap (r, t) is halo row p + D + d,
//     or, where the tap leaves the image, the zero block at the same offset
//     within a 256-byte bank window (so those lanes keep the bank pattern).
//     Both are formed once per lane for all nine taps; buffer, sub-step and
//     the second buffer's distance are immediate offsets of the reads.
//   * The epilogue is dgrad_wide's.
#include "dgrad_internal.h"
#include "kernel_common.h"

namespace cbw {
namespace {

template <int BM, int BN, int WM, int WN>
struct HaloShape {
    static constexpr int NW = WM * WN;
    static constexpr int FSTAGE = 64 * BN * 2;    // one filter slice (bytes)
    static constexpr int LDS = 160 * 1024;
    static constexpr int TAPS = 9;
    static constexpr int ROW = 9 * 16;            // bytes per halo row
    static constexpr int RPL = 7 * NW;            // halo rows one load of every wave fills
    static constexpr int HPS = 2;                 // halo loads per wave in each of the first HSL slices of a chunk
    static constexpr int HSL = TAPS - 2;
    static constexpr int HL = HPS * HSL;          // halo loads per wave per chunk
    static constexpr int HR = HL * RPL;           // halo rows a buffer holds
    static constexpr int HBUF = (HR + 1) * ROW;   // and the row the last load's last lane writes
    static constexpr int ZREG = 512;              // zeros before each buffer
    static constexpr int Z0 = 3 * FSTAGE;
    static constexpr int B0 = Z0 + ZREG;
    static constexpr int XB = ZREG + HBUF;        // the second buffer and its zeros lie XB further
    static constexpr int LDS_USED = B0 + XB + HBUF;
};

// Halo rows of one chunk for shift bound D: the tile and D on each side,
// rounded up to whole loads.
__host__ __device__ constexpr int halo_rows(int BM, int rows_per_load, int D)
{
    return (BM + 2 * D + rows_per_load - 1) / rows_per_load * rows_per_load;
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(1, 1)))
dgrad_halo(KernelArgs a)
{
    using Sh = HaloShape<BM, BN, WM, WN>;
    constexpr int BK = 64;
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int B_ROW = BN * 2;                 // one k row of a filter slice
    constexpr int FSTAGE = Sh::FSTAGE;
    constexpr int B_INSTR = FSTAGE / 1024 / NW;   // filter loads per wave per slice
    constexpr int TAPS = Sh::TAPS, HPS = Sh::HPS, HSL = Sh::HSL;
    constexpr int ROW = Sh::ROW, RPL = Sh::RPL;
    constexpr int Z0 = Sh::Z0, B0 = Sh::B0, XB = Sh::XB;
    constexpr int HB_MIN = (BM + 2 + RPL - 1) / RPL;   // halo loads of the narrowest halo (D = 2)
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(FSTAGE % (1024 * NW) == 0, "whole 1 KiB blocks per wave");
    static_assert(BN % 64 == 0, "filter rows of at least 8 chunks");
    static_assert(NW * 32 * TN * 2 <= FSTAGE, "the output staging fits one filter stage");
    static_assert(Sh::LDS_USED <= Sh::LDS, "LDS budget");
    static_assert(Z0 % 256 == 0 && Sh::ZREG >= 256 + 3 * 32 + 16, "zeros: a bank window and the sub-step offsets");
    static_assert(XB + 3 * 32 < 65536, "the second buffer within a read's immediate offset");
    static_assert(TAPS % 3 == 0, "the filter stage of tap t is t mod 3 in every chunk");
    static_assert(HPS + B_INSTR + HPS < 64, "vmcnt range");

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
    const int RSC = pin(a.R * a.S * C);   // filter elements per k
    const int last = pin((K + BK - 1) / BK - 1);
    const bool ragged = K % BK != 0;

    // ---- this workgroup's tile (one phase; the grid is the tile count)
    const int tile = xcd_remap(blockIdx.x, gridDim.x, a.group, a.xcd_mode);
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
    const int D = pin(Q + 1);                                 // the halo: buffer row x holds dy pixel m0 - D + x
    const int HB = pin(halo_rows(BM, RPL, D) / RPL);          // halo loads per wave that carry rows

    const i32x4 dy_desc = raw_descriptor(a.dy, a.dy_bytes);
    const i32x4 w_desc = raw_descriptor(a.w, a.w_bytes);

    // ---- halo loads. Load j of wave v fills block b = j*NW + v: units
    // 63b .. 63b + 63 of the buffer, lane l unit 63b + l = row 7b + l/9,
    // unit l%9 (lane 63 writes the first unit of row 7b + 7, which block
    // b + 1 writes with the same bytes). The lane's dy pixel is
    // m0 - D + 7*NW*j + 7v + l/9, its k offset 8*(l%9) into the chunk (the
    // chunk in the scalar offset). A row whose pixel lies outside the image
    // holds whatever the range check gives: only taps that leave the image
    // would read it, and they read zeros instead. Lanes that load nothing:
    // the unused unit of a row, the units past K in the last chunk of a
    // ragged K, and every lane of a load past the halo or of the last chunk.
    const int hq = lane / 9;
    const int hr = lane - 9 * hq;
    const uint32_t hoff0 = (uint32_t)(m0 - D + 7 * wave + hq) * (uint32_t)(2 * K) + (uint32_t)(16 * hr);
    const bool h_skip = hr == 8;
    const bool h_skip_last = h_skip || last * BK + 8 * hr >= K;
    const uint32_t VSTEP = pin((uint32_t)(RPL * 2 * K));    // dy bytes between a wave's consecutive loads
    const uint32_t h_wave = pin(lds_u32 + (uint32_t)(B0 + wave * 63 * 16));
    // halo load j of chunk kn (into buffer BUF = (last - kn) & 1, compile-time)
    auto issue_halo = [&](auto buf_c, auto j_c, int kn) __attribute__((always_inline)) {
        constexpr int BUF = decltype(buf_c)::value;
        constexpr int J = decltype(j_c)::value;
        bool live = true;
        if constexpr (J >= HB_MIN)
            live = J < HB;
        const bool skip = !live || (ragged && kn == last ? h_skip_last : h_skip);
        const uint32_t vo = hoff0 + (uint32_t)J * VSTEP;
        dma16_at<(uint32_t)(BUF * XB + J * NW * 63 * 16)>(dy_desc, skip ? 0x80000000u : vo,
                                                           pin((uint32_t)(kn * BK * 2)), h_wave);
    };

    // ---- filter slices: item i = chunk i / 9, tap i % 9, at byte offset
    // 2*(c0 + tap*C + 64*chunk*9*C) (tap (r, t) = 3r + t lies 3rC + tC
    // elements in). Byte 16*l of block jn*NW + v of a stage is row k,
    // position p, holding logical chunk p ^ w_swizzle(k); in the last chunk
    // of a ragged K the rows past K load zeros. Items past the end load the
    // last item again (into stages no slice reads).
    uint32_t w_vt[B_INSTR], w_vl[B_INSTR], w_vo[B_INSTR];
#pragma unroll
    for (int jn = 0; jn < B_INSTR; ++jn) {
        const int byte = (jn * NW + wave) * 1024 + 16 * lane;
        const int k = byte / B_ROW;
        const int pos = (byte % B_ROW) / 16;
        const int cc = (pos ^ w_swizzle<B_ROW>(k)) * 8;
        w_vt[jn] = c0 + cc >= C ? 0x80000000u : (uint32_t)(k * RSC + cc) * 2u;
        w_vl[jn] = last * BK + k >= K ? 0x80000000u : w_vt[jn];
        w_vo[jn] = last == 0 ? w_vl[jn] : w_vt[jn];
    }
    const uint32_t WTAP = pin((uint32_t)(2 * C));                        // the next tap
    const uint32_t WCHUNK = pin((uint32_t)(2 * (BK * RSC - TAPS * C)));  // the next chunk's first tap, after a WTAP step
    uint32_t so_w = pin((uint32_t)(2 * c0));                             // the offset of the item to issue next
    const uint32_t dma_base = pin(lds_u32 + (uint32_t)(wave * 1024));
    auto issue_filter = [&](auto st_c, auto x_c) __attribute__((always_inline)) {
        constexpr int ST = decltype(st_c)::value;
        constexpr int X = decltype(x_c)::value;
        dma16_at<(uint32_t)(ST * FSTAGE + X * NW * 1024)>(w_desc, w_vo[X], so_w, dma_base);
    };

    // ---- fragment rows. dy^T (B): tile pixel p = wm*TM + fm*32 + lane%32 at
    // k chunk 2*kk + lane/32 is halo row p + D + d for tap shift d, at byte
    // 144*(p + D + d) + 16*(2*kk + lane/32) of its buffer; b_off holds it for
    // the first buffer (or the zero block's byte at the same bank offset),
    // formed once the prologue's loads are out.
    uint32_t b_off[TAPS][FM];
    // filter^T (A), as in dgrad_wide: group g = lane/16 covers channels
    // +16*(g&1), k +8*(g>>1); within it lane 4r+q reads row r, channels 4q..4q+3.
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

    float16_t acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[fn][fm][e] = 0.0f;
    // fragments of sub-step KK of tap T: the filter from stage ST, dy rows
    // from halo buffer BUF
    auto read_frags = [&](auto st_c, auto t_c, auto buf_c, auto kk_c, half8_t (&af)[FN], half8_t (&bf)[FM])
        __attribute__((always_inline)) {
        constexpr int SB = decltype(st_c)::value * FSTAGE;
        constexpr int T = decltype(t_c)::value;
        constexpr int BUF = decltype(buf_c)::value;
        constexpr int KK = decltype(kk_c)::value;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const lds_char* p = (lds_char*)lds + SB + a_frag[fn] + KK * 16 * B_ROW;
            const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)p);
            const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p + 4 * B_ROW));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
            af[fn] = __builtin_bit_cast(half8_t, u32x4{l2.x, l2.y, h2.x, h2.y});
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            bf[fm] = __builtin_bit_cast(half8_t, *(const __attribute__((address_space(3))) u32x4*)(
                                                     (lds_char*)lds + b_off[T][fm] + (BUF * XB + KK * 32)));
    };

    // ---- the fused epilogue's z tile (BM pixels x BN channels), loaded into
    // LDS during the last chunk by the loads that would otherwise carry no
    // work: its halo loads put z blocks 0 .. ZH - 1 into the halo buffer no
    // slice reads any more, the filter loads of its tap 7 put blocks
    // ZH .. ZB - 1 into filter stage 0. A 1 KiB block holds z rows 4b .. 4b + 3
    // (256 bytes each), row p's 16-byte chunk c at position c ^ (p % 16).
    constexpr int ZROW = BN * 2;
    constexpr int ZCH = ZROW / 16;                    // chunks per z row
    constexpr int ZRPB = 1024 / ZROW;                 // z rows per block
    constexpr int ZB = BM / ZRPB;                     // z blocks
    constexpr int ZHL = Sh::HBUF / 1024 / NW;         // halo loads per wave that carry z blocks
    constexpr int ZH = ZHL * NW;                      // z blocks in the halo buffer
    constexpr int ZF = (ZB - ZH + NW - 1) / NW;       // filter loads per wave that carry z blocks
    static_assert(ZROW <= 1024 && 1024 % ZROW == 0 && 64 % ZCH == 0 && ZCH == 16, "whole z rows per block");
    static_assert(ZHL <= Sh::HL && ZF <= B_INSTR && ZH + ZF * NW >= ZB, "the z tile fits the free loads");
    static_assert(ZH * 1024 + 1024 <= Sh::HBUF, "a block for the loads with no work past the z blocks");
    const bool zpre = a.epi != kEpiNone;
    const i32x4 z_desc = raw_descriptor(zpre ? a.z : a.dx, a.dx_bytes);
    const int s = pin(a.stride);
    auto pixel_offset = [&](int m) __attribute__((always_inline)) -> uint32_t {   // dx element offset of pixel m
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        const uint32_t pix = (n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)i)) * (uint32_t)a.W
                             + (uint32_t)(ph.pw + s * (int)j);
        return pix * (uint32_t)C;
    };
    // this lane's byte offset in z for block b (2^31: nothing to load)
    auto z_voff = [&](int b) __attribute__((always_inline)) -> uint32_t {
        int ln = lane;
        asm volatile("" : "+v"(ln));      // formed here, in the last chunk, not hoisted to live through the walk
        const int row = b * ZRPB + ln / ZCH;
        const int c = ((ln % ZCH) ^ (row % ZCH)) * 8;
        const int m = m0 + row;
        const uint32_t bad = (uint32_t)!zpre | (uint32_t)(b >= ZB) | (uint32_t)(m >= M) | (uint32_t)(c0 + c >= C);
        return out_of_range_if(bad, bad ? 0u : (pixel_offset(m) + (uint32_t)(c0 + c)) * 2u);
    };
    const uint32_t z_wave = pin(lds_u32 + (uint32_t)(B0 + wave * 1024));
    // the last chunk's halo load J: z block J*NW + v into buffer BUF (past
    // the z blocks: nothing, into one block every wave shares)
    auto issue_zhalo = [&](auto buf_c, auto j_c) __attribute__((always_inline)) {
        constexpr int BUF = decltype(buf_c)::value;
        constexpr int J = decltype(j_c)::value;
        if constexpr (J < ZHL)
            dma16_at<(uint32_t)(BUF * XB + J * NW * 1024)>(z_desc, z_voff(J * NW + wave), 0u, z_wave);
        else
            dma16(dy_desc, 0x80000000u, 0u, lds_u32 + (uint32_t)(B0 + BUF * XB + ZH * 1024));
    };

    // ---- the slices, as in dgrad_wide: one barrier in the middle of a
    // slice (after sub-step 2's operations are issued, the wave waits for
    // the loads it needs, and for its fragment reads), then the next slice's
    // first fragments are read under sub-step 3.
    //
    // Loads, in issue order per slice: filter item it + 2 (B_INSTR loads, in
    // sub-steps 0 and 1), then, in the first HSL slices of a chunk, HPS halo
    // loads (sub-step 2). The wait lets this slice's loads and the previous
    // slice's halo loads stay in flight: so it covers filter item it + 1, and
    // at the last slice of a chunk the whole halo of the next chunk.
    // Who may overwrite what: the halo of chunk kc + 1 goes into the buffer
    // chunk kc - 1 read, from the first slice of chunk kc on; every read of
    // chunk kc - 1 ended before the barrier of its last slice. Filter item
    // it + 2 goes into the stage of slice it - 1, whose reads ended before
    // slice it - 1's barrier.
    constexpr int OPS = FM * FN;          // operations per sub-step
    static_assert(OPS >= 2 * B_INSTR && OPS >= 2 * HPS, "issue slots");
    half8_t af[2][FN], bf[2][FM];
    auto ops = [&](auto kk_c, int f, auto issue) __attribute__((always_inline)) {
        static_for<0, OPS>([&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            constexpr int fm = J / FN, fn = J % FN;
            acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[f][fn], bf[f][fm], acc[fn][fm], 0, 0, 0);
            issue(j_c);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // slice of tap T of chunk kc (halo buffer PAR = (last - kc) & 1; LAST: the last chunk)
    auto slice = [&](auto par_c, auto t_c, auto last_c, int kc) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_c)::value;
        constexpr int T = decltype(t_c)::value;
        constexpr bool LAST = decltype(last_c)::value;
        constexpr IC<T % 3> st_c{};
        constexpr IC<(T + 1) % 3> next_c{};
        constexpr IC<(T + 2) % 3> req_c{};
        constexpr IC<(T + 1) % TAPS> nt_c{};
        constexpr IC<T + 1 == TAPS ? 1 - PAR : PAR> nbuf_c{};
        constexpr int HN = T < HSL ? HPS : 0;                         // halo loads of this slice
        constexpr int HPREV = (T == 0 ? TAPS - 1 : T - 1) < HSL ? HPS : 0;
        constexpr IC<1 - PAR> hbuf_c{};
        auto no_issue = [](auto) {};
        // filter load X of this slice: item it + 2, or, in the last chunk,
        // z blocks (tap 7) or nothing (tap 8: no item left)
        auto filter_slot = [&](auto x_c) __attribute__((always_inline)) {
            constexpr int X = decltype(x_c)::value;
            if constexpr (!LAST || T + 2 < TAPS)
                issue_filter(req_c, x_c);
            else if constexpr (T + 2 == TAPS && X < ZF)
                dma16_at<(uint32_t)(((T + 2) % 3) * FSTAGE + X * NW * 1024)>(z_desc, z_voff(ZH + X * NW + wave), 0u,
                                                                            dma_base);
            else
                dma16_at<(uint32_t)(((T + 2) % 3) * FSTAGE + X * NW * 1024)>(dy_desc, 0x80000000u, 0u, dma_base);
        };
        ops(IC<0>{}, 0, [&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            static_for<0, B_INSTR>([&](auto x_c) {
                if constexpr (decltype(x_c)::value * 2 * OPS / B_INSTR == J)
                    filter_slot(x_c);
            });
        });
        read_frags(st_c, t_c, par_c, IC<2>{}, af[0], bf[0]);
        ops(IC<1>{}, 1, [&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            static_for<0, B_INSTR>([&](auto x_c) {
                if constexpr (decltype(x_c)::value * 2 * OPS / B_INSTR == OPS + J)
                    filter_slot(x_c);
            });
        });
        read_frags(st_c, t_c, par_c, IC<3>{}, af[1], bf[1]);
        ops(IC<2>{}, 0, [&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            if constexpr (HN > 0) {
                static_for<0, HN>([&](auto h_c) {
                    if constexpr (decltype(h_c)::value * OPS / HN == J) {
                        constexpr IC<HPS * T + decltype(h_c)::value> hj_c{};
                        if constexpr (LAST)
                            issue_zhalo(hbuf_c, hj_c);
                        else
                            issue_halo(hbuf_c, hj_c, kc + 1);
                    }
                });
            }
        });
        constexpr bool has_next = !LAST || T + 1 < TAPS;
        if constexpr (has_next) {
            wait_vmcnt<HPREV + B_INSTR + HN>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
            read_frags(next_c, nt_c, nbuf_c, IC<0>{}, af[0], bf[0]);
        }
        ops(IC<3>{}, 1, no_issue);
        if constexpr (has_next)
            read_frags(next_c, nt_c, nbuf_c, IC<1>{}, af[1], bf[1]);
        // the next filter item: tap T + 3 of this chunk, or of the next
        if constexpr (T + 3 < TAPS) {
            so_w += WTAP;
        } else if constexpr (!LAST) {
            so_w += WTAP;
            if constexpr (T + 3 == TAPS) {
                so_w += WCHUNK;
                // (a select, not a branch: a branch here lets the compiler
                // split the loop, and the copies no longer fit the registers)
                const bool to_last = kc + 1 == last;
#pragma unroll
                for (int jn = 0; jn < B_INSTR; ++jn)
                    w_vo[jn] = to_last ? w_vl[jn] : w_vo[jn];
            }
        }
    };
    auto chunk = [&](auto par_c, auto last_c, int kc) __attribute__((always_inline)) {
        static_for<0, TAPS>([&](auto t_c) { slice(par_c, t_c, last_c, kc); });
    };

    // ---- prologue: the zeros (ds writes), the halo of chunk 0, filter
    // items 0 and 1
    if (wave == 0) {
        const int zb = lane < 32 ? Z0 + lane * 16 : Z0 + XB + (lane - 32) * 16;
        *(__attribute__((address_space(3))) u32x4*)((lds_char*)lds + zb) = u32x4{0u, 0u, 0u, 0u};
    }
    if (last & 1)
        static_for<0, Sh::HL>([&](auto j_c) { issue_halo(IC<1>{}, j_c, 0); });
    else
        static_for<0, Sh::HL>([&](auto j_c) { issue_halo(IC<0>{}, j_c, 0); });
    static_for<0, B_INSTR>([&](auto x_c) { issue_filter(IC<0>{}, x_c); });
    so_w += WTAP;
    static_for<0, B_INSTR>([&](auto x_c) { issue_filter(IC<1>{}, x_c); });
    so_w += WTAP;
    // the fragment rows, while those loads are in flight: tap (r, t) = 3r + t
    // stays inside for the pixel at (i, j) when row i + 1 - r and column
    // j + 1 - t do
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
    wait_vmcnt<B_INSTR>();                // all but filter item 1
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    if (last & 1) {
        read_frags(IC<0>{}, IC<0>{}, IC<1>{}, IC<0>{}, af[0], bf[0]);
        read_frags(IC<0>{}, IC<0>{}, IC<1>{}, IC<1>{}, af[1], bf[1]);
    } else {
        read_frags(IC<0>{}, IC<0>{}, IC<0>{}, IC<0>{}, af[0], bf[0]);
        read_frags(IC<0>{}, IC<0>{}, IC<0>{}, IC<1>{}, af[1], bf[1]);
    }
    // two chunks per pass, so every halo buffer index is a compile-time
    // constant (one exit, so the accumulators keep their registers); the
    // last chunk on its own (no next chunk: its halo loads carry z)
    // Chunk kc reads halo buffer (last - kc) & 1, so the last chunk reads the
    // first one and is compiled on its own (its halo loads carry z). The
    // chunks before it run in pairs (second buffer, then first), after one
    // chunk alone when their count is odd; every buffer index is a
    // compile-time constant, and the accumulators keep their registers.
    int kc = 0;
    if (last & 1) {
        chunk(IC<1>{}, IC<false>{}, 0);
        kc = 1;
    }
    for (; kc < last; kc += 2) {
        chunk(IC<0>{}, IC<false>{}, kc);
        chunk(IC<1>{}, IC<false>{}, kc + 1);
    }
    chunk(IC<0>{}, IC<true>{}, last);

    // ---- epilogue: acc x g(z) -> fp16 (RNE), staged through the filter
    // stage of the last slice (tap 8: stage 2) and stored as whole pixel rows
    // (as in dgrad_wide).
    constexpr int SDONE = (TAPS - 1) % 3;
    constexpr int CH = TN / 8;            // 16-byte chunks per staged pixel row
    constexpr int EROW = TN * 2;          // bytes per staged pixel row
    constexpr int EBLK = 32 * EROW;       // bytes per wave per pixel group
    constexpr int PPI = 64 / CH;          // pixels per store instruction
    constexpr int EST = 32 / PPI;         // store instructions per pixel group
    static_assert(CH >= 2 && CH <= 64 && 64 % CH == 0, "whole pixel rows per store");
    auto epilogue = [&](auto tag) __attribute__((always_inline)) {
        constexpr int E = decltype(tag)::value;
        const __amdgpu_buffer_rsrc_t e_dx = make_rsrc(a.dx, a.dx_bytes);
        const int cw = c0 + wn * TN;      // first channel of this wave's block
        const int pw = lane & 31;
        lds_char* blk = (lds_char*)lds + SDONE * FSTAGE + wave * EBLK;
        wait_vmcnt<0>();   // this wave's z blocks are in LDS (and no load writes LDS after the end)
        __syncthreads();   // every wave is done reading the stage's operands, and the z tile is whole
        constexpr int zbuf = B0 + XB;   // the halo buffer the last chunk filled with z
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            // the lane's z: pixel pw of group fm, channels 8*gq + 4*(lane/32) .. +3 of block fn
            u32x2 zr[FN][4];
            if constexpr (E != kEpiNone) {
                const int p = wm * TM + fm * 32 + pw;
                const int b = p / ZRPB;
                const int rowb = (b < ZH ? zbuf + b * 1024 : (b - ZH) * 1024) + (p % ZRPB) * ZROW;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int cz = (wn * TN + fn * 32 + 8 * gq) >> 3;
                        zr[fn][gq] = *(const __attribute__((address_space(3))) u32x2*)(
                            (lds_char*)lds + rowb + ((cz ^ (p % ZCH)) * 16) + (lane >> 5) * 8);
                    }
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
                        const half4_t zz = __builtin_bit_cast(half4_t, zr[fn][gq]);
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
                const uint32_t bad = (uint32_t)(m >= M) | (uint32_t)(c >= C);
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

// The layers this kernel runs: 3x3, stride 1, pad 1, P = H and Q = W (so the
// tap shifts are constant along the linear pixel index), and a halo of at
// most the rows a buffer holds.
template <int BM, int BN, int WM, int WN>
bool halo_fits(int R, int S, int stride, int pad, int H, int W, int P, int Q)
{
    using Sh = HaloShape<BM, BN, WM, WN>;
    if (stride != 1 || R != 3 || S != 3 || pad != 1 || P != H || Q != W || Q > Sh::HR)
        return false;
    return halo_rows(BM, Sh::RPL, Q + 1) <= Sh::HR;
}

// The launch must be that one phase (taps from (0, 0), dy offsets of the
// first tap = 1) in GEMM tiles only, one per workgroup.
template <int BM, int BN, int WM, int WN>
hipError_t halo_launch(const KernelArgs& a, hipStream_t stream)
{
    const PhaseArg& ph = a.ph[0];
    if (a.sk || a.nzphases > 0 || a.ncomp > 0 || a.zstripes > 0 || a.nphases != 1 || a.total_tiles != a.gemm_tiles ||
        a.grid != a.gemm_tiles || ph.nr != 3 || ph.nt != 3 || ph.r0 != 0 || ph.t0 != 0 || ph.dr0 != 1 ||
        ph.dt0 != 1 || ph.ph != 0 || ph.pw != 0 || ph.Wp != a.W || ph.div_hw.d != (uint32_t)(a.H * a.W) ||
        !halo_fits<BM, BN, WM, WN>(a.R, a.S, a.stride, 1, a.H, a.W, a.P, a.Q))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((dgrad_halo<BM, BN, WM, WN>), dim3(a.grid), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
int halo_resident(void)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(dgrad_halo<BM, BN, WM, WN>),
                                                     64 * WM * WN, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    return n > 0 ? n : 1;
}

template <int BM, int BN, int WM, int WN>
int halo_private(void)
{
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(dgrad_halo<BM, BN, WM, WN>)) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return (int)attr.localSizeBytes;
}

// The compiled configurations of this kernel: (BM, BN, WM, WN).
#define CBW_HALO_CONFIGS(X) \
    X(256, 128, 2, 2)

#define CBW_HALO_ENTRY(BM, BN, WM, WN) \
    {BM, BN, 64, WM, WN, #BM "x" #BN "x64/" #WM "x" #WN "h", HaloShape<BM, BN, WM, WN>::LDS_USED, false, false, true, true},
const TileConfig kHaloConfigs[] = {CBW_HALO_CONFIGS(CBW_HALO_ENTRY)};
constexpr int kNumHalo = sizeof(kHaloConfigs) / sizeof(kHaloConfigs[0]);

using HaloLaunchFn = hipError_t (*)(const KernelArgs&, hipStream_t);
using HaloFitsFn = bool (*)(int, int, int, int, int, int, int, int);
#define CBW_HALO_LAUNCH(BM, BN, WM, WN) &halo_launch<BM, BN, WM, WN>,
#define CBW_HALO_FITS(BM, BN, WM, WN) &halo_fits<BM, BN, WM, WN>,
#define CBW_HALO_RESIDENT(BM, BN, WM, WN) &halo_resident<BM, BN, WM, WN>,
#define CBW_HALO_PRIVATE(BM, BN, WM, WN) &halo_private<BM, BN, WM, WN>,
const HaloLaunchFn kHaloLaunch[] = {CBW_HALO_CONFIGS(CBW_HALO_LAUNCH)};
const HaloFitsFn kHaloFits[] = {CBW_HALO_CONFIGS(CBW_HALO_FITS)};
int (*const kHaloResident[])(void) = {CBW_HALO_CONFIGS(CBW_HALO_RESIDENT)};
int (*const kHaloPrivate[])(void) = {CBW_HALO_CONFIGS(CBW_HALO_PRIVATE)};

}  // namespace

int halo_num_configs() { return kNumHalo; }

const TileConfig& halo_config(int i) { return kHaloConfigs[i]; }

bool halo_admits(int i, int R, int S, int stride, int pad, int H, int W, int P, int Q)
{
    return i >= 0 && i < kNumHalo && kHaloFits[i](R, S, stride, pad, H, W, P, Q);
}

hipError_t launch_halo(int i, const KernelArgs& a, hipStream_t stream)
{
    if (i < 0 || i >= kNumHalo)
        return hipErrorInvalidValue;
    return kHaloLaunch[i](a, stream);
}

int halo_blocks_per_cu(int i) { return (i >= 0 && i < kNumHalo) ? kHaloResident[i]() : 1; }

int halo_private_bytes(int i) { return (i >= 0 && i < kNumHalo) ? kHaloPrivate[i]() : -1; }

}  // namespace cbw
