// A third dgrad kernel, for stride-1 layers whose dx and dy images have the
// same extent (P = H, Q = W: "same" padding) and whose filter is at least 3x3:
// per 64-wide k chunk, the dy rows a tile needs for all of its taps are
// loaded into LDS once, with the halo the taps reach, and every tap reads its
// shifted rows from there.
//
// The operation is that of dgrad_igemm and dgrad_wide (the backward-data
// convolution of "[CUTLASS] Conv2d dgrad", apache/tvm PR #10110, as an
// implicit GEMM). With stride 1 and P = H, Q = W, output pixel m (linear in
// n, h, w) takes tap (r, t) from dy pixel m + d, with the constant shift
// d = (pad - r) * W + (pad - t), when the shifted row and column stay inside
// the image. So the BM pixels of a tile read, per k chunk and for all R * S
// taps, only the dy pixels [m0 - D, m0 + BM + D) with D = pad * W + pad,
// where dgrad_wide loads BM rows per tap. On a 3x3 layer with a 256 x 128
// tile that cuts what a slice brings into LDS from 48 KiB to about 20 KiB.
//
// Layout and walk (one tile per workgroup, four waves of 128 x 64 as in
// dgrad_wide):
//   * LDS: a ring of three filter stages (64 k rows x BN channels, as in
//     dgrad_wide), 1 KiB of zeros, and two halo buffers. A halo row is one
//     dy pixel's 64-wide k chunk in eight 16-byte units plus one unused unit
//     (144 bytes), so row x starts 9x units into its buffer: 16 consecutive
//     rows then start in 16 distinct 16-byte bank groups of the 256-byte bank
//     window, whatever the first row, and a fragment read needs no per-lane
//     permutation. One 16-byte load per lane fills 63 units (seven rows) and
//     one more that the next load fills with the same bytes.
//   * Slice it covers k chunk it / RS and tap it % RS (chunks outer, taps
//     inner). Each slice issues one filter slice, two ahead, and then HPS
//     halo loads per wave (loads HPS*tap .. HPS*tap + HPS - 1 of the next
//     chunk's halo, into the buffer the previous chunk used). Loads with no
//     work (past the halo's end, or in the last chunk) write zeros over the
//     zero block, and filter items past the end load the last item again
//     into stages no slice reads, so every slice issues the same count and
//     one vmcnt wait fits all.
//   * Fragments: the filter^T operand as in dgrad_wide (transpose reads);
//     the dy^T fragment of tile pixel p for tap (r, t) is halo row
//     p + D + d, or, where the tap leaves the image, the zero block at the
//     same offset within a 256-byte bank window (so those lanes keep the
//     bank pattern too). Which taps stay inside is a per-lane bit mask
//     formed once.
//   * The per-slice address arithmetic (the halo loads' offsets, the next
//     tap's fragment rows) runs between the matrix-core operations, a few
//     instructions at a time.
//   * The epilogue is dgrad_wide's, with z loaded from HBM into registers
//     at the start of the last slice.
#include "dgrad_internal.h"
#include "kernel_common.h"

namespace cbw {
namespace {

template <int BM, int BN, int WM, int WN>
struct HaloShape {
    static constexpr int NW = WM * WN;
    static constexpr int FSTAGE = 64 * BN * 2;                 // one filter slice (bytes)
    static constexpr int LDS = 160 * 1024;
    static constexpr int ZREG = 1024;                          // the zero block
    static constexpr int ROW = 9 * 16;                         // bytes per halo row
    static constexpr int RPL = 7 * NW;                         // halo rows one load of every wave fills
    static constexpr int HPS = 2;                              // halo loads per wave per slice
    static constexpr int MAX_TAPS = 32;                        // bits of the tap mask
    static constexpr int ZERO0 = 3 * FSTAGE;
    static constexpr int HALO0 = ZERO0 + ZREG;
    // halo rows a buffer holds (plus one row the last load's last lane
    // writes), two buffers in what the filter ring and the zeros leave
    static constexpr int HR_MAX = ((LDS - HALO0) / (2 * ROW) - 1) / RPL * RPL;
    static constexpr int HBUF = (HR_MAX + 1) * ROW;
    static constexpr int LDS_USED = HALO0 + 2 * HBUF;
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
    constexpr int HPS = Sh::HPS;
    constexpr int LDH = B_INSTR + HPS;            // loads per wave per slice
    constexpr int ROW = Sh::ROW;
    constexpr int RPL = Sh::RPL;
    constexpr int HALO0 = Sh::HALO0;
    constexpr int HBUF = Sh::HBUF;
    constexpr int ZERO0 = Sh::ZERO0;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(FSTAGE % (1024 * NW) == 0, "whole 1 KiB blocks per wave");
    static_assert(BN % 64 == 0, "filter rows of at least 8 chunks");
    static_assert(NW * 32 * TN * 2 <= FSTAGE, "the output staging fits one filter stage");
    static_assert(Sh::LDS_USED <= Sh::LDS, "LDS budget");
    static_assert(Sh::HR_MAX >= BM + 2 * RPL, "halo rows");
    static_assert(ZERO0 % 256 == 0 && Sh::ZREG >= 256 + 4 * 32, "zero block: a whole bank window and the sub-step offsets");
    static_assert(LDH + HPS < 64, "vmcnt range");

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
    const int nchunks = (K + BK - 1) / BK;

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
    const int ntap = pin(ph.nt);
    const int RS = pin(ph.nr * ph.nt);
    const int niter = pin(RS * nchunks);
    const int dr0 = pin(ph.dr0), dt0 = pin(ph.dt0);
    const int wt0 = pin(ph.r0 * SC + ph.t0 * C + c0);
    const int M = pin(ph.M);
    // the halo: buffer row x holds dy pixel m0 - D + x
    const int D = pin(dr0 * Q + dt0);
    const int HB = pin(halo_rows(BM, RPL, D) / RPL);   // halo loads per wave per chunk

    const i32x4 dy_desc = raw_descriptor(a.dy, a.dy_bytes);
    const i32x4 w_desc = raw_descriptor(a.w, a.w_bytes);
    const int last = nchunks - 1;
    const bool ragged = K % BK != 0;

    // ---- halo loads. Load j of wave v fills block b = j*NW + v: units
    // 63b .. 63b + 63 of the buffer, lane l unit 63b + l = row 7b + l/9,
    // unit l%9 (unit 8 of a row is unused; lane 63 writes the first unit of
    // row 7b + 7, which block b + 1 writes with the same bytes). The lane's
    // dy pixel is m0 - D + 7*NW*j + 7v + l/9, its k offset 8*(l%9) into the
    // chunk (in the scalar offset); the unused units load nothing. A row whose pixel lies outside the image
    // holds whatever the range check gives: only taps that leave the image
    // would read it, and they read the zero block.
    //
    // While the slices of chunk kc run, they issue loads 0 .. HB - 1 of
    // chunk kc + 1's halo (within the chunk's first RS - 2 slices), into
    // buffer (kc + 1) & 1; the slices' remaining halo loads, and all of them
    // in the last chunk, load nothing and write zeros over the zero block.
    const int hq = lane / 9;
    const int hr = lane - 9 * hq;
    const uint32_t hoff0 = (uint32_t)(m0 - D + 7 * wave + hq) * (uint32_t)(2 * K) + (uint32_t)(16 * hr);
    // lanes that load nothing: the unused unit of a row (no memory access,
    // so a load touches seven rows' lines only), and in the last chunk of a
    // ragged K the units past K
    const bool h_skip = hr == 8;
    const bool h_skip_last = h_skip || last * BK + 8 * hr >= K;
    constexpr uint32_t LSTEP = NW * 63 * 16;                // LDS bytes between a wave's consecutive loads
    const uint32_t VSTEP = pin((uint32_t)(RPL * 2 * K));    // dy bytes between them
    const uint32_t h_wave = lds_u32 + (uint32_t)(HALO0 + wave * 63 * 16);
    int hj = 0;                   // next load of the halo
    uint32_t h_v = 0;             // hj * VSTEP
    uint32_t h_l = 0;             // LDS address of load hj (the zero block once the halo is done)
    uint32_t h_soff = 0;          // k offset of the chunk loaded (bytes)
    bool h_ragged = false;        // that chunk is the last and K is ragged
    bool h_done = true;           // no halo left to load while this chunk runs
    const uint32_t h_zero = lds_u32 + (uint32_t)ZERO0;
    // aim the halo loads at chunk kc + 1 while chunk kc runs
    auto halo_target = [&](int kc_now) __attribute__((always_inline)) {
        const int hk = kc_now + 1;
        hj = 0;
        h_v = 0;
        h_done = hk > last;
        h_l = h_done ? h_zero : pin(h_wave + (uint32_t)((hk & 1) * HBUF));
        h_soff = pin((uint32_t)(hk * BK * 2));
        h_ragged = ragged && hk == last;
    };
    auto issue_halo = [&]() __attribute__((always_inline)) {
        const uint32_t vo = hoff0 + h_v;
        const bool skip = h_done || (h_ragged ? h_skip_last : h_skip);
        dma16(dy_desc, skip ? 0x80000000u : vo, h_soff, h_l);
        ++hj;
        h_v += VSTEP;
        h_done = h_done || hj == HB;
        h_l = h_done ? h_zero : h_l + LSTEP;
    };

    // ---- filter slices: item i = chunk i / RS, tap i % RS, at byte offset
    // 2*(c0 + tap*C + 64*chunk*R*S*C) (one phase with every tap: tap
    // (r, t) = r*S + t lies r*S*C + t*C elements in). Byte 16*l of block
    // jn*NW + v of a stage is row k, position p, holding logical chunk
    // p ^ w_swizzle(k); in the last chunk of a ragged K the rows past K load
    // zeros. Items past the end load the last item again (into stages no
    // slice reads).
    int b_k[B_INSTR];
    uint32_t w_vt[B_INSTR], w_vl[B_INSTR], w_vo[B_INSTR];
#pragma unroll
    for (int jn = 0; jn < B_INSTR; ++jn) {
        const int byte = (jn * NW + wave) * 1024 + 16 * lane;
        const int k = byte / B_ROW;
        const int pos = (byte % B_ROW) / 16;
        const int cc = (pos ^ w_swizzle<B_ROW>(k)) * 8;
        b_k[jn] = k;
        w_vt[jn] = c0 + cc >= C ? 0x80000000u : (uint32_t)(k * RSC + cc) * 2u;
        w_vl[jn] = last * BK + k >= K ? 0x80000000u : w_vt[jn];
        w_vo[jn] = last == 0 ? w_vl[jn] : w_vt[jn];
    }
    const uint32_t WTAP = pin((uint32_t)(2 * C));                     // next tap
    const uint32_t WCHUNK = pin((uint32_t)(2 * (BK * RSC - RS * C)));  // first tap of the next chunk, after a WTAP step
    int item = 0, i_t = 0, i_k = 0;
    uint32_t so_w = pin((uint32_t)(2 * wt0));
    const uint32_t dma_base = pin(lds_u32 + (uint32_t)(wave * 1024));
    auto issue_filter = [&](auto st_c, auto x_c) __attribute__((always_inline)) {
        constexpr int ST = decltype(st_c)::value;
        constexpr int X = decltype(x_c)::value;
        dma16_at<(uint32_t)(ST * FSTAGE + X * NW * 1024)>(w_desc, w_vo[X], so_w, dma_base);
    };
    auto advance_item = [&]() __attribute__((always_inline)) {
        if (item + 1 < niter) {
            so_w += WTAP;
            if (++i_t == RS) {
                i_t = 0;
                so_w += WCHUNK;
                if (++i_k == last) {
#pragma unroll
                    for (int jn = 0; jn < B_INSTR; ++jn)
                        w_vo[jn] = w_vl[jn];
                }
            }
        }
        ++item;
    };

    // ---- fragment rows. dy^T (B): tile pixel p = wm*TM + fm*32 + lane%32 at
    // k chunk 2*kk + lane/32 is halo row p + D + d for the tap's shift d, at
    // byte 144*(p + D + d) + 16*(2*kk + lane/32) of the chunk's buffer.
    // tmask bit t: tap t keeps the pixel inside the image (none for a pixel
    // past the end).
    int b_lane[FM];          // 144*(p + D) + 16*(lane/32)
    uint32_t tmask[FM];      // formed after the prologue's loads are issued
    uint32_t b_addr[FM];     // LDS byte address of the fragment row for the tap in hand
    // fragment row fm for tap `tp`, whose rows start at LDS byte u (the
    // buffer start plus 144*d)
    auto set_row = [&](int fm, int tp, uint32_t u) __attribute__((always_inline)) {
        const uint32_t ad = (uint32_t)b_lane[fm] + u;
        b_addr[fm] = (tmask[fm] >> tp) & 1u ? ad : ((ad & 255u) | (uint32_t)ZERO0);
    };
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
    // fragments of sub-step kk: the filter from stage ST, dy rows at b_addr
    auto read_frags = [&](auto st_c, auto kk_c, half8_t (&af)[FN], half8_t (&bf)[FM]) __attribute__((always_inline)) {
        constexpr int sb = decltype(st_c)::value * FSTAGE;
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
        for (int fm = 0; fm < FM; ++fm)
            bf[fm] = __builtin_bit_cast(half8_t, *(const __attribute__((address_space(3))) u32x4*)((lds_char*)lds + b_addr[fm] + KK * 32));
    };

    // ---- the slice loop, as in dgrad_wide: one barrier in the middle of a
    // slice (after sub-step 2's operations are issued, the wave waits for
    // the loads it needs, and for its fragment reads), then the next slice's
    // first fragments are read under sub-step 3.
    //
    // Loads, in issue order per slice: filter item it + 2 (B_INSTR loads, in
    // sub-steps 0 and 1), then HPS halo loads (sub-step 2). The wait lets the
    // last LDH + HPS loads stay in flight: this slice's and the previous
    // slice's halo loads; so it covers filter item it + 1 and every halo load
    // from before the previous slice: at the last slice of a chunk, the whole
    // halo of the next chunk (loaded within its first RS - 2 slices).
    // Who may overwrite what: the halo of chunk kc + 1 goes into the buffer
    // chunk kc - 1 read, from the first slice of chunk kc on; every read of
    // chunk kc - 1 ended before the barrier of its last slice. Filter item
    // it + 2 goes into the stage of slice it - 1, whose reads ended before
    // slice it - 1's barrier.
    constexpr int OPS = FM * FN;          // operations per sub-step
    static_assert(OPS >= 8 && FM <= 4, "slots for the per-slice work");
    half8_t af[2][FN], bf[2][FM];
    // what runs after operation J of sub-step KK
    auto slot = [&](auto st_c, auto kk_c, auto j_c, int ntp, uint32_t nu) __attribute__((always_inline)) {
        constexpr int KK = decltype(kk_c)::value;
        constexpr int J = decltype(j_c)::value;
        if constexpr (KK < 2) {
            static_for<0, B_INSTR>([&](auto x_c) {
                if constexpr (decltype(x_c)::value * 2 * OPS / B_INSTR == KK * OPS + J)
                    issue_filter(st_c, x_c);
            });
        } else if constexpr (KK == 2) {
            static_for<0, HPS>([&](auto h_c) {
                if constexpr (decltype(h_c)::value * OPS / HPS == J)
                    issue_halo();
            });
            // the next slice's fragment rows (every read of this slice's rows is issued)
            static_for<0, FM>([&](auto f_c) {
                if constexpr (OPS - FM + decltype(f_c)::value == J)
                    set_row(decltype(f_c)::value, ntp, nu);
            });
        }
    };
    auto ops = [&](auto st_c, int f, auto kk_c, int ntp, uint32_t nu) __attribute__((always_inline)) {
        static_for<0, OPS>([&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            constexpr int fm = J / FN, fn = J % FN;
            acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[f][fn], bf[f][fm], acc[fn][fm], 0, 0, 0);
            slot(st_c, kk_c, j_c, ntp, nu);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // ---- the fused epilogue's z: the lane's share (pixel lane%32 of group
    // fm, channels 8*gq + 4*(lane/32) .. +3 of block fn of the wave's
    // columns), loaded into registers at the start of the last slice so the
    // latency hides behind its operations
    const bool zpre = a.epi != kEpiNone;
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
    u32x2 zr[FM][FN][4];
    auto load_z = [&]() __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t z_rsrc = make_rsrc(a.z, a.dx_bytes);
        const int cw = c0 + wn * TN;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int m = m0 + wm * TM + fm * 32 + (lane & 31);
            const uint32_t pix = pixel_offset(m);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int c = cw + fn * 32 + 8 * gq + 4 * (lane >> 5);
                    zr[fm][fn][gq] = __builtin_amdgcn_raw_buffer_load_b64(
                        z_rsrc, out_of_range_if((uint32_t)(m >= M) | (uint32_t)(c >= C), (pix + (uint32_t)c) * 2u), 0, 0);
                }
        }
    };
    // the walk: tap `tap` (column `at`) of chunk `kc`, whose fragment rows
    // start at u_d = 144*d past the buffer start
    int kc = 0, tap = 0, at = 0;
    const uint32_t D144 = pin((uint32_t)(ROW * D));
    const uint32_t ROWSTEP = pin((uint32_t)(ROW * (Q - ntap)));   // next filter row, after a column step
    uint32_t u_d = D144;
    // slice it (filter in stage ST = it % 3); filter item it + 2 goes into
    // stage (ST + 2) % 3
    auto slice = [&](auto st_c, int it) __attribute__((always_inline)) {
        constexpr IC<(decltype(st_c)::value + 1) % 3> next_c{};
        constexpr IC<(decltype(st_c)::value + 2) % 3> req_c{};
        if (zpre && it + 1 == niter)
            load_z();
        // the next slice: tap + 1, or the first tap of the next chunk
        int ntp = tap + 1, nat = at + 1;
        uint32_t nd = u_d - (uint32_t)ROW;
        if (nat == ntap) {
            nat = 0;
            nd -= ROWSTEP;
        }
        const bool new_chunk = ntp == RS;
        if (new_chunk) {
            ntp = 0;
            nd = D144;
        }
        const uint32_t nu = pin((uint32_t)(HALO0 + ((kc + (int)new_chunk) & 1) * HBUF) + nd);
        ops(req_c, 0, IC<0>{}, ntp, nu);
        read_frags(st_c, IC<2>{}, af[0], bf[0]);
        ops(req_c, 1, IC<1>{}, ntp, nu);
        read_frags(st_c, IC<3>{}, af[1], bf[1]);
        ops(req_c, 0, IC<2>{}, ntp, nu);
        const bool has_next = it + 1 < niter;
        if (has_next) {
            wait_vmcnt<LDH + HPS>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
            read_frags(next_c, IC<0>{}, af[0], bf[0]);
        }
        ops(req_c, 1, IC<3>{}, ntp, nu);
        if (has_next)
            read_frags(next_c, IC<1>{}, af[1], bf[1]);
        advance_item();
        tap = ntp;
        at = nat;
        u_d = nd;
        if (new_chunk) {
            ++kc;
            halo_target(kc);
        }
    };

    // ---- prologue: the zero block (wave 0, a load with every lane out of
    // range), the halo of chunk 0, filter items 0 and 1, and HPS loads with
    // no work standing in for the halo loads of a slice before slice 0 (the
    // slice loop's waits count on them)
    if (wave == 0)
        dma16(dy_desc, 0x80000000u, 0u, lds_u32 + (uint32_t)ZERO0);
    for (int j = 0; j < HB; ++j) {
        const uint32_t vo = hoff0 + (uint32_t)j * VSTEP;
        dma16(dy_desc, (last == 0 ? h_skip_last : h_skip) ? 0x80000000u : vo, 0u, h_wave + (uint32_t)j * LSTEP);
    }
    static_for<0, B_INSTR>([&](auto x_c) { issue_filter(IC<0>{}, x_c); });
    advance_item();
    static_for<0, B_INSTR>([&](auto x_c) { issue_filter(IC<1>{}, x_c); });
    advance_item();
    static_for<0, HPS>([&](auto) { dma16(dy_desc, 0x80000000u, 0u, lds_u32 + (uint32_t)ZERO0); });
    halo_target(0);
    // the tap masks, while those loads are in flight: tap (r, t) = r*S + t
    // stays inside for the pixel at (i, j) when row i + pad - r and column
    // j + pad - t do
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int pr = wm * TM + fm * 32 + (lane & 31);
        const int m = m0 + pr;
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const int i = (int)fastdiv(rem, ph.div_w);
        const int jj = (int)(rem - (uint32_t)i * (uint32_t)ph.Wp);
        uint32_t cols = 0;
        for (int t = 0; t < ntap; ++t)
            cols |= (uint32_t)((unsigned)(jj + dt0 - t) < (unsigned)Q) << t;
        uint32_t mask = 0;
        for (int r = 0, sh = 0; sh < RS; ++r, sh += ntap)
            mask |= (unsigned)(i + dr0 - r) < (unsigned)P ? cols << sh : 0u;
        tmask[fm] = m < M ? mask : 0u;
        b_lane[fm] = ROW * (pr + D) + 16 * (lane >> 5);
    }
    wait_vmcnt<B_INSTR + HPS>();          // all but filter item 1 and those
    __syncthreads();
    {
        const uint32_t u0 = pin((uint32_t)HALO0 + D144);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            set_row(fm, 0, u0);
    }
    read_frags(IC<0>{}, IC<0>{}, af[0], bf[0]);
    read_frags(IC<0>{}, IC<1>{}, af[1], bf[1]);
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

    // ---- epilogue: acc x g(z) -> fp16 (RNE), staged through the filter
    // stage of the last slice and stored as whole pixel rows (as in
    // dgrad_wide).
    const int sdone = (niter - 1) % 3;
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
        lds_char* blk = (lds_char*)lds + sdone * FSTAGE + wave * EBLK;
        wait_vmcnt<0>();   // the z loads, and no load writes LDS after the end
        __syncthreads();   // every wave is done reading the stage's operands
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
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

// The layers this kernel runs: stride 1 with P = H and Q = W (so the tap
// shifts are constant along the linear pixel index), a filter of 3x3 up to
// 32 taps (one bit each in the tap mask), and a halo that fits its buffers
// and is loaded within the first R*S - 2 slices of a chunk.
template <int BM, int BN, int WM, int WN>
bool halo_fits(int R, int S, int stride, int pad, int H, int W, int P, int Q)
{
    using Sh = HaloShape<BM, BN, WM, WN>;
    if (stride != 1 || P != H || Q != W || R < 3 || S < 3 || R * S > Sh::MAX_TAPS || pad < 0 || pad >= R || pad >= S)
        return false;
    const long D = (long)pad * Q + pad;
    if (D > Sh::HR_MAX)
        return false;
    const int hr = halo_rows(BM, Sh::RPL, (int)D);
    return hr <= Sh::HR_MAX && hr / Sh::RPL <= Sh::HPS * (R * S - 2);
}

// The launch must be one such phase (taps from (0, 0), dy offsets of the
// first tap = pad) in GEMM tiles only, one per workgroup.
template <int BM, int BN, int WM, int WN>
hipError_t halo_launch(const KernelArgs& a, hipStream_t stream)
{
    const PhaseArg& ph = a.ph[0];
    if (a.sk || a.nzphases > 0 || a.ncomp > 0 || a.zstripes > 0 || a.nphases != 1 || a.total_tiles != a.gemm_tiles ||
        a.grid != a.gemm_tiles || ph.nr != a.R || ph.nt != a.S || ph.r0 != 0 || ph.t0 != 0 || ph.dr0 != ph.dt0 ||
        ph.ph != 0 || ph.pw != 0 || ph.Wp != a.W || ph.div_hw.d != (uint32_t)(a.H * a.W) ||
        !halo_fits<BM, BN, WM, WN>(a.R, a.S, a.stride, ph.dr0, a.H, a.W, a.P, a.Q))
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
