// HIP kernels for conv2d backward-data on CDNA4 (gfx950).
//
// The operation is the backward-data convolution of "[CUTLASS] Conv2d dgrad"
// (apache/tvm PR #10110), computed as an implicit GEMM per stride phase (see
// dgrad_plan.h). One launch covers up to 16 phases; each workgroup owns one
// BM x BN tile of one phase's GEMM:
//     rows    = BM dx pixels of the phase lattice (h = ph + s*i, w = pw + s*j)
//     columns = BN dx channels
//     reduce  = the phase's taps x K, in 64-wide slices
//
// Operand path (per 64-wide slice):
//   * dy slice (BM gathered dy rows x 64 k) and filter slice (64 k rows x BN
//     channels, channel-contiguous as the KRSC layout stores them) travel
//     HBM/L2 -> LDS with 16-byte buffer loads that write LDS directly. Each
//     wave instruction fills a contiguous 1 KiB block (lane l at +16*l);
//     out-of-range lanes (padding rows, dead rows, ragged K or C) use an
//     offset past the buffer and the hardware writes zeros. No staging
//     registers are involved.
//   * Three LDS stages form a ring: slice it+2 is requested while slice it is
//     on the matrix cores, with one barrier per slice. The loads are issued
//     from inline assembly and waited for with exact counts: the compiler's
//     own wait insertion does not tell LDS buffers apart and would wait for
//     every outstanding load before any LDS read.
//   * Matrix cores: v_mfma_f32_32x32x16_f16 with A = filter^T (rows =
//     channels) and B = dy^T (columns = pixels). The dy fragment is one
//     16-byte LDS read per lane. The filter fragment (8 consecutive k of one
//     channel) comes from two ds_read_b64_tr_b16 transpose reads: within each
//     group of 16 lanes, lane 4r+q reads row r, channels 4q..4q+3, and lane i
//     receives channel i of the four rows. Fragments are double-buffered
//     across the four 16-wide sub-steps of a slice.
//
// LDS layouts (per stage):
//   dy slice: BM rows x 128 bytes; chunk c of row m at position c ^ ((m>>1)&7)
//             (16 lanes reading one chunk of 16 consecutive rows hit 16
//             distinct 16-byte bank groups of the 256-byte bank window)
//   w  slice: 64 rows x 2*BN bytes; chunk c of row k at position
//             c ^ 4*(k&3) (c ^ 4*((k>>1)&1) for 128-byte rows)
//             (the 32 lanes of half a transpose read cover 256 distinct bytes
//             of the bank window)
//
// Persistent walk: the grid holds as many workgroups as can be resident;
// each walks its tiles in rounds, and the slice stream runs across tile
// boundaries, so a tile's first slices are in flight while the previous tile
// finishes (short reductions, 2..8 slices per tile, would otherwise pay the
// full load latency per tile).
//
// Epilogue: each lane holds 4 consecutive channels of one pixel per register
// group; it multiplies by g(z) (relu' or hardswish' of the saved
// pre-activation, fp32), rounds once to fp16 (RNE) and stores 8 bytes. dx is
// never read. Zero phases (no tap reaches the lattice) store zeros with
// 16-byte stores.
#include <algorithm>
#include <map>
#include <mutex>

#include "dgrad_internal.h"
#include "kernel_common.h"

namespace cbw {
namespace {

// The kernel's arguments, read again from the kernarg segment where they are
// used. The empty asm keeps the compiler from hoisting these loads, so that
// values needed only now and then (the epilogue's descriptors) are not held
// in scalar registers through the main loop.
__device__ inline const __attribute__((address_space(4))) KernelArgs* kernargs()
{
    auto p = (const __attribute__((address_space(4))) KernelArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return p;
}

// The phase-interleaved tile order (order 2) exists for every configuration
// but 256x64/4x1, whose scalar registers are full without it.
template <int BM, int BN, int WM, int WN>
constexpr bool kHasPhaseOrder = !(BM == 256 && BN == 64 && WM == 4);

// Kernel variants by the work a launch carries (MODE): kPlain for GEMM tiles
// alone, kCompanion when zero phases ride along only as companion stores,
// kZeroWork for zero stripes and standalone zero chunks (and companions),
// kStreamK for a split reduction (never with zero work). Each drops the state
// the others need, which keeps the uniform values of the main loop in scalar
// registers.
constexpr int kPlain = 0;
constexpr int kZeroWork = 1;
constexpr int kStreamK = 2;
constexpr int kCompanion = 3;

template <int BM, int BN, int WM, int WN, int MODE>
__global__ void __launch_bounds__(64 * WM * WN) dgrad_igemm(KernelArgs a)
{
    constexpr bool SK = MODE == kStreamK;
    constexpr bool ZW = MODE == kZeroWork;                 // zero stripes and chunks
    constexpr bool CP = ZW || MODE == kCompanion;          // companion stores
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
    static_assert(LD + 2 * kMaxZeroPerSlice < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE];
    const uint32_t lds_u32 = (uint32_t)(uintptr_t)((lds_char*)lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int s = pin(a.stride);
    const int C = pin(a.C);
    const int K = pin(a.K);
    const int P = pin(a.P);
    const int Q = pin(a.Q);
    const int ksteps = (K + BK - 1) / BK;
    const int SC = pin(a.S * C);          // filter elements per tap row
    const int RSC = pin(a.R * SC);        // filter elements per k
    const uint32_t zps = ZW ? pin((uint32_t)a.zps) : 0u;
    const uint32_t zt = ZW ? pin((uint32_t)a.zt) : 0u;
    const uint32_t zabsorbed = ZW ? pin(a.zabsorbed) : 0u;
    const int ncomp = CP ? pin(a.ncomp) : 0;

    const __amdgpu_buffer_rsrc_t dx_rsrc = make_rsrc(a.dx, a.dx_bytes);
    const i32x4 dy_desc = raw_descriptor(a.dy, a.dy_bytes);
    const i32x4 w_desc = raw_descriptor(a.w, a.w_bytes);

    // ---- persistent tile walk: the grid is the number of resident workgroups;
    // in round k this workgroup owns logical tile k*G + remap(blockIdx.x).
    const int G = gridDim.x;
    const int slot = xcd_remap(blockIdx.x, G, a.group, a.xcd_mode);
    struct Tile {
        int pi, m0, c0, niter, s0;   // s0: the tile's first slice in the launch's numbering
    };
    // GEMM tile `tile` (< gemm_tiles): its phase, first lattice row, first channel, slices.
    // `round` is tile / G, which the walk knows.
    auto decode = [&](int tile, int round) -> Tile {
        int pi = 0, local = 0;
        if (MODE == kPlain && kHasPhaseOrder<BM, BN, WM, WN> && kernargs()->order == 2) {   // the phases of one block side by
            // side, rotating with the round (every phase has the same tiles and
            // the grid is a multiple of the phase count, so this is a bijection
            // onto phase-major numbers); launches of the plain variant only.
            // Read in place: nothing of this is held through the main loop.
            const int np = kernargs()->nphases;
            const int blk = tile / np;
            const int j = tile - blk * np;
            pi = (j + round) % np;
            local = blk;
        } else {
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
        const int niter = a.ph[pi].nr * a.ph[pi].nt * ksteps;
        return Tile{pi, tm * BM, tn * BN, niter, a.slice_begin[pi] + local * niter};
    };

    // ---- work segments: slices [lo, hi) of one tile. Without stream-K the
    // k-th segment of this workgroup is the whole tile k*G + slot. With it
    // (segment() below), workgroup `slot` owns slices
    // [floor(slot*T/G), floor((slot+1)*T/G)) of the launch's T slices, tile
    // after tile.
    struct Seg {
        int tile, lo, hi;
        bool ok;
    };
    const uint32_t skT = (uint32_t)a.sk_slices;
    auto sk_start = [&](uint32_t w) -> uint32_t { return (uint32_t)(((uint64_t)w * skT) / (uint32_t)G); };
    auto sk_owner = [&](uint32_t sl) -> uint32_t {   // the workgroup whose range holds slice sl
        return (uint32_t)((((uint64_t)sl + 1) * (uint32_t)G - 1) / skT);
    };
    auto segment = [&](int k, Tile& t) -> Seg {
        // this workgroup's range and its first tile (recomputed at each
        // segment boundary rather than held in registers through the loop)
        const uint32_t sk_s0 = sk_start((uint32_t)slot);
        const uint32_t sk_s1 = sk_start((uint32_t)slot + 1);
        if (sk_s1 <= sk_s0)
            return Seg{0, 0, 0, false};
        int pi = 0;
        for (int i = 1; i < a.nphases; ++i)
            if (sk_s0 >= (uint32_t)a.slice_begin[i])
                pi = i;
        const int niter0 = a.ph[pi].nr * a.ph[pi].nt * ksteps;
        const int tile = a.ph[pi].tile_begin + (int)((sk_s0 - (uint32_t)a.slice_begin[pi]) / (uint32_t)niter0) + k;
        if (tile >= a.gemm_tiles)
            return Seg{0, 0, 0, false};
        t = decode(tile, 0);
        const int lo = k == 0 ? (int)(sk_s0 - (uint32_t)t.s0) : 0;
        if ((uint32_t)(t.s0 + lo) >= sk_s1)
            return Seg{0, 0, 0, false};
        const int hi = (uint32_t)(t.s0 + t.niter) <= sk_s1 ? t.niter : (int)(sk_s1 - (uint32_t)t.s0);
        return Seg{tile, lo, hi, true};
    };

    // dx element offset of lattice row m of phase ph (pixel n, h = ph + s*i, w = pw + s*j)
    auto pixel_offset = [&](const PhaseArg& ph, int m) -> uint32_t {
        const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
        const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
        const uint32_t i = fastdiv(rem, ph.div_w);
        const uint32_t j = rem - i * (uint32_t)ph.Wp;
        const uint32_t pix = (n * (uint32_t)a.H + (uint32_t)(ph.ph + s * (int)i)) * (uint32_t)a.W
                             + (uint32_t)(ph.pw + s * (int)j);
        return pix * (uint32_t)C;
    };

    // Zero stripe `stripe` (uniform): vectors stripe*NT .. stripe*NT+NT-1 of the
    // zero list, one 16-byte store of zeros per thread. A stripe lies in one
    // zero phase (ranges are stripe-aligned); padding vectors past the phase's
    // M*C/8 and stripes past the list are dropped by the range check. The
    // stripes a workgroup stores only increase, so the zero phase in use is a
    // cursor that moves forward.
    int zc = -1;                          // current zero phase
    uint32_t zc_begin = 0, zc_next = 0;   // its first vector, and the next phase's
    int zc_ph = 0, zc_pw = 0, zc_Wp = 0, zc_M = 0;
    FastDiv zc_hw{1, 0, 0}, zc_w{1, 0, 0};
    auto zero_stripe = [&](uint32_t stripe, bool valid) {
        const uint32_t vb = stripe * (uint32_t)NT;
        if (valid) {
            while (vb >= zc_next) {       // rare: enter the next zero phase
                ++zc;
                const ZeroPhaseArg& z = a.zph[zc];
                zc_begin = z.vbegin;
                zc_next = zc + 1 < a.nzphases ? a.zph[zc + 1].vbegin : 0xffffffffu;
                zc_ph = z.ph;
                zc_pw = z.pw;
                zc_Wp = z.Wp;
                zc_M = z.M;
                zc_hw = z.div_hw;
                zc_w = z.div_w;
            }
        }
        const uint32_t u = vb - zc_begin + (uint32_t)tid;
        const uint32_t m = fastdiv(u, a.div_c8);
        const uint32_t c = (u - m * a.div_c8.d) * 8u;
        const uint32_t n = fastdiv(m, zc_hw);
        const uint32_t rem = m - n * zc_hw.d;
        const uint32_t i = fastdiv(rem, zc_w);
        const uint32_t j = rem - i * (uint32_t)zc_Wp;
        const uint32_t pix = (n * (uint32_t)a.H + (uint32_t)zc_ph + (uint32_t)s * i) * (uint32_t)a.W
                             + (uint32_t)zc_pw + (uint32_t)s * j;
        const uint32_t bad = (uint32_t)!valid | (uint32_t)(m >= (uint32_t)zc_M);
        const u32x4 zero{0u, 0u, 0u, 0u};
        __builtin_amdgcn_raw_buffer_store_b128(zero, dx_rsrc, out_of_range_if(bad, (pix * (uint32_t)C + c) * 2u), 0, kStoreSystem);
    };

    // ---- request side: the stream of slices of this workgroup's GEMM tiles,
    // running up to two slices ahead of the matrix cores. A tile's slices go
    // tap by tap and, within a tap, over k in BK-wide steps. A lane's dy
    // address then changes only at tap boundaries: for a whole tap it is a
    // per-lane byte offset (or the out-of-range offset 2^31 for a padding tap
    // or a dead row) plus the wave-uniform 2*k0, which goes into the load's
    // scalar offset; a full-width slice needs no per-lane arithmetic at all.
    // Only a ragged last k step (K not a multiple of BK) masks lanes further.
    // DMA block b = jn*NW + wave of a dy slice covers tile rows 8b..8b+7; lane l
    // fills row 8b + l/8 at chunk position l%8, holding logical chunk
    // (l%8) ^ dy_swizzle(row). Byte 16*l of block jn*NW + wave of a filter
    // slice is row k, position p, holding logical chunk p ^ w_swizzle(k).
    int a_k[A_INSTR], b_k[B_INSTR], b_c[B_INSTR];
    uint32_t w_lane[B_INSTR];  // byte offset of the lane's filter element within a slice
#pragma unroll
    for (int jn = 0; jn < A_INSTR; ++jn)
        a_k[jn] = ((lane & 7) ^ dy_swizzle((jn * NW + wave) * 8 + (lane >> 3))) * 8;
#pragma unroll
    for (int jn = 0; jn < B_INSTR; ++jn) {
        const int byte = (jn * NW + wave) * 1024 + 16 * lane;
        const int k = byte / B_ROW;
        const int pos = (byte % B_ROW) / 16;
        b_k[jn] = k;
        b_c[jn] = (pos ^ w_swizzle<B_ROW>(k)) * 8;
        w_lane[jn] = (uint32_t)(k * RSC + b_c[jn]) * 2u;
    }
    uint32_t a_off[A_INSTR];   // byte offset of dy[n, i, j, chunk*8], modulo 2^32: a
    int a_i[A_INSTR];          // lattice row i may exceed P, but every offset that is
    int a_j[A_INSTR];          // loaded (0 <= i+dr < P, 0 <= j+dt < Q) is exact
    uint32_t dy_vo[A_INSTR];   // the lane's dy byte offset for the current tap and k step
    uint32_t w_vt[B_INSTR];    // the lane's filter byte offset for the tile (2^31: channel past C)
    uint32_t w_vo[B_INSTR];    // ... for the current k step
    int rq_round = 0, rq_left = 0, rq_c0 = 0, rq_tile = 0, rq_niter = 0;
    // taps of the tile being requested (scalar copies of its phase's fields)
    int rq_dr0 = 0, rq_dt0 = 0, rq_nt = 1, rq_wt0 = 0;
    int ar = 0, at = 0, k0 = 0;
    bool new_tap = true;       // the cursor entered a new tap: recompute the lanes' offsets
    uint32_t q_wtap = 0;       // filter byte offset of the current tap (wave-uniform)
    uint32_t q_base = 0;       // LDS address of the stage being filled
    // Pick the next slice of the stream; false when the stream is exhausted.
    auto prepare_next = [&](int buf) -> bool {
        while (rq_left == 0) {  // move to the next segment
            Tile t;
            Seg g;
            if constexpr (SK) {
                g = segment(rq_round, t);
                if (!g.ok)
                    return false;
            } else {
                const int tile = rq_round * G + slot;
                if (tile >= a.gemm_tiles)
                    return false;
                t = decode(tile, rq_round);
                g = Seg{tile, 0, t.niter, true};
            }
            ++rq_round;
            rq_c0 = t.c0;
            rq_left = g.hi - g.lo;
            rq_niter = g.hi - g.lo;
            rq_tile = g.tile;
            const PhaseArg& ph = a.ph[t.pi];
            {   // the cursor at slice g.lo of the tile (k innermost, then taps)
                const int tap = g.lo / ksteps;
                ar = tap / ph.nt;
                at = tap - ar * ph.nt;
                k0 = (g.lo - tap * ksteps) * BK;
            }
            new_tap = true;
            rq_dr0 = pin(ph.dr0);
            rq_dt0 = pin(ph.dt0);
            rq_nt = pin(ph.nt);
            rq_wt0 = pin(ph.r0 * SC + ph.t0 * C);
#pragma unroll
            for (int jn = 0; jn < A_INSTR; ++jn) {
                const int m = t.m0 + (jn * NW + wave) * 8 + (lane >> 3);
                const uint32_t n = fastdiv((uint32_t)m, ph.div_hw);
                const uint32_t rem = (uint32_t)m - n * ph.div_hw.d;
                const uint32_t i = fastdiv(rem, ph.div_w);
                const uint32_t j = rem - i * (uint32_t)ph.Wp;
                a_i[jn] = m < ph.M ? (int)i : -(1 << 24);   // a dead row fails every p >= 0 test
                a_j[jn] = (int)j;
                a_off[jn] = (((n * (uint32_t)P + i) * (uint32_t)Q + j) * (uint32_t)K + (uint32_t)a_k[jn]) * 2u;
            }
#pragma unroll
            for (int jn = 0; jn < B_INSTR; ++jn)
                w_vt[jn] = rq_c0 + b_c[jn] >= C ? 0x80000000u : w_lane[jn];
        }
        if (new_tap) {          // once per tap: padding checks and dy offsets
            new_tap = false;
            const int dr = rq_dr0 - ar;
            const int dt = rq_dt0 - at;
            const uint32_t tapoff = (uint32_t)((dr * Q + dt) * K) * 2u;
#pragma unroll
            for (int jn = 0; jn < A_INSTR; ++jn) {
                const bool ok = ((unsigned)(a_i[jn] + dr) < (unsigned)P) & ((unsigned)(a_j[jn] + dt) < (unsigned)Q);
                dy_vo[jn] = ok ? a_off[jn] + tapoff : 0x80000000u;
            }
#pragma unroll
            for (int jn = 0; jn < B_INSTR; ++jn)
                w_vo[jn] = w_vt[jn];
            q_wtap = (uint32_t)(rq_wt0 + ar * s * SC + at * s * C + rq_c0) * 2u;
        }
        if (k0 + BK > K) {      // ragged last k step of a tap: mask the lanes past K
#pragma unroll
            for (int jn = 0; jn < A_INSTR; ++jn)
                dy_vo[jn] = k0 + a_k[jn] >= K ? 0x80000000u : dy_vo[jn];
#pragma unroll
            for (int jn = 0; jn < B_INSTR; ++jn)
                w_vo[jn] = k0 + b_k[jn] >= K ? 0x80000000u : w_vo[jn];
        }
        q_base = lds_u32 + (uint32_t)(buf * STAGE);
        return true;
    };
    // Issue part `part` (of 4) of the prepared slice's direct-to-LDS loads:
    // load number x (dy blocks first, then filter blocks) is in part x*4/LD.
    auto issue_part = [&](int part) {
#pragma unroll
        for (int x = 0; x < LD; ++x) {
            if (x * 4 / LD != part)
                continue;
            if (x < A_INSTR) {
                const int jn = x;
                dma16(dy_desc, dy_vo[jn], (uint32_t)k0 * 2u, q_base + (uint32_t)((jn * NW + wave) * 1024));
            } else {
                const int jn = x - A_INSTR;
                dma16(w_desc, w_vo[jn], q_wtap + (uint32_t)(k0 * RSC) * 2u,
                      q_base + (uint32_t)(A_BYTES + (jn * NW + wave) * 1024));
            }
        }
    };
    // The zero stripes that ride with the prepared slice: slice number si of
    // GEMM tile t stores stripes t*zt + si*zps + j (j < zps) of its share.
    // Exactly zps stores per request, so the waits below can count them;
    // those outside the tile's share are dropped by the range check.
    auto issue_zero = [&]() {
        if constexpr (!ZW)
            return;
        const uint32_t first = (uint32_t)(rq_niter - rq_left) * zps;
        for (uint32_t jz = 0; jz < zps; ++jz) {
            const uint32_t idx = first + jz;
            const uint32_t stripe = (uint32_t)rq_tile * zt + idx;
            zero_stripe(stripe, idx < zt && stripe < zabsorbed);
        }
    };
    // Advance the cursor past the issued slice: k innermost, then taps.
    auto finish_request = [&]() {
        k0 += BK;
        if (k0 >= K) {
            k0 = 0;
            new_tap = true;
            if (++at == rq_nt) {
                at = 0;
                ++ar;
            }
        }
        --rq_left;
    };
    auto request_next = [&](int buf) -> bool {
        if (!prepare_next(buf))
            return false;
        for (int part = 0; part < 4; ++part)
            issue_part(part);
        issue_zero();
        finish_request();
        return true;
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
        const int cl = wn * TN + fn * 32 + (g & 1) * 16 + 4 * qq;   // first channel this lane reads
        const int krow = (g >> 1) * 8 + rr;
        a_frag[fn] = A_BYTES + krow * B_ROW + (((cl >> 3) ^ w_swizzle<B_ROW>(krow)) * 16) + (cl & 7) * 2;
    }

    float16_t acc[FN][FM];
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
    // One slice on the matrix cores; when `issue` is set, the prepared next
    // slice's loads go out in four parts between the sub-steps, so their
    // address arithmetic and issue overlap matrix-core work.
    auto compute = [&](int buf, bool issue) {
        const int sb = buf * STAGE;
        half8_t af0[FN], bf0[FM], af1[FN], bf1[FM];
        read_frags(sb, 0, af0, bf0);
        read_frags(sb, 1, af1, bf1);
        if (issue)
            issue_part(0);
        mfma_step(af0, bf0);
        read_frags(sb, 2, af0, bf0);
        if (issue)
            issue_part(1);
        mfma_step(af1, bf1);
        read_frags(sb, 3, af1, bf1);
        if (issue)
            issue_part(2);
        mfma_step(af0, bf0);
        if (issue) {
            issue_part(3);
            issue_zero();
        }
        mfma_step(af1, bf1);
    };

    // ---- epilogue. The lane holds channels 8*gq + 4*(lane/32) .. +3 of
    // block fn, pixel lane%32 of pixel group fm. The fused kinds load z in
    // that layout (every load issued before the first use) and scale by g(z)
    // in fp32; each value is rounded once to fp16. The fp16 results then pass
    // through the LDS stage of the slice just computed (no request targets it
    // until the next slice's barrier): each wave writes a block of 32 pixels x
    // TN channels and reads it back as whole 16-byte chunks, so that one store
    // instruction covers 64/CH pixels x TN*2 contiguous bytes instead of 32
    // scattered 16-byte pieces. Chunk q of staged row p sits at position
    // q ^ ((p >> 1) % CH).
    constexpr int CH = TN / 8;            // 16-byte chunks per staged pixel row
    constexpr int EROW = TN * 2;          // bytes per staged pixel row
    constexpr int EBLK = 32 * EROW;       // bytes per wave per pixel group
    constexpr int PPI = 64 / CH;          // pixels per store instruction
    constexpr int EST = 32 / PPI;         // store instructions per pixel group
    static_assert(NW * EBLK <= STAGE, "the staging blocks fit in one stage");
    static_assert(CH >= 2 && CH <= 64 && 64 % CH == 0, "whole pixel rows per store");
    constexpr int kEpiStores = FM * EST;     // stores of one epilogue (per wave)
    // launches with zero phases are mostly stores: their dx goes out with the
    // system-scope policy, the others' with the non-temporal hint
    constexpr int kEpiPolicy = (MODE == kCompanion || MODE == kZeroWork) ? kStoreSystem : kStoreNT;
    static_assert(LD + 2 * kMaxZeroPerSlice + kEpiStores < 64, "vmcnt range");
    auto epilogue = [&](auto tag, const Tile& t, const PhaseArg& ph, int stage) {
        constexpr int E = decltype(tag)::value;
        const auto* ka = kernargs();
        const __amdgpu_buffer_rsrc_t e_dx = make_rsrc(ka->dx, ka->dx_bytes);
        const __amdgpu_buffer_rsrc_t z_rsrc = make_rsrc(E != kEpiNone ? ka->z : ka->dx, ka->dx_bytes);
        const int cw = t.c0 + wn * TN;    // first channel of this wave's block
        u32x2 zr[FM][FN][4];
        if constexpr (E != kEpiNone) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int m = t.m0 + wm * TM + fm * 32 + (lane & 31);
                const uint32_t pix = pixel_offset(ph, m);
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
        lds_char* blk = (lds_char*)lds + stage * STAGE + wave * EBLK;
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
                const int m = t.m0 + wm * TM + fm * 32 + pr;
                const int c = cw + q * 8;
                const uint32_t bad = (uint32_t)(m >= ph.M) | (uint32_t)(c >= C);
                const uint32_t off = (pixel_offset(ph, m) + (uint32_t)c) * 2u;
                __builtin_amdgcn_raw_buffer_store_b128(v, e_dx, out_of_range_if(bad, off), 0, kEpiPolicy);
                const u32x4 zero{0u, 0u, 0u, 0u};
                for (int qc = 0; qc < ncomp; ++qc)   // companion zero pixels (same lattice point)
                    __builtin_amdgcn_raw_buffer_store_b128(zero, e_dx, out_of_range_if(bad, off + (uint32_t)a.comp_delta[qc] * 2u), 0, kEpiPolicy);
            }
        }
    };

    // ---- stream-K fix-up for a share of a split tile. The share's fp32
    // partial sums go to workspace slot [tile][segment] in register order
    // (16-byte group q of thread tid at float offset (q*NT + tid)*4), and the
    // tile's counter counts the arrival. The last share to arrive (no share
    // ever waits for another) adds all shares in segment order, its own from
    // registers, leaves the sum in acc, resets the counter and returns true.
    // A share that finds every other share already arrived is the last one
    // without writing its own partial sums (nor arriving).
    // The workspace is the caller's device memory; every access to it is
    // system-scope (sc0 sc1), so neither side needs an L2 writeback or
    // invalidate across the XCDs' separate L2 caches: a share's stores have
    // reached memory once its vmcnt drains, which precedes its arrival on the
    // counter.
    auto sk_fixup = [&](int tile, const Tile& t, int stage) -> bool {
        constexpr int NQ = FN * FM * 4;   // 16-byte groups of accumulators per thread
        constexpr int QB = NQ < 8 ? NQ : 8;   // groups summed per pass (loads in flight per thread)
        constexpr int kSys = 17;          // cache policy sc0 sc1
        static_assert(NQ % QB == 0, "accumulator groups per pass");
        const uint32_t first = sk_owner((uint32_t)t.s0);
        const int seg = (int)((uint32_t)slot - first);
        const int nseg = (int)(sk_owner((uint32_t)(t.s0 + t.niter - 1)) - first) + 1;
        constexpr uint32_t kSegBytes = (uint32_t)BM * BN * 4;
        const auto* ka = kernargs();
        int* const count = ka->sk_count + tile;
        const __amdgpu_buffer_rsrc_t ws =
            make_rsrc(ka->sk_part + (size_t)tile * (size_t)ka->sk_maxseg * (size_t)(BM * BN), (uint32_t)ka->sk_maxseg * kSegBytes);
        const uint32_t lane_off = (uint32_t)tid * 16u;
        __attribute__((address_space(3))) int* flag = (__attribute__((address_space(3))) int*)((lds_char*)lds + stage * STAGE);
        __syncthreads();                  // no wave reads the stage's operands any more
        if (tid == 0)
            *flag = __hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nseg - 1 ? 1 : 0;
        __syncthreads();
        // one value for the whole workgroup: taken from the first lane so the
        // branches below are uniform in the compiler's eyes too
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
                                                               (uint32_t)seg * kSegBytes + (uint32_t)(g * NT) * 16u + lane_off, 0, kSys);
                    }
            wait_vmcnt<0>();              // this wave's partial sums are in memory
            __syncthreads();              // ... and every wave's; every wave has read the flag
            if (tid == 0) {
                const int old = __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                *flag = old == nseg - 1 ? 1 : 0;
            }
            __syncthreads();
            if (__builtin_amdgcn_readfirstlane(*flag) == 0)
                return false;
        }
#pragma unroll
        for (int g0 = 0; g0 < NQ; g0 += QB) {
            float4_t sum[QB];
#pragma unroll
            for (int u = 0; u < QB; ++u)
                sum[u] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            for (int sg = 0; sg < nseg; ++sg) {
                float4_t v[QB];
                if (sg == seg) {
#pragma unroll
                    for (int u = 0; u < QB; ++u) {
                        const int g = g0 + u, fn = g / (FM * 4), fm = (g / 4) % FM, q = g % 4;
                        v[u] = float4_t{acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2], acc[fn][fm][4 * q + 3]};
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < QB; ++u)
                        v[u] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                ws, (uint32_t)sg * kSegBytes + (uint32_t)((g0 + u) * NT) * 16u + lane_off, 0, kSys));
                }
#pragma unroll
                for (int u = 0; u < QB; ++u)
                    sum[u] += v[u];
            }
#pragma unroll
            for (int u = 0; u < QB; ++u) {
                const int g = g0 + u, fn = g / (FM * 4), fm = (g / 4) % FM, q = g % 4;
                acc[fn][fm][4 * q] = sum[u][0];
                acc[fn][fm][4 * q + 1] = sum[u][1];
                acc[fn][fm][4 * q + 2] = sum[u][2];
                acc[fn][fm][4 * q + 3] = sum[u][3];
            }
        }
        if (tid == 0)
            __hip_atomic_store(count, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    };

    // ---- the walk. The k-th slice of the stream lives in LDS stage k % 3:
    // rbuf is the stage of the next request, cbuf that of the next slice to
    // compute; requests run two slices ahead.
    int rbuf = 0, cbuf = 0, inflight = 0;   // inflight: slices requested, not yet computed
    int post_epi = 0;                        // slices left whose loads precede the last epilogue
    if (request_next(rbuf)) {
        rbuf = 1;
        ++inflight;
    }
    if (request_next(rbuf)) {
        rbuf = 2;
        ++inflight;
    }
    const int epi = a.epi;
    for (int round = 0;; ++round) {
        Tile t;
        Seg g;
        if constexpr (SK) {
            g = segment(round, t);
            if (!g.ok)
                break;
        } else if constexpr (ZW) {
            const int tile = round * G + slot;
            if (tile >= a.total_tiles)
                break;
            if (tile >= a.gemm_tiles) {   // a chunk of zero stripes (no request is in flight any more)
                const uint32_t first = a.zabsorbed + (uint32_t)(tile - a.gemm_tiles) * kZeroChunkStripes;
#pragma unroll
                for (int u = 0; u < kZeroChunkStripes; ++u)
                    zero_stripe(first + u, first + u < a.zstripes);
                continue;
            }
            t = decode(tile, round);
            g = Seg{tile, 0, t.niter, true};
        } else {
            const int tile = round * G + slot;
            if (tile >= a.gemm_tiles)
                break;
            t = decode(tile, round);
            g = Seg{tile, 0, t.niter, true};
        }
        const PhaseArg& ph = a.ph[t.pi];

#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[fn][fm][e] = 0.0f;
        for (int it = g.lo; it < g.hi; ++it) {
            // This slice must have landed. Memory operations complete in issue
            // order, and after its last load came its zps zero stores, the
            // next request (LD loads, zps stores) when it was issued, and, in
            // the first two slices after an epilogue, that epilogue's kEpiStores
            // stores (its z loads only make the wait stricter).
            if (inflight >= 2) {
                if (ZW && zps != 0) {
                    if (post_epi > 0)
                        wait_vmcnt<LD + 2 * kMaxZeroPerSlice + kEpiStores>();
                    else
                        wait_vmcnt<LD + 2 * kMaxZeroPerSlice>();
                } else {
                    if (post_epi > 0)
                        wait_vmcnt<LD + kEpiStores>();
                    else
                        wait_vmcnt<LD>();
                }
            } else {
                wait_vmcnt<0>();
            }
            post_epi = post_epi > 0 ? post_epi - 1 : 0;
            __syncthreads();     // every wave's part of the slice is in LDS, and every
                                 // wave is done with the stage the next request reuses
            const bool more = prepare_next(rbuf);
            compute(cbuf, more);
            if (more) {
                finish_request();
                rbuf = rbuf == 2 ? 0 : rbuf + 1;
            } else {
                --inflight;
            }
            cbuf = cbuf == 2 ? 0 : cbuf + 1;
        }

        // ---- epilogue (one specialisation per kind; the kind is uniform),
        // staged through the stage of the slice just computed. The two slices
        // in flight were requested before it. A share of a split tile first
        // leaves its partial sums; only the share that completes the tile goes on.
        const int sdone = cbuf == 0 ? 2 : cbuf - 1;
        post_epi = 2;
        if constexpr (SK) {
            if ((g.lo != 0 || g.hi != t.niter) && !sk_fixup(g.tile, t, sdone))
                continue;
        }
        switch (epi) {
        case kEpiDRelu: epilogue(EpiTag<kEpiDRelu>{}, t, ph, sdone); break;
        case kEpiDHardswish: epilogue(EpiTag<kEpiDHardswish>{}, t, ph, sdone); break;
        default: epilogue(EpiTag<kEpiNone>{}, t, ph, sdone); break;
        }
    }
}

// A stream-K variant exists for every configuration but 256x64/4x1, whose
// uniform state does not fit the scalar register file once the fix-up is added.
template <int BM, int BN, int WM, int WN>
constexpr bool kHasStreamK = !(BM == 256 && BN == 64 && WM == 4);

// The variant a launch needs (the host never asks 256x64/4x1 to split).
inline int launch_mode(const KernelArgs& a)
{
    if (a.sk)
        return kStreamK;
    if (a.total_tiles > a.gemm_tiles || a.zstripes > 0)
        return kZeroWork;
    return a.ncomp > 0 ? kCompanion : kPlain;
}

template <int BM, int BN, int WM, int WN>
hipError_t launch(const KernelArgs& a, hipStream_t stream)
{
    const dim3 grid(a.grid), block(64 * WM * WN);
    switch (launch_mode(a)) {
    case kStreamK:
        if constexpr (kHasStreamK<BM, BN, WM, WN>) {
            hipLaunchKernelGGL((dgrad_igemm<BM, BN, WM, WN, kStreamK>), grid, block, 0, stream, a);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;   // the host never plans this
    case kZeroWork:
        hipLaunchKernelGGL((dgrad_igemm<BM, BN, WM, WN, kZeroWork>), grid, block, 0, stream, a);
        return hipGetLastError();
    case kCompanion:
        hipLaunchKernelGGL((dgrad_igemm<BM, BN, WM, WN, kCompanion>), grid, block, 0, stream, a);
        return hipGetLastError();
    default:
        hipLaunchKernelGGL((dgrad_igemm<BM, BN, WM, WN, kPlain>), grid, block, 0, stream, a);
        return hipGetLastError();
    }
}

// Resident workgroups of one configuration per CU on the current device: the
// fewest over its variants (a launch's grid assumes that many are resident).
template <int BM, int BN, int WM, int WN>
int resident(void)
{
    auto blocks = [](const void* f) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 64 * WM * WN, 0) != hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        return n;
    };
    int n = std::min(blocks(reinterpret_cast<const void*>(dgrad_igemm<BM, BN, WM, WN, kPlain>)),
                     blocks(reinterpret_cast<const void*>(dgrad_igemm<BM, BN, WM, WN, kZeroWork>)));
    n = std::min(n, blocks(reinterpret_cast<const void*>(dgrad_igemm<BM, BN, WM, WN, kCompanion>)));
    if constexpr (kHasStreamK<BM, BN, WM, WN>)
        n = std::min(n, blocks(reinterpret_cast<const void*>(dgrad_igemm<BM, BN, WM, WN, kStreamK>)));
    return n > 0 ? n : 1;
}

// The compiled tile configurations: (BM, BN, WM, WN).
#define CBW_TILE_CONFIGS(X) \
    X(128, 128, 2, 2)       \
    X(256, 64, 4, 1)        \
    X(128, 64, 2, 2)        \
    X(64, 64, 2, 2)         \
    X(256, 128, 4, 2)       \
    X(128, 256, 2, 4)

#define CBW_CONFIG_ENTRY(BM, BN, WM, WN) \
    {BM, BN, 64, WM, WN, #BM "x" #BN "x64/" #WM "x" #WN, 3 * (BM + BN) * 64 * 2, kHasStreamK<BM, BN, WM, WN>, \
     kHasPhaseOrder<BM, BN, WM, WN>, false, false},
const TileConfig kConfigs[] = {CBW_TILE_CONFIGS(CBW_CONFIG_ENTRY)};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
static_assert(kNumConfigs <= 64, "the launcher keeps per-config state for at most 64 configs");

// Private (scratch) bytes per lane, summed over the configuration's variants,
// or -1 if the runtime cannot tell.
template <int BM, int BN, int WM, int WN>
int private_bytes(void)
{
    auto bytes = [](const void* f) -> long {
        hipFuncAttributes attr;
        if (hipFuncGetAttributes(&attr, f) != hipSuccess) {
            (void)hipGetLastError();
            return -1;
        }
        return (long)attr.localSizeBytes;
    };
    long b[4] = {bytes(reinterpret_cast<const void*>(dgrad_igemm<BM, BN, WM, WN, kPlain>)),
                 bytes(reinterpret_cast<const void*>(dgrad_igemm<BM, BN, WM, WN, kZeroWork>)),
                 bytes(reinterpret_cast<const void*>(dgrad_igemm<BM, BN, WM, WN, kCompanion>)), 0};
    if constexpr (kHasStreamK<BM, BN, WM, WN>)
        b[3] = bytes(reinterpret_cast<const void*>(dgrad_igemm<BM, BN, WM, WN, kStreamK>));
    if (b[0] < 0 || b[1] < 0 || b[2] < 0 || b[3] < 0)
        return -1;
    return (int)(b[0] + b[1] + b[2] + b[3]);
}

using LaunchFn = hipError_t (*)(const KernelArgs&, hipStream_t);
using ResidentFn = int (*)(void);
#define CBW_LAUNCH_ENTRY(BM, BN, WM, WN) &launch<BM, BN, WM, WN>,
#define CBW_RESIDENT_ENTRY(BM, BN, WM, WN) &resident<BM, BN, WM, WN>,
#define CBW_PRIVATE_ENTRY(BM, BN, WM, WN) &private_bytes<BM, BN, WM, WN>,
const LaunchFn kLaunch[] = {CBW_TILE_CONFIGS(CBW_LAUNCH_ENTRY)};
const ResidentFn kResident[] = {CBW_TILE_CONFIGS(CBW_RESIDENT_ENTRY)};
const ResidentFn kPrivate[] = {CBW_TILE_CONFIGS(CBW_PRIVATE_ENTRY)};

}  // namespace

// Configuration ids: dgrad_igemm's first, then dgrad_wide's, dgrad_halo's,
// dgrad_pgemm's, dgrad_halo1's and dgrad_pwide's. `kind` returns which table
// id falls in, and the index there.
namespace {
int kind(int id, int& i)
{
    i = id;
    if (i < kNumConfigs)
        return 0;
    i -= kNumConfigs;
    if (i < wide_num_configs())
        return 1;
    i -= wide_num_configs();
    if (i < halo_num_configs())
        return 2;
    i -= halo_num_configs();
    if (i < pgemm_num_configs())
        return 3;
    i -= pgemm_num_configs();
    if (i < halo1_num_configs())
        return 4;
    i -= halo1_num_configs();
    return 5;
}
}  // namespace

int num_tile_configs()
{
    return kNumConfigs + wide_num_configs() + halo_num_configs() + pgemm_num_configs() + halo1_num_configs() +
           pwide_num_configs();
}

const TileConfig& tile_config(int id)
{
    int i = 0;
    switch (kind(id, i)) {
    case 0: return kConfigs[i];
    case 1: return wide_config(i);
    case 2: return halo_config(i);
    case 3: return pgemm_config(i);
    case 4: return halo1_config(i);
    default: return pwide_config(i);
    }
}

bool tile_config_admits(int id, int R, int S, int stride, int pad, int H, int W, int P, int Q, int K, int epi)
{
    int i = 0;
    switch (kind(id, i)) {
    case 2: return halo_admits(i, R, S, stride, pad, H, W, P, Q);
    case 3: return pgemm_admits(i, R, S, stride, pad, K, epi);
    case 4: return halo1_admits(i, R, S, stride, pad, H, W, P, Q, K, epi);
    case 5: return pwide_admits(i, R, S, stride, epi);
    default: return true;
    }
}

bool tile_config_runs(int id, const KernelArgs& a)
{
    int i = 0;
    const int kd = kind(id, i);
    return kd == 4 ? halo1_runs_launch(i, a) : kd == 5 ? pwide_runs_launch(i, a) : true;
}

int plain_fallback(int id)
{
    const TileConfig& tc = tile_config(id);
    if (!tc.plain_only && !tc.restricted)
        return id;
    int best = 0;
    for (int i = 0; i < kNumConfigs; ++i)
        if (kConfigs[i].BM == tc.BM && kConfigs[i].BN == tc.BN)
            best = i;
    return best;
}

int blocks_per_cu(int id)
{
    int i = 0;
    switch (kind(id, i)) {
    case 0: return id >= 0 ? kResident[i]() : 1;
    case 1: return wide_blocks_per_cu(i);
    case 2: return halo_blocks_per_cu(i);
    case 3: return pgemm_blocks_per_cu(i);
    case 4: return halo1_blocks_per_cu(i);
    default: return pwide_blocks_per_cu(i);
    }
}

int kernel_private_bytes(int id)
{
    int i = 0;
    switch (kind(id, i)) {
    case 0: return id >= 0 ? kPrivate[i]() : -1;
    case 1: return wide_private_bytes(i);
    case 2: return halo_private_bytes(i);
    case 3: return pgemm_private_bytes(i);
    case 4: return halo1_private_bytes(i);
    default: return pwide_private_bytes(i);
    }
}

hipError_t launch_tile_config(int id, const KernelArgs& a, hipStream_t stream)
{
    if (id < 0 || id >= num_tile_configs())
        return hipErrorInvalidValue;
    int i = 0;
    switch (kind(id, i)) {
    case 0: return kLaunch[i](a, stream);
    case 1: return launch_wide(i, a, stream);
    case 2: return launch_halo(i, a, stream);
    case 3: return launch_pgemm(i, a, stream);
    case 4: return launch_halo1(i, a, stream);
    default: return launch_pwide(i, a, stream);
    }
}

// ============================================================ zero fill
//
// 16-byte zero stores over a buffer, one per thread in a grid-stride loop
// (plain stores: the lines stay in the caches). Used to clear the no-
// allocation scratch's counter area and, in the profiler, to push a layer's
// operands out of the caches before a timed launch.

namespace {

__global__ void __launch_bounds__(256) fill_zero(u32x4* p, uint64_t n16)
{
    const u32x4 zero{0u, 0u, 0u, 0u};
    for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < n16; i += (uint64_t)gridDim.x * 256u)
        p[i] = zero;
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream)
{
    if (p == nullptr || ((uintptr_t)p & 15u) || (bytes & 15u))
        return hipErrorInvalidValue;
    const uint64_t n16 = bytes / 16;
    if (n16 == 0)
        return hipSuccess;
    const uint64_t blocks = std::min<uint64_t>((n16 + 255) / 256, 8192);
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, (u32x4*)p, n16);
    return hipGetLastError();
}

// ============================================================ no-allocation scratch
//
// The device memory of conv2d_dgrad_nhwc_noalloc, for callers that cannot
// allocate: one static array per device, laid out like a caller's workspace
// (arrival counters, then partial sums). Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol); it
// passes the device address that hipGetSymbolAddress returned for the current
// device, kept per device from the first use on.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_addr;   // device -> address of its copy of `scratch`
}  // namespace

hipError_t noalloc_scratch(void** ptr, hipStream_t stream)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_addr.find(dev);
    if (it != g_scratch_addr.end()) {
        *ptr = it->second;
        return hipSuccess;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return e;
    if (p == nullptr || ((uintptr_t)p & 255u))
        return hipErrorInvalidSymbol;
    // the counters must start at zero (every launch leaves them so after that)
    e = launch_fill_zero(p, kCounterBytes, stream);
    if (e != hipSuccess)
        return e;
    g_scratch_addr[dev] = p;
    *ptr = p;
    return hipSuccess;
}

// ===================================================================== wgrad
//
// The filter gradient of the same layer,
//   dw[k,r,t,c] = sum over pixels m = (n,p,q) of dy[m,k] * x[n, p*s-pad+r, q*s-pad+t, c],
// as one GEMM per tap (r,t): D[c][k] = sum_m x_tap[m][c] * dy[m][k], with A =
// x_tap^T (rows = channels c) and B = dy (columns = output channels k). The
// reduction runs over the N*P*Q pixels in slices of 64; both slices are
// [64 pixels][channels] tiles in LDS, loaded row by row straight from HBM
// like the dgrad filter slice, and both fragments (8 consecutive pixels of
// one channel) come from transpose reads. A launch covers tiles x splits
// workgroups: workgroup b runs tile b mod tiles over the b / tiles-th of the
// launch's contiguous slice ranges, and writes its fp32 accumulators to the
// partial buffer in register order; a second kernel adds the splits in order.

namespace {

template <int BC, int BK, int WC, int WK>
__global__ void __launch_bounds__(64 * WC * WK) wgrad_igemm(WgradArgs a)
{
    constexpr int BR = 64;                        // pixels per slice
    constexpr int NW = WC * WK;
    constexpr int NT = 64 * NW;
    constexpr int TC = BC / WC, TK = BK / WK;     // wave tile: TC channels x TK output channels
    constexpr int FN = TC / 32, FM = TK / 32;
    constexpr int XROW = BC * 2, DROW = BK * 2;   // bytes of one pixel row of each slice
    constexpr int X_BYTES = BR * XROW, D_BYTES = BR * DROW;
    constexpr int STAGE = X_BYTES + D_BYTES;
    constexpr int X_INSTR = X_BYTES / 1024 / NW, D_INSTR = D_BYTES / 1024 / NW;
    constexpr int LD = X_INSTR + D_INSTR;         // loads per lane per slice
    constexpr int XCH = XROW / 16, DCH = DROW / 16;   // 16-byte chunks per row
    static_assert(TC % 32 == 0 && TK % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(X_BYTES % (1024 * NW) == 0 && D_BYTES % (1024 * NW) == 0, "whole 1 KiB blocks per wave");
    static_assert(XROW % 256 == 0 && DROW % 256 == 0, "rows of whole bank windows");
    static_assert(3 * STAGE <= 160 * 1024, "LDS budget");
    static_assert(2 * LD < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char lds[3 * STAGE];
    const uint32_t lds_u32 = (uint32_t)(uintptr_t)((lds_char*)lds);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wc = wave % WC;
    const int wk = wave / WC;

    const int tiles = pin(a.tiles);
    const int tile = pin((int)(blockIdx.x % (uint32_t)tiles));
    const int split = pin((int)(blockIdx.x / (uint32_t)tiles));
    const int kb = tile % a.tiles_k;
    const int rest = tile / a.tiles_k;
    const int cb = rest % a.tiles_c;
    const int tap = rest / a.tiles_c;
    const int r = tap / a.S;
    const int t = tap - r * a.S;
    const int c0 = pin(cb * BC);
    const int k0 = pin(kb * BK);
    const int C = pin(a.C);
    const int K = pin(a.K);
    const int npq = pin(a.npq);
    const int s_begin = pin((int)(((int64_t)split * a.slices) / a.splits));
    const int s_end = pin((int)(((int64_t)(split + 1) * a.slices) / a.splits));
    const int ns = s_end - s_begin;

    const i32x4 x_desc = raw_descriptor(a.x, a.x_bytes);
    const i32x4 dy_desc = raw_descriptor(a.dy, a.dy_bytes);

    // Lane geometry of the loads. Block b = j*NW + wave of a slice covers
    // 1024/ROW consecutive pixel rows; lane l fills row b*(1024/ROW) + l/CH at
    // chunk position l % CH, which holds logical chunk (l % CH) ^ w_swizzle(row).
    int x_row[X_INSTR], d_row[D_INSTR];
    uint32_t x_c[X_INSTR];                // element offset of the lane's chunk within a row (c0 included)
    uint32_t d_off[D_INSTR];              // byte offset of the lane's dy chunk within a pixel row (k0 included)
    bool x_cok[X_INSTR], d_kok[D_INSTR];  // the chunk lies inside C / K
#pragma unroll
    for (int j = 0; j < X_INSTR; ++j) {
        const int b = j * NW + wave;
        x_row[j] = b * (1024 / XROW) + lane / XCH;
        const int chunk = (lane % XCH) ^ w_swizzle<XROW>(x_row[j]);
        x_c[j] = (uint32_t)(c0 + chunk * 8);
        x_cok[j] = c0 + chunk * 8 < C;
    }
#pragma unroll
    for (int j = 0; j < D_INSTR; ++j) {
        const int b = j * NW + wave;
        d_row[j] = b * (1024 / DROW) + lane / DCH;
        const int chunk = (lane % DCH) ^ w_swizzle<DROW>(d_row[j]);
        d_off[j] = (uint32_t)(k0 + chunk * 8) * 2u;
        d_kok[j] = k0 + chunk * 8 < K;
    }
    const int Hh = a.H, Ww = a.W, str = a.stride, pad = a.pad;
    // Issue the loads of slice si into LDS stage st.
    auto issue = [&](int si, int st) {
        const int m0 = si * BR;
        const uint32_t base = lds_u32 + (uint32_t)(st * STAGE);
#pragma unroll
        for (int j = 0; j < X_INSTR; ++j) {
            const int m = m0 + x_row[j];
            const uint32_t n = fastdiv((uint32_t)m, a.div_pq);
            const uint32_t rem = (uint32_t)m - n * a.div_pq.d;
            const uint32_t p = fastdiv(rem, a.div_q);
            const uint32_t q = rem - p * a.div_q.d;
            const int h = (int)p * str - pad + r;
            const int w = (int)q * str - pad + t;
            const bool ok = x_cok[j] & (m < npq) & ((unsigned)h < (unsigned)Hh) & ((unsigned)w < (unsigned)Ww);
            const uint32_t off = ((((n * (uint32_t)Hh + (uint32_t)h) * (uint32_t)Ww + (uint32_t)w) * (uint32_t)C) + x_c[j]) * 2u;
            dma16(x_desc, ok ? off : 0x80000000u, 0u, base + (uint32_t)((j * NW + wave) * 1024));
        }
#pragma unroll
        for (int j = 0; j < D_INSTR; ++j) {
            const int m = m0 + d_row[j];
            const bool ok = d_kok[j] & (m < npq);
            dma16(dy_desc, ok ? (uint32_t)m * (uint32_t)K * 2u + d_off[j] : 0x80000000u, 0u,
                  base + (uint32_t)(X_BYTES + (j * NW + wave) * 1024));
        }
    };

    // Fragment addresses (bytes within a stage, sub-step 0): 32 columns of a
    // [64 pixels][ROW] slice starting at column `col0`; group g = lane/16
    // covers columns +16*(g&1), pixels +8*(g>>1); within it lane 4r+q reads
    // pixel row r, columns 4q..4q+3 (two transpose reads give 8 pixels).
    const int g = (lane >> 4) & 3;
    const int rr = (lane & 15) >> 2;
    const int qq = lane & 3;
    const int prow = (g >> 1) * 8 + rr;
    int xa[FN], db[FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int cl = wc * TC + fn * 32 + (g & 1) * 16 + 4 * qq;
        xa[fn] = prow * XROW + (((cl >> 3) ^ w_swizzle<XROW>(prow)) * 16) + (cl & 7) * 2;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int kl = wk * TK + fm * 32 + (g & 1) * 16 + 4 * qq;
        db[fm] = X_BYTES + prow * DROW + (((kl >> 3) ^ w_swizzle<DROW>(prow)) * 16) + (kl & 7) * 2;
    }
    auto tr8 = [&](const lds_char* p, int row_bytes) -> half8_t {
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)p);
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p + 4 * row_bytes));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(half8_t, u32x4{l2.x, l2.y, h2.x, h2.y});
    };

    float16_t acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[fn][fm][e] = 0.0f;

    auto compute = [&](int st) {
        const lds_char* sb = (const lds_char*)lds + st * STAGE;
#pragma unroll
        for (int kk = 0; kk < BR / 16; ++kk) {
            half8_t af[FN], bf[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                af[fn] = tr8(sb + xa[fn] + kk * 16 * XROW, XROW);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                bf[fm] = tr8(sb + db[fm] + kk * 16 * DROW, DROW);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[fn], bf[fm], acc[fn][fm], 0, 0, 0);
        }
    };

    // The slice stream: requests run two slices ahead in a ring of three
    // stages. Loads complete in issue order, so the wait for slice i allows
    // exactly the LD loads of slice i+1 when those were issued.
    if (ns > 0)
        issue(s_begin, 0);
    if (ns > 1)
        issue(s_begin + 1, 1);
    for (int i = 0; i < ns; ++i) {
        if (i + 1 < ns)
            wait_vmcnt<LD>();
        else
            wait_vmcnt<0>();
        __syncthreads();        // every wave's part of slice i is in LDS, and every wave
                                // is done with the stage the next request reuses
        if (i + 2 < ns)
            issue(s_begin + i + 2, (i + 2) % 3);
        compute(i % 3);
    }

    // One split without a partial buffer: the sums are dw itself. A lane holds
    // channels 8*q + 4*(lane/32) .. +3 of output channel lane % 32 in each
    // 32x32 block (the mapping wgrad_reduce applies).
    if (a.part == nullptr) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = c0 + wc * TC + fn * 32 + 8 * q + 4 * (lane >> 5);
                    const int k = k0 + wk * TK + fm * 32 + (lane & 31);
                    if (c < C && k < K)   // C % 8 == 0: the 4 channels are all inside or all outside
                        *(float4_t*)(a.dw + ((size_t)k * (size_t)(a.R * a.S) + (size_t)tap) * (size_t)C + (size_t)c) =
                            float4_t{acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                                     acc[fn][fm][4 * q + 3]};
                }
        return;
    }
    // partial sums in register order: 16-byte group q of thread tid at float
    // offset (q*NT + tid)*4 of this (split, tile) block
    float* out = a.part + ((size_t)split * (size_t)tiles + (size_t)tile) * (size_t)(BC * BK);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gi = (fn * FM + fm) * 4 + q;
                *(float4_t*)(out + (size_t)(gi * NT + tid) * 4) =
                    float4_t{acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2], acc[fn][fm][4 * q + 3]};
            }
}

// dw from the partial sums: one thread per 16-byte group of one tile; the
// splits are added in order (so the result does not depend on timing), and
// the group is mapped back to its 4 channels and output channel. In the
// 32x32 accumulator block a lane holds rows 8*q + 4*(lane/32) .. +3 (here
// channels) of column lane % 32 (here the output channel).
template <int BC, int BK, int WC, int WK>
__global__ void __launch_bounds__(256) wgrad_reduce(WgradArgs a)
{
    constexpr int NW = WC * WK;
    constexpr int NT = 64 * NW;
    constexpr int TC = BC / WC, TK = BK / WK;
    constexpr int FM = TK / 32;
    constexpr int GROUPS = BC * BK / 4;           // 16-byte groups per tile
    const uint32_t u = blockIdx.x * 256u + threadIdx.x;
    if (u >= (uint32_t)a.tiles * (uint32_t)GROUPS)
        return;
    const int tile = (int)(u / GROUPS);
    const int gq = (int)(u % GROUPS);
    // eight loads in flight at a time; the adds stay in split order
    const float* src = a.part + ((size_t)tile * (size_t)GROUPS + (size_t)gq) * 4;
    const size_t split_stride = (size_t)a.tiles * (size_t)GROUPS * 4;
    float4_t sum{0.0f, 0.0f, 0.0f, 0.0f};
    int sp = 0;
    for (; sp + 8 <= a.splits; sp += 8) {
        float4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = *(const float4_t*)(src + (size_t)(sp + u) * split_stride);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            sum += v[u];
    }
    for (; sp < a.splits; ++sp)
        sum += *(const float4_t*)(src + (size_t)sp * split_stride);
    const int gi = gq / NT;
    const int th = gq % NT;
    const int wave = th / 64, lane = th % 64;
    const int wc = wave % WC, wk = wave / WC;
    const int fn = gi / (FM * 4), fm = (gi / 4) % FM, q = gi % 4;
    const int kb = tile % a.tiles_k;
    const int rest = tile / a.tiles_k;
    const int cb = rest % a.tiles_c;
    const int tap = rest / a.tiles_c;
    const int c = cb * BC + wc * TC + fn * 32 + 8 * q + 4 * (lane >> 5);
    const int k = kb * BK + wk * TK + fm * 32 + (lane & 31);
    if (c < a.C && k < a.K)   // C is a multiple of 8: the 4 channels are all inside or all outside
        *(float4_t*)(a.dw + ((size_t)k * (size_t)(a.R * a.S) + (size_t)tap) * (size_t)a.C + (size_t)c) = sum;
}

// The compiled wgrad tile configurations: (BC, BK, WC, WK).
#define CBW_WGRAD_CONFIGS(X) \
    X(128, 128, 2, 4)        \
    X(256, 128, 4, 2)

#define CBW_WGRAD_ENTRY(BC, BK, WC, WK) {BC, BK, WC, WK, #BC "x" #BK "/" #WC "x" #WK},
const WgradConfig kWgradConfigs[] = {CBW_WGRAD_CONFIGS(CBW_WGRAD_ENTRY)};
constexpr int kNumWgradConfigs = sizeof(kWgradConfigs) / sizeof(kWgradConfigs[0]);

template <int BC, int BK, int WC, int WK>
hipError_t wgrad_launch(const WgradArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((wgrad_igemm<BC, BK, WC, WK>), dim3(a.tiles * a.splits), dim3(64 * WC * WK), 0, stream, a);
    return hipGetLastError();
}

template <int BC, int BK, int WC, int WK>
hipError_t wgrad_reduce_launch(const WgradArgs& a, hipStream_t stream)
{
    const uint32_t groups = (uint32_t)a.tiles * (uint32_t)(BC * BK / 4);
    hipLaunchKernelGGL((wgrad_reduce<BC, BK, WC, WK>), dim3((groups + 255) / 256), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int BC, int BK, int WC, int WK>
int wgrad_private(void)
{
    hipFuncAttributes a1, a2;
    if (hipFuncGetAttributes(&a1, reinterpret_cast<const void*>(wgrad_igemm<BC, BK, WC, WK>)) != hipSuccess ||
        hipFuncGetAttributes(&a2, reinterpret_cast<const void*>(wgrad_reduce<BC, BK, WC, WK>)) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return (int)(a1.localSizeBytes + a2.localSizeBytes);
}

using WgradLaunchFn = hipError_t (*)(const WgradArgs&, hipStream_t);
#define CBW_WGRAD_LAUNCH(BC, BK, WC, WK) &wgrad_launch<BC, BK, WC, WK>,
#define CBW_WGRAD_REDUCE(BC, BK, WC, WK) &wgrad_reduce_launch<BC, BK, WC, WK>,
#define CBW_WGRAD_PRIVATE(BC, BK, WC, WK) &wgrad_private<BC, BK, WC, WK>,
const WgradLaunchFn kWgradLaunch[] = {CBW_WGRAD_CONFIGS(CBW_WGRAD_LAUNCH)};
const WgradLaunchFn kWgradReduce[] = {CBW_WGRAD_CONFIGS(CBW_WGRAD_REDUCE)};
int (*const kWgradPrivate[])(void) = {CBW_WGRAD_CONFIGS(CBW_WGRAD_PRIVATE)};

}  // namespace

int wgrad_num_configs() { return kNumWgradConfigs; }

const WgradConfig& wgrad_config(int id) { return kWgradConfigs[id]; }

hipError_t launch_wgrad(int id, const WgradArgs& a, hipStream_t stream)
{
    if (id < 0 || id >= kNumWgradConfigs)
        return hipErrorInvalidValue;
    return kWgradLaunch[id](a, stream);
}

hipError_t launch_wgrad_reduce(int id, const WgradArgs& a, hipStream_t stream)
{
    if (id < 0 || id >= kNumWgradConfigs)
        return hipErrorInvalidValue;
    return kWgradReduce[id](a, stream);
}

int wgrad_private_bytes(int id)
{
    return (id >= 0 && id < kNumWgradConfigs) ? kWgradPrivate[id]() : -1;
}

// ================================================================== forward
//
// The forward layer with the fused bias + activation epilogue:
//   z[m,k] = bias[k] + sum over taps (r,t) and c of x[n, p*s-pad+r, q*s-pad+t, c] * w[k,r,t,c]
//   y[m,k] = hardswish(z) (act 1) or z (act 0), for output pixel m = (n,p,q).
// GEMM D[k][m] with A = w (rows = output channels k, reduction c) and B =
// x_tap^T (columns = output pixels, reduction c). Both slices are
// [rows][64 channels] tiles of 128-byte rows in LDS, loaded like dgrad's dy
// slice, and both fragments are single ds_read_b128 (8 consecutive c of one
// row). Slices go tap by tap and, within a tap, over C in 64-wide steps; a
// lane's x offset and padding check change only at tap boundaries.

namespace {

// hardswish(z) = z * min(max(z + 3, 0), 6) / 6, in fp32
__device__ inline float hardswish_f(float z)
{
    return z * fminf(fmaxf(z + 3.0f, 0.0f), 6.0f) * (1.0f / 6.0f);
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) fwd_igemm(FwdArgs a)
{
    constexpr int BK = 64;
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;     // wave tile: TM pixels x TN output channels
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int X_BYTES = BM * 128, W_BYTES = BN * 128;
    constexpr int STAGE = X_BYTES + W_BYTES;
    constexpr int X_INSTR = X_BYTES / 1024 / NW, W_INSTR = W_BYTES / 1024 / NW;
    constexpr int LD = X_INSTR + W_INSTR;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(X_BYTES % (1024 * NW) == 0 && W_BYTES % (1024 * NW) == 0, "whole 1 KiB blocks per wave");
    static_assert(3 * STAGE <= 160 * 1024, "LDS budget");
    static_assert(2 * LD < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char lds[3 * STAGE];
    const uint32_t lds_u32 = (uint32_t)(uintptr_t)((lds_char*)lds);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;
    const int wn = wave / WM;

    const int tn_ = pin((int)(blockIdx.x % (uint32_t)a.tiles_n));
    const int tm_ = pin((int)(blockIdx.x / (uint32_t)a.tiles_n));
    const int m0 = pin(tm_ * BM);
    const int n0 = pin(tn_ * BN);
    const int C = pin(a.C);
    const int K = pin(a.K);
    const int Hh = pin(a.H), Ww = pin(a.W);
    const int S = pin(a.S);
    const int csteps = pin(a.csteps);
    const int ns = a.R * S * csteps;
    const i32x4 x_desc = raw_descriptor(a.x, a.x_bytes);
    const i32x4 w_desc = raw_descriptor(a.w, a.w_bytes);

    // Lane geometry: block b = j*NW + wave of a slice covers rows 8b..8b+7;
    // lane l fills row 8b + l/8 at chunk position l%8, holding logical chunk
    // (l%8) ^ dy_swizzle(row).
    uint32_t x_base[X_INSTR];   // element offset of the row's pixel at tap (0,0), modulo 2^32
    int x_h0[X_INSTR], x_w0[X_INSTR];
    int x_ch[X_INSTR];
    uint32_t x_vo[X_INSTR];     // the lane's byte offset for the current tap (2^31: outside)
#pragma unroll
    for (int j = 0; j < X_INSTR; ++j) {
        const int row = (j * NW + wave) * 8 + (lane >> 3);
        x_ch[j] = ((lane & 7) ^ dy_swizzle(row)) * 8;
        const int m = m0 + row;
        const uint32_t n = fastdiv((uint32_t)m, a.div_pq);
        const uint32_t rem = (uint32_t)m - n * a.div_pq.d;
        const uint32_t p = fastdiv(rem, a.div_q);
        const uint32_t q = rem - p * a.div_q.d;
        x_h0[j] = m < a.npq ? (int)p * a.stride - a.pad : -(1 << 24);   // a dead row fails every h >= 0 test
        x_w0[j] = (int)q * a.stride - a.pad;
        x_base[j] = ((n * (uint32_t)Hh + (uint32_t)x_h0[j]) * (uint32_t)Ww + (uint32_t)x_w0[j]) * (uint32_t)C + (uint32_t)x_ch[j];
    }
    uint32_t w_lane[W_INSTR];   // byte offset of the lane's filter chunk at tap (0,0), c0 = 0 (2^31: k >= K)
    int w_ch[W_INSTR];
#pragma unroll
    for (int j = 0; j < W_INSTR; ++j) {
        const int row = (j * NW + wave) * 8 + (lane >> 3);
        w_ch[j] = ((lane & 7) ^ dy_swizzle(row)) * 8;
        const int k = n0 + row;
        w_lane[j] = k < K ? (uint32_t)(k * a.R * S * C + w_ch[j]) * 2u : 0x80000000u;
    }

    // request cursor: tap (r, t) and channel step c0
    int rq_r = 0, rq_t = 0, rq_c0 = 0;
    bool new_tap = true;
    uint32_t w_tap = 0;
    auto issue = [&](int st) {
        if (new_tap) {
            new_tap = false;
            const uint32_t tapoff = (uint32_t)(rq_r * Ww + rq_t) * (uint32_t)C;
#pragma unroll
            for (int j = 0; j < X_INSTR; ++j) {
                const bool ok = ((unsigned)(x_h0[j] + rq_r) < (unsigned)Hh) & ((unsigned)(x_w0[j] + rq_t) < (unsigned)Ww);
                x_vo[j] = ok ? (x_base[j] + tapoff) * 2u : 0x80000000u;
            }
            w_tap = (uint32_t)((rq_r * S + rq_t) * C) * 2u;
        }
        const uint32_t base = lds_u32 + (uint32_t)(st * STAGE);
#pragma unroll
        for (int j = 0; j < X_INSTR; ++j) {
            const uint32_t vo = rq_c0 + x_ch[j] >= C ? 0x80000000u : x_vo[j];
            dma16(x_desc, vo, (uint32_t)rq_c0 * 2u, base + (uint32_t)((j * NW + wave) * 1024));
        }
#pragma unroll
        for (int j = 0; j < W_INSTR; ++j) {
            const uint32_t vo = rq_c0 + w_ch[j] >= C ? 0x80000000u : w_lane[j];
            dma16(w_desc, vo, w_tap + (uint32_t)rq_c0 * 2u, base + (uint32_t)(X_BYTES + (j * NW + wave) * 1024));
        }
        rq_c0 += BK;
        if (rq_c0 >= C) {
            rq_c0 = 0;
            new_tap = true;
            if (++rq_t == S) {
                rq_t = 0;
                ++rq_r;
            }
        }
    };

    // fragments: row (lane % 32) of each 32-row block, chunk 2*kk + lane/32
    const int xr0 = wm * TM + (lane & 31);
    const int wr0 = wn * TN + (lane & 31);
    const int x_sw = dy_swizzle(xr0), w_sw = dy_swizzle(wr0);   // the same for every block (32 keeps bits 1..3)
    float16_t acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[fn][fm][e] = 0.0f;
    auto compute = [&](int st) {
        const int sb = st * STAGE;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            half8_t af[FN], bf[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                af[fn] = __builtin_bit_cast(half8_t, *(const u32x4*)(lds + sb + X_BYTES + (wr0 + fn * 32) * 128 +
                                                                    (((kk * 2 + (lane >> 5)) ^ w_sw) * 16)));
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                bf[fm] = __builtin_bit_cast(half8_t, *(const u32x4*)(lds + sb + (xr0 + fm * 32) * 128 +
                                                                    (((kk * 2 + (lane >> 5)) ^ x_sw) * 16)));
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[fn], bf[fm], acc[fn][fm], 0, 0, 0);
        }
    };

    if (ns > 0)
        issue(0);
    if (ns > 1)
        issue(1);
    for (int i = 0; i < ns; ++i) {
        if (i + 1 < ns)
            wait_vmcnt<LD>();
        else
            wait_vmcnt<0>();
        __syncthreads();        // every wave's part of slice i is in LDS, and every wave
                                // is done with the stage the next request reuses
        if (i + 2 < ns)
            issue((i + 2) % 3);
        compute(i % 3);
    }

    // epilogue: the lane holds output channels 8*gq + 4*(lane/32) .. +3 of
    // block fn, pixel lane%32 of block fm; z = acc + bias, y = act(z), each
    // rounded once to fp16. Each wave's 32 pixels x TN channels pass through
    // LDS (chunk q of staged row p at position q ^ ((p >> 1) % CH)) and go out
    // as 16-byte chunks, so that one store covers 64/CH whole pixel rows of the
    // wave's TN*2 bytes; first z, then y.
    constexpr int CH = TN / 8;             // 16-byte chunks per staged pixel row
    constexpr int EROW = TN * 2;
    constexpr int EBLK = 32 * EROW;
    constexpr int PPI = 64 / CH;           // pixels per store instruction
    constexpr int EST = 32 / PPI;          // store instructions per pixel block
    static_assert(NW * EBLK <= 3 * STAGE, "the staging blocks fit in LDS");
    static_assert(CH >= 2 && CH <= 64 && 64 % CH == 0, "whole pixel rows per store");
    __syncthreads();                       // no wave reads a slice any more (every load has landed)
    const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(a.y, a.y_bytes);
    const __amdgpu_buffer_rsrc_t z_rsrc = make_rsrc(a.z != nullptr ? a.z : a.y, a.y_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(a.bias, (uint32_t)K * 2u);
    const bool store_z = a.z != nullptr;
    const bool hs = a.act == 1;
    lds_char* blk = (lds_char*)lds + wave * EBLK;
    half4_t bh[FN][4];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int k = n0 + wn * TN + fn * 32 + 8 * gq + 4 * (lane >> 5);
            bh[fn][gq] = __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(
                                                         b_rsrc, out_of_range_if((uint32_t)(k >= K), (uint32_t)k * 2u), 0, 0));
        }
    const int cw = n0 + wn * TN;           // first output channel of this wave's block
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int out = 0; out < 2; ++out) {
            if (out == 0 && !store_z)
                continue;
            const int pw = lane & 31;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float zv = acc[fn][fm][4 * gq + i] + (float)bh[fn][gq][i];
                        v[i] = (out == 1 && hs) ? hardswish_f(zv) : zv;
                    }
                    const half4_t o{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
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
                const uint32_t bad = (uint32_t)(m >= a.npq) | (uint32_t)(c >= K);
                const uint32_t off = ((uint32_t)m * (uint32_t)K + (uint32_t)c) * 2u;
                __builtin_amdgcn_raw_buffer_store_b128(v, out == 0 ? z_rsrc : y_rsrc, out_of_range_if(bad, off), 0, kStoreNT);
            }
        }
    }
}

// The compiled forward tile configurations: (BM, BN, WM, WN).
#define CBW_FWD_CONFIGS(X) \
    X(256, 128, 4, 2)      \
    X(128, 128, 2, 2)      \
    X(128, 64, 2, 2)

#define CBW_FWD_ENTRY(BM, BN, WM, WN) {BM, BN, WM, WN, #BM "x" #BN "x64/" #WM "x" #WN},
const FwdConfig kFwdConfigs[] = {CBW_FWD_CONFIGS(CBW_FWD_ENTRY)};
constexpr int kNumFwdConfigs = sizeof(kFwdConfigs) / sizeof(kFwdConfigs[0]);

template <int BM, int BN, int WM, int WN>
hipError_t fwd_launch(const FwdArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((fwd_igemm<BM, BN, WM, WN>), dim3(a.tiles_m * a.tiles_n), dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
int fwd_private(void)
{
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(fwd_igemm<BM, BN, WM, WN>)) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return (int)attr.localSizeBytes;
}

using FwdLaunchFn = hipError_t (*)(const FwdArgs&, hipStream_t);
#define CBW_FWD_LAUNCH(BM, BN, WM, WN) &fwd_launch<BM, BN, WM, WN>,
#define CBW_FWD_PRIVATE(BM, BN, WM, WN) &fwd_private<BM, BN, WM, WN>,
const FwdLaunchFn kFwdLaunch[] = {CBW_FWD_CONFIGS(CBW_FWD_LAUNCH)};
int (*const kFwdPrivate[])(void) = {CBW_FWD_CONFIGS(CBW_FWD_PRIVATE)};

}  // namespace

int fwd_num_configs() { return kNumFwdConfigs; }

const FwdConfig& fwd_config(int id) { return kFwdConfigs[id]; }

hipError_t launch_fwd(int id, const FwdArgs& a, hipStream_t stream)
{
    if (id < 0 || id >= kNumFwdConfigs)
        return hipErrorInvalidValue;
    return kFwdLaunch[id](a, stream);
}

int fwd_private_bytes(int id)
{
    return (id >= 0 && id < kNumFwdConfigs) ? kFwdPrivate[id]() : -1;
}

}  // namespace cbw
