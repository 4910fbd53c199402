// Internal interface between the host launcher (dgrad_api.cpp) and the HIP
// kernels (dgrad_kernels.hip). Not part of the public ABI.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "fastdiv.h"

namespace cbw {

// Phases per launch; strides above 4 are split over several launches.
constexpr int kMaxPhasesPerLaunch = 16;

// Bytes at the start of every workspace that hold arrival counters (one int32
// per GEMM tile of a split launch); the rest holds partial sums.
constexpr size_t kCounterBytes = 64 * 1024;

// Device memory behind the no-allocation entry point (per device, static).
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;

// One stride phase with taps, as the kernel sees it (see dgrad_plan.h for the algebra).
struct PhaseArg {
    int ph, pw;          // lattice offsets
    int Wp;              // lattice width
    int nr, nt;          // tap counts (0: zero phase)
    int r0, t0;          // first taps
    int dr0, dt0;        // dy offsets of the first taps
    int M;               // N*Hp*Wp
    int tiles_m;         // ceil(M / BM)
    int tile_begin;      // first tile id of this phase in the launch
    FastDiv div_hw;      // division by Hp*Wp
    FastDiv div_w;       // division by Wp
};

// One zero phase (no tap reaches its lattice): its M*C/8 16-byte vectors of
// zeros form the range [vbegin, vbegin + M*C/8) of the launch's zero-vector
// list. Each phase's range is padded to a whole number of stripes (one
// vector per thread of the workgroup), so a stripe never straddles phases.
struct ZeroPhaseArg {
    int ph, pw;          // lattice offsets
    int Wp;              // lattice width
    int M;               // N*Hp*Wp
    uint32_t vbegin;     // first vector of this phase in the list (a stripe boundary)
    FastDiv div_hw;      // division by Hp*Wp
    FastDiv div_w;       // division by Wp
};

// Work of one launch, walked by a persistent grid:
//   items [0, gemm_tiles)            GEMM tiles of the phases with taps; tile t
//                                    also stores zero stripes [t*zt, (t+1)*zt)
//                                    of the zero list, zps stripes with each of
//                                    its slice requests
//   items [gemm_tiles, total_tiles)  chunks of 8 zero stripes each, starting
//                                    at stripe zabsorbed
struct KernelArgs {
    const uint16_t* dy;
    const uint16_t* w;
    uint16_t* dx;
    const uint16_t* z;
    uint32_t dy_bytes;   // buffer sizes for the hardware range check
    uint32_t w_bytes;
    uint32_t dx_bytes;   // also the size of z
    int H, W, C, K, R, S, P, Q;
    int stride;
    int epi;
    int tiles_n;         // tiles along C
    int gemm_tiles;      // GEMM tiles over all phases with taps
    int total_tiles;     // GEMM tiles + zero chunks
    int grid;            // resident workgroups walking them (<= total_tiles)
    int order;           // 0: channel tiles of a pixel block consecutive; 1: pixel blocks of a channel tile;
                         // 2: the phases of a pixel block side by side (equal tile counts, grid % nphases == 0)
                         //    with channel tiles next
    int xcd_mode;        // 0: rotating groups of `group` tiles per XCD; 1: contiguous eighths
    int group;           // consecutive tiles kept on one XCD (mode 0)
    int nphases;
    PhaseArg ph[kMaxPhasesPerLaunch];
    // zero phases
    int nzphases;
    uint32_t zstripes;   // stripes in the zero list (padded)
    uint32_t zabsorbed;  // stripes stored by GEMM tiles (min(gemm_tiles * zt, zstripes))
    int zps;             // zero stripes per slice request: 0 or kMaxZeroPerSlice
    int zt;              // zero stripes per GEMM tile (<= zps * fewest slices of a tile)
    FastDiv div_c8;      // division by C/8
    ZeroPhaseArg zph[kMaxPhasesPerLaunch];
    // Companion zero phases: when the launch's only GEMM phase and its zero
    // phases share one lattice shape, zero pixel (n, ph' + s*i, pw' + s*j) lies
    // a fixed comp_delta[q] elements from GEMM pixel (n, ph + s*i, pw + s*j);
    // the epilogue stores those zeros beside each GEMM chunk (and the zero
    // list above is empty).
    int ncomp;
    int comp_delta[kMaxPhasesPerLaunch];
    // Stream-K: the launch's GEMM slices (tile after tile, phase i's first
    // at slice_begin[i]) are cut into `grid` equal contiguous ranges, one per
    // workgroup, so a tile may be shared by consecutive workgroups. Each
    // share of a split tile leaves its fp32 partial sums in workspace slot
    // [tile][segment]; the last share to arrive (per-tile counter) adds the
    // shares in segment order, runs the epilogue and resets the counter.
    int sk;              // 1: stream-K split (launches without zero phases only)
    int sk_slices;       // GEMM slices of the launch
    int sk_maxseg;       // workspace slots per tile
    float* sk_part;      // [gemm_tiles][sk_maxseg][BM*BN] fp32, in register order
    int* sk_count;       // [gemm_tiles] arrival counters, zero between launches
    int slice_begin[kMaxPhasesPerLaunch];   // first slice of each GEMM phase's tiles
};

// Zero stripes a slice request may carry (each is one 16-byte store per thread).
constexpr int kMaxZeroPerSlice = 4;
// Zero stripes per standalone chunk.
constexpr int kZeroChunkStripes = 8;

struct TileConfig {
    int BM;              // dx pixels per tile (GEMM rows)
    int BN;              // dx channels per tile (GEMM columns)
    int BK;              // reduction slice per pipeline stage
    int WM, WN;          // wave grid (64-lane waves) over the tile
    const char* name;
    int lds_bytes;
    bool streamk;        // compiled with a stream-K variant
    bool phase_order;    // supports tile order 2 (phases of a pixel block side by side)
    bool plain_only;     // runs launches of GEMM tiles only, one tile per workgroup (dgrad_wide,
                         // dgrad_halo); the host gives launches with zero phases to plain_fallback(id)
    bool restricted;     // runs only the layers tile_config_admits() accepts (dgrad_halo, dgrad_pgemm,
                         // dgrad_halo1, dgrad_pwide); the host gives other layers to plain_fallback(id)
    bool chunk_split;    // splits by k chunk, one workgroup per tile and chunk (dgrad_halo1), instead of
                         // stream-K's equal slice ranges; a launch tile_config_runs() refuses goes to
                         // plain_fallback(id)
};

// ------------------------------------------------------------------ wgrad

// Filter gradient of the same layer (see wgrad_igemm in dgrad_kernels.hip):
// dw[k,r,t,c] = sum over pixels m = (n,p,q) of dy[m,k] * x[n, p*s-pad+r, q*s-pad+t, c].
// One GEMM per tap, D[c][k] = sum_m x_tap[m][c] * dy[m][k], over tiles of BC
// channels x BK output channels; the pixel reduction (64-pixel slices) is cut
// into `splits` contiguous ranges whose fp32 partial sums a second kernel adds
// in split order.
struct WgradArgs {
    const uint16_t* dy;
    const uint16_t* x;
    float* dw;           // [K][R][S][C] fp32, fully written
    float* part;         // [splits][tiles][BC*BK] fp32 partial sums in register order, or NULL
                         // with splits == 1: the kernel writes dw directly
    uint32_t dy_bytes;
    uint32_t x_bytes;
    int N, H, W, C, K, R, S, P, Q, stride, pad;
    int npq;             // N*P*Q: reduction length
    int slices;          // ceil(npq / 64)
    int tiles_c, tiles_k, tiles;   // tiles = R*S*tiles_c*tiles_k (tap outermost, output channels fastest)
    int splits;
    FastDiv div_pq;      // division by P*Q
    FastDiv div_q;       // division by Q
};

struct WgradConfig {
    int BC, BK, WC, WK;
    const char* name;
};
int wgrad_num_configs();
const WgradConfig& wgrad_config(int id);
hipError_t launch_wgrad(int id, const WgradArgs& a, hipStream_t stream);
hipError_t launch_wgrad_reduce(int id, const WgradArgs& a, hipStream_t stream);
int wgrad_private_bytes(int id);   // scratch bytes per lane of both kernels, -1 if unknown

// ------------------------------------------------------------------ forward

// The forward layer with its fused epilogue (see fwd_igemm in
// dgrad_kernels.hip): z[m,k] = bias[k] + sum over taps and c of
// x[n, p*s-pad+r, q*s-pad+t, c] * w[k,r,t,c] for output pixel m = (n,p,q),
// y = hardswish(z) (act 1) or z (act 0). GEMM rows are output pixels, columns
// output channels, the reduction runs tap by tap over C in 64-wide slices.
struct FwdArgs {
    const uint16_t* x;
    const uint16_t* w;
    const uint16_t* bias;
    uint16_t* z;         // [N][P][Q][K] fp16 pre-activation, or NULL
    uint16_t* y;         // [N][P][Q][K] fp16 output
    uint32_t x_bytes;
    uint32_t w_bytes;
    uint32_t y_bytes;    // also the size of z
    int N, H, W, C, K, R, S, P, Q, stride, pad, act;
    int npq;             // N*P*Q
    int tiles_m, tiles_n;
    int csteps;          // ceil(C / 64)
    FastDiv div_pq;
    FastDiv div_q;
};

struct FwdConfig {
    int BM, BN, WM, WN;
    const char* name;
};
int fwd_num_configs();
const FwdConfig& fwd_config(int id);
hipError_t launch_fwd(int id, const FwdArgs& a, hipStream_t stream);
int fwd_private_bytes(int id);

// ------------------------------------------------------------------ chain

// Two dgrad steps of a bottleneck in one kernel (see chain_igemm in
// chain_kernels.hip): t[m,c] = fp16(g(z[m,c]) * stride-1 dgrad of dy through
// the RxS filter w1 [K][R][S][Cm]), then dx[m,ci] = fp16(sum over c of
// t[m,c] * w2[c,ci]) with the 1x1 filter w2 [Cm][C]; t stays in LDS.
struct ChainArgs {
    const uint16_t* dy;  // [N][P][Q][K]
    const uint16_t* w1;  // [K][R][S][Cm]
    const uint16_t* z;   // [N][H][W][Cm] (read for epi 1 and 2)
    const uint16_t* w2;  // [Cm][C]
    uint16_t* dx;        // [N][H][W][C]
    uint32_t dy_bytes, w1_bytes, z_bytes, w2_bytes, dx_bytes;
    int N, H, W, Cm, K, R, S, pad, P, Q, C, epi;
    int M;               // N*H*W
    int tiles;           // ceil(M / 128)
    FastDiv div_hw;      // division by H*W
    FastDiv div_w;       // division by W
};
hipError_t launch_chain(const ChainArgs& a, hipStream_t stream);
int chain_private_bytes(int Cm, int epi);   // scratch bytes per lane, -1 if unknown
int chain_lds_bytes(int Cm);

// Zero fill of a device buffer (16-byte aligned, a multiple of 16 bytes).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

// The no-allocation scratch of the current device (kNoAllocScratchBytes,
// 256-byte aligned): its device address, found and its counter area cleared
// (on `stream`) the first time per device.
hipError_t noalloc_scratch(void** ptr, hipStream_t stream);

// The configurations of dgrad_wide (dgrad_wide.hip), numbered after those of
// dgrad_igemm in the table of every configuration.
int wide_num_configs();
const TileConfig& wide_config(int i);
hipError_t launch_wide(int i, const KernelArgs& a, hipStream_t stream);
int wide_blocks_per_cu(int i);
int wide_private_bytes(int i);

// The configurations of dgrad_halo (dgrad_halo.hip), numbered after those of
// dgrad_wide.
int halo_num_configs();
const TileConfig& halo_config(int i);
bool halo_admits(int i, int R, int S, int stride, int pad, int H, int W, int P, int Q);
hipError_t launch_halo(int i, const KernelArgs& a, hipStream_t stream);
int halo_blocks_per_cu(int i);
int halo_private_bytes(int i);

// The configurations of dgrad_pgemm (dgrad_pgemm.hip), numbered after those of
// dgrad_halo.
int pgemm_num_configs();
const TileConfig& pgemm_config(int i);
bool pgemm_admits(int i, int R, int S, int stride, int pad, int K, int epi);
hipError_t launch_pgemm(int i, const KernelArgs& a, hipStream_t stream);
int pgemm_blocks_per_cu(int i);
int pgemm_private_bytes(int i);

// The configurations of dgrad_halo1 (dgrad_halo1.hip), numbered after those
// of dgrad_pgemm.
int halo1_num_configs();
const TileConfig& halo1_config(int i);
bool halo1_admits(int i, int R, int S, int stride, int pad, int H, int W, int P, int Q, int K, int epi);
bool halo1_runs_launch(int i, const KernelArgs& a);
constexpr int kHalo1MaxChunks = 8;   // k chunks of 64 a split dgrad_halo1 launch may have
hipError_t launch_halo1(int i, const KernelArgs& a, hipStream_t stream);
int halo1_blocks_per_cu(int i);
int halo1_private_bytes(int i);

// The configurations of dgrad_pwide (dgrad_pwide.hip), numbered after those
// of dgrad_halo1.
int pwide_num_configs();
const TileConfig& pwide_config(int i);
bool pwide_admits(int i, int R, int S, int stride, int epi);
bool pwide_runs_launch(int i, const KernelArgs& a);   // no zero phases, no split
hipError_t launch_pwide(int i, const KernelArgs& a, hipStream_t stream);
int pwide_blocks_per_cu(int i);
int pwide_private_bytes(int i);

int num_tile_configs();
const TileConfig& tile_config(int id);
// Whether config `id` runs the layer itself (true for all but restricted
// configs outside their layers).
bool tile_config_admits(int id, int R, int S, int stride, int pad, int H, int W, int P, int Q, int K, int epi);
// Whether config `id` runs launch `a` as planned (false only for a
// dgrad_halo1 launch of more than one k chunk that is not split, and a
// dgrad_pwide launch with zero phases).
bool tile_config_runs(int id, const KernelArgs& a);
int plain_fallback(int id);   // for a plain_only or restricted config: the dgrad_igemm config of the same tile
hipError_t launch_tile_config(int id, const KernelArgs& a, hipStream_t stream);
int blocks_per_cu(int id);   // resident workgroups per CU (current device)
int kernel_private_bytes(int id);   // scratch bytes per lane of a config's kernel (-1: unknown)
inline int threads_per_block(const TileConfig& tc) { return 64 * tc.WM * tc.WN; }

}  // namespace cbw
