/*
 * conv2d_dgrad.h -- C ABI of the MI355X (gfx950) conv2d backward-data library.
 *
 * The operation. The forward layer is a 2-D cross-correlation with one stride
 * s and one symmetric zero padding `pad`:
 *     y[n,p,q,k] = sum_{r,t,c} x[n, p*s - pad + r, q*s - pad + t, c] * w[k,r,t,c]
 * with P = floor((H + 2*pad - R)/s) + 1 and Q = floor((W + 2*pad - S)/s) + 1.
 * Backward-data ("dgrad", the subject of "[CUTLASS] Conv2d dgrad", apache/tvm
 * PR #10110, and of cuDNN's ConvolutionBackwardData in "Performance
 * improvements by calling cuDNN API", JuliaGPU/CUDA.jl PR #321) is its adjoint:
 *     dx[n,h,w,c] = sum_{k,r,t} dy[n,p,q,k] * w[k,r,t,c]
 * over the taps where h = p*s - pad + r and w = q*s - pad + t for some
 * 0 <= p < P, 0 <= q < Q. Positions that no tap reaches are written as 0.
 * It is computed as an implicit GEMM with M = N*H*W rows, C columns and a
 * reduction over K*R*S, split for stride s into s*s phase sub-GEMMs so that no
 * inserted-zero products are formed.
 *
 * Precision. fp16 storage, fp32 accumulation (the tvm PR's review remarks that
 * training needs fp32 accumulation), one round-to-nearest-even conversion to
 * fp16 at the end.
 *
 * Fused epilogue (the fusion the tvm PR notes is "not enabled for dgrad yet",
 * and the Conv2D + BiasAdd + Hardswish pattern of the Bolt paper notes,
 * KuangjuX/Paper-reading #28, "Insights"): dx = acc * g(z) with z the saved
 * pre-activation, g = relu'(z) = [z > 0] or g = hardswish'(z) = 0 (z < -3),
 * z/3 + 1/2 (-3 <= z <= 3), 1 (z > 3). g is evaluated in fp32.
 *
 * Layouts (all C-contiguous fp16, i.e. IEEE binary16 bit patterns):
 *     dy [N][P][Q][K]   NHWC gradient of the forward output
 *     w  [K][R][S][C]   KRSC filter (k = output channel of the forward layer)
 *     dx [N][H][W][C]   NHWC result; write-only, every element overwritten
 *     z  [N][H][W][C]   NHWC saved pre-activation (epilogue only)
 *
 * Ownership and execution. All tensor pointers are device pointers owned by
 * the caller, who keeps them alive until the enqueued work completes. Calls
 * are asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 * The library allocates no device memory, ever. dx is never read (it may hold
 * anything, NaN included, before the call). dx must not overlap dy, w or z.
 *
 * Workspace (the FindEx pattern of the CUDA.jl PR: the caller, not the
 * library, allocates, so a pool allocator stays in charge of device memory).
 * The *_ws and *_config entry points take an optional device workspace that
 * lets a call split its reduction (stream-K for dgrad, split-K for wgrad).
 * The *_workspace_size queries give the bytes that let every candidate of a
 * problem split; a smaller workspace only narrows the choice, and without one
 * (NULL, 0 bytes) every launch runs whole tiles. Layout and contract:
 *   - at least 65536 bytes, 16-byte aligned, not overlapping any tensor;
 *   - the first 65536 bytes hold arrival counters: ZERO THEM ONCE before the
 *     workspace's first use (e.g. torch.zeros or hipMemset). Every call leaves
 *     them zero again when its work completes, so one workspace serves any
 *     number of later calls, of any shape and entry point, without clearing;
 *   - the rest holds fp32 partial sums; its contents between calls are free;
 *   - calls that share a workspace must be ordered (one stream, or
 *     synchronised); calls that overlap in time on one workspace race.
 *
 * Tile-config selection. The first call for a new problem key (every shape
 * argument, the epilogue kind and the device) picks a tile configuration:
 * when autotuning is on and the stream is not capturing, every compiled
 * candidate is timed on the caller's own buffers and stream (the "Find"
 * approach described in the CUDA.jl PR; this call then synchronises the
 * stream once); otherwise a shape heuristic picks one (the "Get" approach).
 * The choice is cached in an unbounded, mutex-guarded table (that PR's final
 * choice: a plain dictionary without a capacity limit, keyed by the full
 * problem) and reused by every later call with the same key.
 *
 * Errors. Every entry point returns a status code. Arguments are validated
 * before any HIP call; on failure nothing is enqueued and
 * conv2d_dgrad_last_error() (per thread) describes the problem.
 */
#ifndef CONV2D_DGRAD_H
#define CONV2D_DGRAD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define CONV2D_DGRAD_OK 0
#define CONV2D_DGRAD_INVALID_ARGUMENT 1 /* null pointer, dim < 1, stride < 1, pad < 0,
                                           P or Q < 1, unknown epilogue, z missing,
                                           pointer not 16-byte aligned, dx overlapping
                                           an input, bad config id, a workspace below
                                           65536 bytes, misaligned or overlapping a
                                           tensor, or NULL with a nonzero size */
#define CONV2D_DGRAD_UNSUPPORTED 2      /* C or K not a multiple of 8, a tensor of
                                           2^30 elements or more, stride > 16 */
#define CONV2D_DGRAD_HIP_ERROR 3        /* a HIP runtime call or launch failed */

/* epilogue kinds */
#define CONV2D_DGRAD_EPI_NONE 0
#define CONV2D_DGRAD_EPI_DRELU 1
#define CONV2D_DGRAD_EPI_DHARDSWISH 2

/*
 * dx = dgrad(dy, w) [* g(z)] on `stream`.
 *   N, H, W, C : batch, dx height, dx width, dx channels
 *   K, R, S    : dy channels, filter height, filter width
 *   stride, pad: the forward layer's stride (1..16) and symmetric padding (>= 0)
 *   epilogue   : CONV2D_DGRAD_EPI_*; z must be non-NULL unless NONE (ignored then)
 * P and Q are derived from H, W, R, S, stride and pad as above (several H give
 * the same P under stride > 1, which is why H and W are passed).
 * Constraints: C % 8 == 0, K % 8 == 0 (16-byte vectors along channels), all
 * pointers 16-byte aligned, every tensor below 2^30 elements (2 GiB).
 */
int conv2d_dgrad_nhwc(const void* dy, const void* w, void* dx,
                      int N, int H, int W, int C, int K, int R, int S,
                      int stride, int pad, int epilogue, const void* z,
                      void* stream);

/*
 * The same with a caller-owned workspace (see "Workspace" above): launches
 * whose tiles would leave workgroups idle may then split their reduction
 * (stream-K, conv2d_dgrad_set_streamk). workspace may be NULL (with
 * workspace_bytes = 0), which is conv2d_dgrad_nhwc. The table keeps separate
 * choices for calls with and without a workspace.
 */
int conv2d_dgrad_nhwc_ws(const void* dy, const void* w, void* dx,
                         int N, int H, int W, int C, int K, int R, int S,
                         int stride, int pad, int epilogue, const void* z,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * *bytes = the workspace size that lets every tile configuration of this
 * problem take its split (the counter area plus the largest partial-sum area
 * any candidate plans), or 0 when no candidate can split. Host-only; the
 * figure assumes the current device's CU count and occupancy.
 */
int conv2d_dgrad_workspace_size(int N, int H, int W, int C, int K, int R, int S,
                                int stride, int pad, int epilogue, size_t* bytes);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * call as conv2d_dgrad_nhwc_ws, with the workspace taken from a static
 * device array of the library, conv2d_dgrad_noalloc_max_bytes() = 128 MiB,
 * which each GPU the library runs on holds until the process ends. Nothing
 * is allocated, by the library or by the caller. The first call on a device
 * looks up the array's address on that device and clears its counter area
 * with a small kernel on `stream`. A problem whose split candidates need
 * more than the array (see conv2d_dgrad_workspace_size) is rejected with
 * CONV2D_DGRAD_UNSUPPORTED before anything is enqueued. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (different
 * streams or host threads without ordering) race and may give wrong
 * results; order them.
 */
int conv2d_dgrad_nhwc_noalloc(const void* dy, const void* w, void* dx,
                              int N, int H, int W, int C, int K, int R, int S,
                              int stride, int pad, int epilogue, const void* z,
                              void* stream);

/* Size of the static array behind conv2d_dgrad_nhwc_noalloc, in bytes. */
size_t conv2d_dgrad_noalloc_max_bytes(void);

/*
 * Same computation with an explicit tile configuration (0 <= config_id <
 * conv2d_dgrad_num_configs()), bypassing the table, and an optional
 * workspace as for conv2d_dgrad_nhwc_ws. For tests that check every
 * candidate and for benchmarks that sweep them.
 */
int conv2d_dgrad_nhwc_config(const void* dy, const void* w, void* dx,
                             int N, int H, int W, int C, int K, int R, int S,
                             int stride, int pad, int epilogue, const void* z,
                             int config_id, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Number of compiled tile configurations, and a readable name for one
 * ("BMxBNxBK/WMxWN"): buf receives at most buflen bytes, NUL-terminated. */
int conv2d_dgrad_num_configs(void);
int conv2d_dgrad_config_name(int config_id, char* buf, int buflen);

/*
 * The configuration the table holds for a problem key (with_workspace: the
 * entry for calls that bring a workspace), without launching: *config_id =
 * the cached choice, or the heuristic's choice when the key is not cached
 * (*cached = 0); *split (if non-NULL) = 1 when the cached choice splits the
 * reduction. Validates the shape like conv2d_dgrad_nhwc. Needs no GPU when
 * the key is not cached.
 */
int conv2d_dgrad_query_config(int N, int H, int W, int C, int K, int R, int S,
                              int stride, int pad, int epilogue, int with_workspace,
                              int* config_id, int* cached, int* split);

/* Autotuning on (1, the default unless the environment sets
 * CONV2D_DGRAD_AUTOTUNE=0) or off (0). Returns the previous setting. */
int conv2d_dgrad_set_autotune(int on);

/*
 * Fault injection for the profilers' failure path (also set by the
 * environment variable CONV2D_DGRAD_FAULT_INJECT=1): while on, every candidate
 * a profiler would time counts as failed before it is launched, so the
 * problem keeps the shape heuristic's choice ("Get"), which the CUDA.jl PR
 * names as the fallback of a failed "Find". Returns the previous setting.
 */
int conv2d_dgrad_set_fault_inject(int on);

/*
 * Stream-K split of the reduction. A launch's reduction slices (all its GEMM
 * tiles' slices, tile after tile) can be cut into equal contiguous ranges,
 * one per workgroup, which helps when the tiles alone would leave workgroups
 * idle. A tile shared by several workgroups is finished by the last of them
 * to arrive, which adds the others' fp32 partial sums in a fixed order
 * (results do not depend on timing, but differ in rounding from the unsplit
 * sum). This is the "parallel split-k" that the "[CUTLASS] Conv2d dgrad" page
 * (apache/tvm PR #10110) names as follow-up work.
 *
 * The partial sums and arrival counters live in the caller's workspace
 * (conv2d_dgrad_nhwc_ws, conv2d_dgrad_nhwc_config); a call without one, or
 * whose workspace is too small for a launch's partial sums, runs that
 * launch with whole tiles. A share's partial sums are written and read with
 * system-scope cache policy, so they pass between the XCDs' separate L2
 * caches without any cache flush. At most 16384 GEMM tiles per launch split.
 *
 *   mode 0: never split.
 *   mode 1: split every eligible launch (no zero phases, 1..16384 GEMM
 *           tiles, partial sums within 1 GiB and within the workspace) as
 *           finely as the device allows.
 *   mode 2 (default): the profiler times each tile configuration with and
 *           without the split, and the table keeps the faster (table files
 *           mark a split choice with "+sk" after the config name). For an
 *           explicit config, or without profiling, a cost model splits when
 *           that shortens the longest workgroup's work by 10% or more.
 * Returns the previous mode, or -1 (with INVALID_ARGUMENT as the last error)
 * for a mode outside 0..2. Choices already in the table are kept.
 */
int conv2d_dgrad_set_streamk(int mode);

/* Kernel launches enqueued with a stream-K split since the library loaded
 * (a diagnostic: it tells a caller whether the split was taken). */
long long conv2d_dgrad_streamk_launches(void);

/* Drop every cached choice; number of entries in the table. */
int conv2d_dgrad_cache_clear(void);
int conv2d_dgrad_cache_size(void);

/* Persist the table to a text file / merge a saved table into it (so a new
 * process skips re-profiling). Lines: the key fields, then the config name. */
int conv2d_dgrad_cache_save(const char* path);
int conv2d_dgrad_cache_load(const char* path);

/*
 * The stride-phase plan (host-only, no GPU): for each phase (ph, pw) in
 * [0,s)^2 the output positions h = ph + s*i, w = pw + s*j form an Hp x Wp
 * sub-grid, and only the filter taps r = r0 + a*s (a < nr), t = t0 + b*s
 * (b < nt) reach it, from dy rows p = i + dr0 - a and columns q = j + dt0 - b.
 * Each phase is an M x C x Kg GEMM with M = N*Hp*Wp and Kg = K*nr*nt; Kg == 0
 * marks a zero phase, whose outputs are all exact zeros. Phases with an empty
 * sub-grid (Hp or Wp == 0, possible when s > H or s > W) are omitted.
 * Phases are returned heaviest first (by nr*nt, ties by (ph, pw)).
 */
typedef struct {
    int ph, pw;      /* phase offsets in [0, stride) */
    int Hp, Wp;      /* sub-grid extents */
    int r0, t0;      /* first row tap, first column tap */
    int nr, nt;      /* number of row taps and column taps */
    int dr0, dt0;    /* dy row/column offsets of the first taps */
    long long M;     /* GEMM rows N*Hp*Wp */
    long long Kg;    /* GEMM reduction length K*nr*nt (0: zero phase) */
} conv2d_dgrad_phase;

int conv2d_dgrad_plan(int N, int H, int W, int C, int K, int R, int S,
                      int stride, int pad, conv2d_dgrad_phase* phases,
                      int max_phases, int* nphases, int* P, int* Q);

/* Validation alone (no HIP call): the status conv2d_dgrad_nhwc would return
 * for these arguments before launching anything. */
int conv2d_dgrad_check(const void* dy, const void* w, void* dx,
                       int N, int H, int W, int C, int K, int R, int S,
                       int stride, int pad, int epilogue, const void* z);

/*
 * Filter gradient (wgrad) of the same forward layer:
 *
 *   dw[k,r,t,c] = sum over n,p,q of dy[n,p,q,k] * x[n, p*s - pad + r, q*s - pad + t, c],
 *
 * where input positions in the padding contribute zero. This is the other
 * half of conv backward, which the "[CUTLASS] Conv2d dgrad" page (apache/tvm
 * PR #10110) leaves for later because of its accuracy issues.
 *
 * Arguments:
 *   dy [N][P][Q][K]   fp16, as for conv2d_dgrad_nhwc
 *   x  [N][H][W][C]   fp16 NHWC input of the forward layer
 *   dw [K][R][S][C]   fp32, fully written (never read)
 * Shapes, alignment (16 bytes), limits and status codes are those of
 * conv2d_dgrad_nhwc; dw must not overlap dy or x.
 *
 * Accumulation is fp32 throughout. With a workspace (conv2d_wgrad_nhwc_ws),
 * the N*P*Q-long reduction is cut into contiguous ranges whose fp32 partial
 * sums (in the workspace after its counter area) a second kernel adds in a
 * fixed order, so results do not depend on timing. Without one, a single
 * range per tile writes dw directly: correct, but with only R*S*ceil(C/BC)*
 * ceil(K/BK) workgroups it leaves most of the chip idle on large layers.
 * Calls are asynchronous on `stream`.
 */
int conv2d_wgrad_nhwc(const void* dy, const void* x, void* dw,
                      int N, int H, int W, int C, int K, int R, int S,
                      int stride, int pad, void* stream);

/* The same with a caller-owned workspace (contract as for dgrad above); the
 * split count is cut to what the workspace holds. */
int conv2d_wgrad_nhwc_ws(const void* dy, const void* x, void* dw,
                         int N, int H, int W, int C, int K, int R, int S,
                         int stride, int pad, void* workspace, size_t workspace_bytes,
                         void* stream);

/* *bytes = the workspace that holds the largest split any wgrad candidate of
 * this problem uses (0 when none splits). Host-only. */
int conv2d_wgrad_workspace_size(int N, int H, int W, int C, int K, int R, int S,
                                int stride, int pad, size_t* bytes);

/* The same with an explicit tile configuration (0 .. conv2d_wgrad_num_configs()-1),
 * reduction split count (0: automatic, about two workgroups per CU; cut to
 * what the workspace holds) and optional workspace. */
int conv2d_wgrad_nhwc_config(const void* dy, const void* x, void* dw,
                             int N, int H, int W, int C, int K, int R, int S,
                             int stride, int pad, int config_id, int splits,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Number of compiled wgrad tile configurations. */
int conv2d_wgrad_num_configs(void);

/* Validation alone (no HIP call) for conv2d_wgrad_nhwc. */
int conv2d_wgrad_check(const void* dy, const void* x, void* dw,
                       int N, int H, int W, int C, int K, int R, int S,
                       int stride, int pad);

/*
 * The forward layer with the fused bias + activation epilogue that the
 * Bolt paper notes (KuangjuX/Paper-reading #28, "Insights") describe as
 * Conv2D + BiasAdd + Hardswish:
 *
 *   z[n,p,q,k] = bias[k] + sum over r,t,c of x[n, p*s - pad + r, q*s - pad + t, c] * w[k,r,t,c]
 *   y = hardswish(z) = z * min(max(z + 3, 0), 6) / 6   (act = 1), or y = z (act = 0),
 *
 * accumulated in fp32; z and y are each rounded once to fp16. z is the saved
 * pre-activation that conv2d_dgrad_nhwc's fused epilogue consumes.
 *
 * Arguments:
 *   x    [N][H][W][C]   fp16 NHWC input
 *   w    [K][R][S][C]   fp16 filter
 *   bias [K]            fp16 (8-byte aligned)
 *   z    [N][P][Q][K]   fp16 pre-activation output, or NULL not to store it
 *   y    [N][P][Q][K]   fp16 output
 * Shapes, limits and status codes are those of conv2d_dgrad_nhwc; y and z
 * must not overlap the inputs or each other. No workspace; asynchronous on
 * `stream`.
 */
int conv2d_forward_nhwc(const void* x, const void* w, const void* bias, void* z, void* y,
                        int N, int H, int W, int C, int K, int R, int S,
                        int stride, int pad, int act, void* stream);

/* The same with an explicit tile configuration (0 .. conv2d_forward_num_configs()-1). */
int conv2d_forward_nhwc_config(const void* x, const void* w, const void* bias, void* z, void* y,
                               int N, int H, int W, int C, int K, int R, int S,
                               int stride, int pad, int act, int config_id, void* stream);

/* Number of compiled forward tile configurations. */
int conv2d_forward_num_configs(void);

/* Validation alone (no HIP call) for conv2d_forward_nhwc. */
int conv2d_forward_check(const void* x, const void* w, const void* bias, void* z, void* y,
                         int N, int H, int W, int C, int K, int R, int S,
                         int stride, int pad, int act);

/*
 * Two dgrad steps of a bottleneck fused into one kernel: the persistent
 * kernel fusion of the Bolt paper notes (KuangjuX/Paper-reading #28,
 * "Persistent kernel (GEMM/Conv) fusion"), with threadblock residence (a
 * workgroup owns all Cm intermediate channels of its 128 pixels) and the
 * intermediate tile held in shared memory (LDS) between the two GEMMs:
 *
 *   t[n,h,w,c]   = fp16( g(z[n,h,w,c]) * sum over r,s,k of
 *                        dy[n, h + pad - r, w + pad - s, k] * w1[k,r,s,c] )
 *   dx[n,h,w,ci] = fp16( sum over c of t[n,h,w,c] * w2[c,ci] )
 *
 * with the taps of the first sum limited to 0 <= h + pad - r < P and
 * 0 <= w + pad - s < Q. The first step is conv2d_dgrad_nhwc at stride 1
 * with its epilogue (g = 1, relu' or hardswish' of z, CONV2D_DGRAD_EPI_*);
 * the second is the dgrad of the 1x1 stride-1 convolution that made the
 * first convolution's input. Both accumulate in fp32; t is rounded once to
 * fp16, as the two separate calls would store it, and is never written to
 * memory.
 *
 * Arguments:
 *   dy [N][P][Q][K]   fp16, P = H + 2*pad - R + 1, Q = W + 2*pad - S + 1
 *   w1 [K][R][S][Cm]  fp16 filter of the RxS convolution (Cm -> K channels)
 *   z  [N][H][W][Cm]  fp16 saved pre-activation (ignored for EPI_NONE)
 *   w2 [Cm][1][1][C]  fp16 filter of the 1x1 convolution (C -> Cm channels)
 *   dx [N][H][W][C]   fp16 output, fully written, never read
 * Limits: those of conv2d_dgrad_nhwc at stride 1 for the first step, plus
 * Cm <= 128 (the resident tile) and C a multiple of 8 with N*H*W*C and Cm*C
 * below 2^30. dx must not overlap any input. Pointers 16-byte aligned. The
 * caller owns all buffers; no workspace; asynchronous on `stream`. Returns
 * a CONV2D_DGRAD_* status; on error nothing is launched.
 */
int conv2d_dgrad_chain_nhwc(const void* dy, const void* w1, const void* z, const void* w2, void* dx,
                            int N, int H, int W, int Cm, int K, int R, int S, int pad, int C,
                            int epilogue, void* stream);

/*
 * The same with a caller-owned workspace (contract as above). When the
 * workspace holds the intermediate t (conv2d_dgrad_chain_workspace_size: the
 * counter area plus N*H*W*Cm fp16), the chain may instead run as two
 * conv2d_dgrad_nhwc calls with t stored there, if that is faster: the first
 * such call for a problem times both paths on the caller's buffers and
 * stream (with autotuning on, outside graph capture; it synchronises the
 * stream once) and caches the faster per problem and device. Both paths give
 * the same bits: t is rounded to fp16 once either way.
 */
int conv2d_dgrad_chain_nhwc_ws(const void* dy, const void* w1, const void* z, const void* w2, void* dx,
                               int N, int H, int W, int Cm, int K, int R, int S, int pad, int C,
                               int epilogue, void* workspace, size_t workspace_bytes, void* stream);

/* *bytes = the workspace that lets conv2d_dgrad_chain_nhwc_ws choose the
 * two-call path. Host-only. */
int conv2d_dgrad_chain_workspace_size(int N, int H, int W, int Cm, int K, int R, int S, int pad, int C,
                                      int epilogue, size_t* bytes);

/* The path cached for a chain problem on the current device: *cached = 0 if
 * none yet; *pair = 1 when the two-call path was found faster. */
int conv2d_dgrad_chain_query(int N, int H, int W, int Cm, int K, int R, int S, int pad, int C,
                             int epilogue, int* pair, int* cached);

/* Validation alone (no HIP call) for conv2d_dgrad_chain_nhwc. */
int conv2d_dgrad_chain_check(const void* dy, const void* w1, const void* z, const void* w2, const void* dx,
                             int N, int H, int W, int Cm, int K, int R, int S, int pad, int C,
                             int epilogue);

/* Thread-local text of the last error ("" if none). */
const char* conv2d_dgrad_last_error(void);

/* Compiler and HIP versions the library was built with, and its target. */
const char* conv2d_dgrad_build_info(void);

#ifdef __cplusplus
}
#endif
#endif /* CONV2D_DGRAD_H */
