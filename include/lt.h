/*
 * lt.h — C ABI of the layout-algebra GEMM library for AMD Instinct MI355X
 * (gfx950).
 *
 * The library has three parts, all behind plain C types:
 *   1. Host layout algebra: Shape:Stride layouts as values, their evaluation,
 *      coalesce, composition, complement, logical/zipped divide, local_tile
 *      and local_partition. Pure integer math, no device, thread-safe.
 *   2. Device layout maps: evaluate or gather through a layout on the GPU.
 *   3. The tiled GEMM D = alpha*A*B + beta*C with fp16/bf16 operands and fp32
 *      accumulation, whose operands, block tiles and thread partitions are
 *      addressed through those layouts.
 *
 * Sources (cited by page title and section):
 *   [P1] "CUTLASS and CuTe layouts" (Day 84)
 *   [P2] "3.5 CUTLASS II — CuTe 레이아웃·텐서"
 *   [P3] "CUTLASS, in depth: the GEMM hierarchy, CuTe layouts, Hopper kernel
 *        schedules and the Python DSL"
 *   [P4] "Layouts as Algebra: CUTLASS & CuTe"
 *
 * Conventions for every function:
 *   - The return value is an lt_status; results come back through pointer
 *     arguments, which the caller owns. On any error nothing is written to
 *     the outputs and nothing is launched.
 *   - Layouts are caller-owned values (lt_layout, no heap, no free function).
 *   - Device pointers are caller-owned device memory; the library never
 *     allocates or frees device memory on the caller's behalf.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device functions are asynchronous on that stream; a launch failure is
 *     reported as LT_ERR_HIP, later faults surface at the caller's next
 *     synchronisation.
 */
#ifndef LT_H_
#define LT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------ */
/* Status                                                                    */
/* ------------------------------------------------------------------------ */

typedef enum lt_status {
    LT_OK = 0,
    LT_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, bad enum, bad count           */
    LT_ERR_INVALID_LAYOUT = 2,     /* incongruent tree, extent < 1, stride < 0    */
    LT_ERR_NOT_ADMISSIBLE = 3,     /* composition/complement has no layout [P4 "Composition, worked by hand"] */
    LT_ERR_NOT_DIVISIBLE = 4,      /* tiler does not divide the mode [P2 3.5.8]   */
    LT_ERR_OUT_OF_RANGE = 5,       /* index >= size, coordinate out of its mode, int64 overflow */
    LT_ERR_MISALIGNED_OPERAND = 6, /* 16-bit operand not 128-bit aligned [P1 "Pitfalls"; P3 "Failure modes"] */
    LT_ERR_UNSUPPORTED = 7,        /* no kernel for this layout/dtype combination */
    LT_ERR_ARCH_MISMATCH = 8,      /* device is not gfx950 [P1 "Results", "Pitfalls"] */
    LT_ERR_LDS_OVERFLOW = 9,       /* tile x stages exceeds LDS [P3 "Failure modes"] */
    LT_ERR_WORKSPACE = 10,         /* workspace missing or too small              */
    LT_ERR_HIP = 11,               /* a HIP runtime call failed                   */
    LT_ERR_CAPACITY = 12           /* result needs more leaves/nodes than lt_layout holds, or text buffer too small */
} lt_status;

/* Static description of a status code (never NULL). Every call reports a
 * status and the caller checks it, as the pages ask of can_implement
 * [P3 "Failure modes": always check the return status; P1 "Pitfalls"]. */
const char* lt_status_string(lt_status s);

/* ------------------------------------------------------------------------ */
/* Layout value                                                              */
/* ------------------------------------------------------------------------ */

#define LT_MAX_LEAVES 32
#define LT_MAX_NODES 64

/*
 * A Shape:Stride layout [P1 "A layout is a shape and a stride"; P2 3.5.3;
 * P4 "The formula gets a name"]: a function from coordinates to offsets,
 * offset = sum over leaves of coordinate * stride. Shape and stride are
 * congruent trees [P4 "A shape is a tree"; P2 3.5.4]; they share one tree
 * here, stored in preorder:
 *   tree[i] == 0 : a leaf; its extent and stride are the next entries of
 *                  shape[] and stride[] (leaves are numbered left to right);
 *   tree[i] == k : a tuple of k >= 1 children, which follow in preorder.
 * nnodes entries of tree[] and nleaves entries of shape[]/stride[] are used.
 * The root may be a single leaf ("8:1"), else a tuple whose children are the
 * top-level modes. Extents are >= 1, strides >= 0 (negative strides are
 * rejected: a reading, the pages use none).
 */
typedef struct lt_layout {
    int32_t nleaves;
    int32_t nnodes;
    int64_t shape[LT_MAX_LEAVES];
    int64_t stride[LT_MAX_LEAVES];
    int8_t tree[LT_MAX_NODES];
} lt_layout;

/* Check that L is well formed: the tree is consistent and shape and stride
 * are congruent [P4 "A shape is a tree"; P2 3.5.4], extents >= 1, strides
 * >= 0. Returns LT_OK or LT_ERR_INVALID_LAYOUT; writes nothing. */
lt_status lt_layout_validate(const lt_layout* L);

/* Parse the printed form, e.g. "((16,16),(16,8)):((128,1),(2048,16))".
 * Spaces and the '_' marks of static integers [P1 "Results"] are ignored. */
lt_status lt_layout_parse(const char* text, lt_layout* out);

/* Print L as shape:stride with no spaces into buf (NUL-terminated). *needed
 * (optional) receives the length including the NUL; if cap is too small the
 * call returns LT_ERR_CAPACITY and writes nothing to buf. */
lt_status lt_layout_format(const lt_layout* L, char* buf, size_t cap, size_t* needed);

/* A flat layout with `rank` leaves as its top-level modes (rank 1 gives a
 * bare "s:d" root): the make_layout(make_shape(...), make_stride(...)) of the
 * pages [P2 3.5.3; P1 "Two programs: the algebra, then the GEMM"]. shape and
 * stride are host arrays of `rank` entries; 1 <= rank <= LT_MAX_LEAVES, else
 * LT_ERR_INVALID_ARGUMENT; a negative extent or stride gives
 * LT_ERR_INVALID_LAYOUT. */
lt_status lt_make_layout(int32_t rank, const int64_t* shape, const int64_t* stride, lt_layout* out);

/* Compact strides: first mode fastest (the natural, colexicographic default
 * [P2 3.5.3-3.5.4]) or last mode fastest (row-major [P2 3.5.3]). */
lt_status lt_make_colmajor(int32_t rank, const int64_t* shape, lt_layout* out);
lt_status lt_make_rowmajor(int32_t rank, const int64_t* shape, lt_layout* out);

/* Concatenate n layouts as the top-level modes of a new layout: shapes and
 * strides nest, so a mode may itself be a tuple [P4 "A shape is a tree"; P3
 * "CuTe: layouts as functions"]. LT_ERR_CAPACITY if the result needs more
 * than LT_MAX_LEAVES leaves or LT_MAX_NODES nodes. */
lt_status lt_make_tuple(int32_t n, const lt_layout* modes, lt_layout* out);

/* Top-level mode i of L (a leaf root has one mode, itself): CuTe's
 * layout<i>, e.g. the tile and tile-grid modes of a zipped divide [P1 "A
 * layout is a shape and a stride"]. LT_ERR_INVALID_ARGUMENT if i < 0 or
 * i >= rank. */
lt_status lt_mode(const lt_layout* L, int32_t i, lt_layout* out);

/* size = product of extents; cosize = largest offset reached + 1, the memory
 * footprint [P2 3.5.5]; rank = number of top-level modes; depth = tuple
 * nesting depth (0 for a leaf root). */
lt_status lt_size(const lt_layout* L, int64_t* out);
lt_status lt_cosize(const lt_layout* L, int64_t* out);
lt_status lt_rank(const lt_layout* L, int32_t* out);
lt_status lt_depth(const lt_layout* L, int32_t* out);

/* Evaluate at a 1-D index, unravelled first-leaf-fastest (colexicographic)
 * [P4 "The formula gets a name"; P2 3.5.4]. idx must be in [0, size). */
lt_status lt_eval_index(const lt_layout* L, int64_t idx, int64_t* offset);

/* Evaluate at a coordinate. ncoord == rank: one integer per top-level mode,
 * each unravelled colexicographically inside its mode. ncoord == nleaves: a
 * natural coordinate, one integer per leaf. Each entry must lie inside its
 * (mode's or leaf's) extent. */
lt_status lt_eval_coord(const lt_layout* L, const int64_t* coord, int32_t ncoord, int64_t* offset);

/* coalesce [P4 "A shape is a tree"; P2 3.5.6]: flatten, drop extent-1 leaves,
 * merge s0:d0 followed by s1:(s0*d0) into (s0*s1):d0. The result has a leaf
 * root if one leaf remains, else a flat tuple; an all-extent-1 layout gives
 * 1:0. */
lt_status lt_coalesce(const lt_layout* L, lt_layout* out);

/* composition A o B [P4 "Composition, worked by hand"; P1 "A layout is a
 * shape and a stride"]: the layout R with B's mode tree (each leaf of B may
 * become a tuple) such that R(x) == A(B(x)) for every x < size(B). Built by
 * walking each leaf of B through A's coalesced leaves. LT_ERR_NOT_ADMISSIBLE
 * when no such layout exists, including when B reaches outside [0, size(A))
 * (a reading: A's last mode is not extended). A leaf of B with extent 1
 * gives 1:0, a leaf with stride 0 gives s:0. */
lt_status lt_compose(const lt_layout* A, const lt_layout* B, lt_layout* out);

/* complement of B in [0, M) [P4 "Divide is tiling"]: the layout B* with
 * strictly increasing values and B*(0) == 0 such that the pair (B, B*) hits
 * every integer of [0, M) exactly once (a reading of "everything B misses";
 * stride-0 leaves of B are ignored). Coalesced. LT_ERR_NOT_ADMISSIBLE if no
 * such layout exists. */
lt_status lt_complement(const lt_layout* B, int64_t M, lt_layout* out);

/* logical_divide(A, B) = A o (B, complement(B, size(A))) [P4 "Divide is
 * tiling"; P1 "A layout is a shape and a stride"; P2 3.5.6]. Mode 0 is inside
 * the tile, mode 1 picks the tile. size(B) must divide size(A)
 * (LT_ERR_NOT_DIVISIBLE otherwise). */
lt_status lt_logical_divide(const lt_layout* A, const lt_layout* tiler, lt_layout* out);

/* The same division by a shape tiler applied mode by mode: tiler[i] divides
 * top-level mode i of A by the layout tiler[i]:1, for i < n (n <= rank);
 * modes past n are kept whole. Result mode i is (in-tile, tile-index). */
lt_status lt_logical_divide_shape(const lt_layout* A, int32_t n, const int64_t* tiler, lt_layout* out);

/* logical_product(A, B) = (A, complement(A, size(A)*cosize(B)) o B) [P4
 * "Divide is tiling": the mirror of the divide, which lays copies of a tile
 * out in a pattern of repetition; the formula is a reading that mirrors the
 * divide's A o (B, B*)]. Mode 0 is A; mode 1 places copy j of A at offset
 * A*(B(j)), in the room A leaves free. E.g. (2,2):(1,2) by 3:1 gives
 * ((2,2),3):((1,2),4). LT_ERR_NOT_ADMISSIBLE when A's complement in
 * [0, size(A)*cosize(B)) does not exist (A's footprint must divide it). */
lt_status lt_logical_product(const lt_layout* A, const lt_layout* B, lt_layout* out);

/* Thread-value layout [P4 "The threads are a layout too"]: for a
 * column-major tile whose mode i has extent thr[i]*val[i], the layout
 * ((T_0..T_n-1),(V_0..V_n-1)) -> offset in the tile (for n == 1 simply
 * (T,V)). Per mode, blocked[i] == 0 interleaves the threads (thread t takes
 * t, t+T, t+2T, ...: logical_product(T:1, V:1) = (T,V):(1,T)); blocked[i] != 0
 * gives each thread a run of V (logical_product(V:1, T:1) with its modes
 * swapped = (T,V):(V,1)). The page's two examples for 8 threads and 32 values
 * are (8,4):(1,8) and (8,4):(4,1). blocked may be NULL (all interleaved).
 * 1 <= n <= 8. */
lt_status lt_make_tv_layout(int32_t n, const int64_t* thr, const int64_t* val, const uint8_t* blocked,
                            lt_layout* out);

/* zipped_divide [P1 "A layout is a shape and a stride"]: the shape-tiler
 * division regrouped so that mode 0 gathers all in-tile modes and mode 1 all
 * tile-index modes (plus untiled modes). E.g. (256,128):(128,1) by (16,16)
 * gives ((16,16),(16,8)):((128,1),(2048,16)). */
lt_status lt_zipped_divide(const lt_layout* A, int32_t n, const int64_t* tiler, lt_layout* out);

/* local_tile [P4 "The kernel, in three lines"; P2 3.5.6-3.5.7]: zipped_divide
 * A by the tiler, then fix the tile-index mode at coord. coord[i] < 0 stands
 * for CuTe's '_' and keeps that tile-index mode free; free modes follow the
 * in-tile modes in the result. step (optional, n entries of 0/1, CuTe's Step)
 * selects which of the n tiler modes apply to A; the selected count must be
 * rank(A). The tile's elements are at *offset + out(x). */
lt_status lt_local_tile(const lt_layout* A, int32_t n, const int64_t* tiler, const int64_t* coord,
                        const uint8_t* step, int64_t* offset, lt_layout* out);

/* local_partition [P4 "The kernel, in three lines"; P2 3.5.6-3.5.7]: thread
 * t's share of the tile T under the thread layout thr. T is zipped-divided by
 * the per-mode sizes of thr; the in-tile mode is fixed at thread t's
 * coordinate (the coordinate that thr maps to t; thr must be a bijection onto
 * [0, size(thr))) and the tile-index mode is kept. step (optional, rank(thr)
 * entries) selects which thread modes partition T. The thread's elements are
 * at *offset + out(x). */
lt_status lt_local_partition(const lt_layout* T, const lt_layout* thr, int64_t t, const uint8_t* step,
                             int64_t* offset, lt_layout* out);

/* ------------------------------------------------------------------------ */
/* Device and architecture                                                  */
/* ------------------------------------------------------------------------ */

/* Check that the current HIP device is gfx950 and record its properties.
 * Runs once per device before anything is launched or allocated [P1
 * "Results": refuse before any allocation]. Returns LT_ERR_ARCH_MISMATCH on
 * another architecture. `arch_out` (optional, cap bytes) receives the
 * device's gcnArchName. */
lt_status lt_device_check(char* arch_out, size_t cap);

/* Test hook: when non-NULL, the library uses this architecture name instead
 * of querying the device (so the refusal path can be exercised without a
 * GPU). NULL restores the real query. Not thread-safe; for tests only. */
lt_status lt_set_arch_override(const char* arch);

/* Device layout maps (the bit-exact layout parity path) [P1 "Two programs:
 * the algebra, then the GEMM" and "Results": a gather through the same layout
 * on the device]. For x < n (n <= size(L)):
 *   lt_layout_eval_device: out[x] = L(x)            (out: n int64 on device)
 *   lt_gather_device:      dst[x] = src[L(x)]       (elem_bytes in {1,2,4,8};
 *                          src must hold cosize(L) elements) */
lt_status lt_layout_eval_device(const lt_layout* L, int64_t* d_out, int64_t n, void* stream);
lt_status lt_gather_device(const lt_layout* L, const void* d_src, void* d_dst, int32_t elem_bytes,
                           int64_t n, void* stream);

/* ------------------------------------------------------------------------ */
/* GEMM                                                                      */
/* ------------------------------------------------------------------------ */

typedef enum lt_dtype { LT_F16 = 1, LT_BF16 = 2 } lt_dtype;

/* A tensor is a pointer plus a layout: a zero-copy view [P2 3.5.7; P3 "CuTe:
 * layouts as functions"]. For the GEMM, A is (M,K), B is (K,N), C and D are
 * (M,N): rank-2 layouts in elements whose two modes each coalesce to a single
 * stride. An operand is named by its stride-1 mode [P4 "One notation, and no
 * more transposes"]: A K-major or M-major, B K-major or N-major, C/D N-major
 * or M-major. */
typedef struct lt_tensor {
    void* ptr;
    int32_t dtype;     /* lt_dtype */
    int32_t reserved;
    lt_layout layout;
} lt_tensor;

/* Kernel families the planner can choose. */
typedef enum lt_kernel {
    LT_KERNEL_AUTO = 0,
    LT_KERNEL_WAVE16 = 1,   /* one wave per 16x16 tile, any layout/ragged shape */
    LT_KERNEL_TILED = 2,    /* 256x256x64 block tile, LDS double buffer, 16x16x32 MFMA, ragged edges predicated */
    LT_KERNEL_SKINNY = 3    /* M <= 32, K-major B streamed once, split-K */
} lt_kernel;

/* Optional planner overrides; zero fields mean "choose". */
typedef struct lt_gemm_options {
    int32_t kernel;     /* lt_kernel */
    int32_t tile_m;     /* block tile (kernel-specific allowed values; TILED: 256x256,
                           256x128 or 128x128, the last never split nor persistent) */
    int32_t tile_n;
    int32_t split_k;    /* SKINNY: number of K slices (>= 1). TILED: K segments of each
                           tile past the last whole round of 256 CUs (0: chosen by a
                           cost model; 1: none, all tiles whole; > 1: forced, on all
                           tiles when they fill no whole round) */
    int32_t persistent; /* TILED: 0 = chosen (persistent when the tiles are whole, K
                           is a multiple of 64 with at least 4 slices, there are
                           more tiles than compute units, and for 256x256 tiles
                           beta = 0, no split remainder and K <= 4096; with beta != 0
                           also C's row stride below 2^27 elements); 1 = one workgroup
                           per tile; 2 = persistent (LT_ERR_UNSUPPORTED where the tile,
                           K, beta, C stride or split conditions fail) */
    int32_t tile_order; /* TILED, the data-parallel launch of 256x256 tiles: 0 = chosen
                           (super-blocks when a last-level-cache model of the two
                           orders, walked round by round, fetches at most 85 % as
                           many operand panels with them and a round's 32 panels fit
                           192 MiB); 1 = raster (groups of 8 tile rows, a stretch per
                           XCD); 2 = super-blocks: each round of 256 tiles a 16 x 16
                           block, each XCD an 8 x 4 part of it (LT_ERR_UNSUPPORTED
                           unless both tile counts are multiples of 16 and every tile
                           is whole, unsplit and not persistent); 3 = raster with the
                           odd rounds walking K downward (chosen where a round's 32
                           panels exceed 192 MiB; LT_ERR_UNSUPPORTED unless K is a
                           multiple of 64, the tiles unsplit, not persistent and more
                           than one round) */
} lt_gemm_options;

/* What the planner chose, for banners and tests [P1 "Exercise": print the
 * tile, warp tile and shared-memory figures]. */
typedef struct lt_gemm_plan_info {
    int32_t kernel;          /* lt_kernel */
    int32_t tile_m, tile_n, tile_k;
    int32_t wave_m, wave_n;  /* tile of one wave (TILED: of the data-parallel launch) */
    int32_t waves;           /* waves per workgroup (TILED: 4, one per SIMD, in the data-parallel
                                launch; the split launch runs 8 waves of 64x128) */
    int32_t stages;          /* LDS pipeline depth */
    int32_t split_k;
    int32_t a_kmajor, b_kmajor, d_nmajor;
    int64_t grid;            /* workgroups launched (all launches) */
    int64_t lds_bytes;       /* per workgroup (TILED: of the persistent or data-parallel launch, its
                                staging region for D beside the LDS ring included) */
    int64_t workspace_bytes; /* caller-provided scratch the run needs */
    int64_t mfma_per_wave_kstep; /* MFMA instructions per wave per K step (tile_k) */
    int32_t mfma_m, mfma_n, mfma_k; /* shape of the MFMA instruction the kernel issues */
    int64_t sk_tiles;        /* TILED: tiles of the last round split into split_k K segments, 0 if none */
    int32_t sk_workgroups;   /* TILED: workgroups of the split launch (sk_tiles * split_k) */
    int64_t tiles;           /* output tiles of the block tiling (TILED: one workgroup per tile,
                                plus split_k - 1 more per split tile, unless persistent) */
    int32_t persistent;      /* TILED: 1 if one workgroup per compute unit walks a list of
                                tiles ["CUTLASS, in depth", "Kernel schedules"]; grid is
                                then the workgroup count. A fused epilogue (lt_gemm_run_ex)
                                runs one workgroup per tile instead. */
    int32_t tile_order;      /* TILED data-parallel launch: 1 raster, 2 super-blocks, 3 raster
                                with odd rounds K-reversed; 0 for the other kernels and the
                                persistent launch */
} lt_gemm_plan_info;

/* Validate and plan without launching: the can_implement half of the
 * pages' check [P3 "A complete Hopper GEMM with the builder API"; P1
 * "Pitfalls"]. Checks: dtypes (A, B fp16 or bf16
 * alike; C and D of one 16-bit type), shapes (A (M,K), B (K,N), C/D (M,N)),
 * each mode a single stride, a stride-1 mode per operand, 16-byte aligned
 * bases and other strides a multiple of 8 elements (LT_ERR_MISALIGNED_OPERAND),
 * D not overlapping A or B (D may equal C). C may be NULL when beta == 0
 * (pass beta_nonzero = 0). */
lt_status lt_gemm_plan(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D,
                       int32_t beta_nonzero, const lt_gemm_options* opt, lt_gemm_plan_info* info);

/* CUTLASS-style split of the same check [P3 "A complete Hopper GEMM with the
 * builder API"]: can_implement, then the workspace size the run needs. */
lt_status lt_gemm_can_implement(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C,
                                const lt_tensor* D, int32_t beta_nonzero, const lt_gemm_options* opt);
lt_status lt_gemm_workspace_size(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C,
                                 const lt_tensor* D, int32_t beta_nonzero, const lt_gemm_options* opt,
                                 size_t* bytes);

/* D = alpha * A*B + beta * C [P3 "The problem CUTLASS solves"], fp32
 * accumulation, fp32 epilogue, output rounded to nearest even. beta == 0
 * never reads C (C may be NULL). M == 0 or N == 0 does nothing; K == 0 gives
 * D = beta*C. `workspace` is caller-owned device memory of at least the
 * planned workspace_bytes, 256-byte aligned (may be NULL when that is 0;
 * LT_ERR_WORKSPACE otherwise). Its contents need no initialisation, but two
 * runs in flight at once must not share it. Asynchronous on
 * `stream`. */
lt_status lt_gemm_run(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D,
                      float alpha, float beta, const lt_gemm_options* opt, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Fused epilogue [P3 "Epilogue fusion": bias, activation and an absolute
 * maximum computed on the accumulators while they are in registers, instead
 * of a second pass over D through HBM]:
 *   D = act(alpha * A*B + beta * C + bias), in fp32, rounded once.
 * bias: device pointer or NULL, values of D's dtype; bias[n * bias_stride] is
 * added to column n (bias_per_row == 0) or bias[m * bias_stride] to row m
 * (bias_per_row != 0); bias_stride 0 means 1. Caller-owned, N (or M) values.
 * activation: LT_ACT_NONE, LT_ACT_RELU (x > 0 ? x : 0) or LT_ACT_GELU
 * (x * Phi(x) = 0.5 x (1 + erf(x / sqrt(2))), the standard normal CDF form;
 * the pages name GELU without a formula).
 * amax: device pointer or NULL; receives max |D| over the stored (rounded)
 * outputs, NaN outputs ignored. The library clears it on the stream first, so
 * concurrent runs must not share it. */
typedef enum lt_activation { LT_ACT_NONE = 0, LT_ACT_RELU = 1, LT_ACT_GELU = 2 } lt_activation;

typedef struct lt_epilogue {
    const void* bias;
    int64_t bias_stride;
    int32_t bias_per_row;
    int32_t activation;      /* lt_activation */
    float* amax;
} lt_epilogue;

/* lt_gemm_run with a fused epilogue (epi may be NULL: exactly lt_gemm_run).
 * LT_ERR_INVALID_ARGUMENT for an unknown activation or a negative
 * bias_stride. Every kernel family takes it; the same plan as lt_gemm_run. */
lt_status lt_gemm_run_ex(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D,
                         float alpha, float beta, const lt_gemm_options* opt, const lt_epilogue* epi,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device scratch array of lt_gemm_run_noalloc, per GPU: 64 MiB
 * for split-K partials plus 4 KiB for arrival counters. Every plan the
 * automatic choice makes fits (a split remainder has at most 256 segments of
 * 256x256 fp32 partials; the skinny split needs under 2 MiB); forced splits
 * may not. */
#define LT_NOALLOC_SCRATCH_BYTES ((size_t)64 * 1024 * 1024 + 4096)

/* lt_gemm_run_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same plan and kernels, with the scratch they need (split-K partials
 * and arrival counters) taken from a static device array of
 * LT_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; no workspace argument, and no device memory is
 * allocated or freed by the call. LT_ERR_WORKSPACE if the plan needs more
 * scratch than that (nothing is launched). What must start at zero is
 * cleared on the stream by the call itself; the array keeps the last call's
 * contents. Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams, or from different threads
 * without ordering) race and give wrong results. Asynchronous on `stream`. */
lt_status lt_gemm_run_noalloc(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D,
                              float alpha, float beta, const lt_gemm_options* opt, const lt_epilogue* epi,
                              void* stream);

/* Library version string (static storage, never NULL). The pages' kernels
 * carry their architecture in the build [P1 "Results"]; this library is built
 * for gfx950 only, and the string names that target. */
const char* lt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LT_H_ */
