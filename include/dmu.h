/*
 * dmu.h -- dense matrix-unit GEMM on AMD Instinct MI355X (gfx950), C ABI.
 *
 * The library computes the tiled dense product
 *
 *     D[b] = A[b] * B[b] + C[b]        for b = 0 .. batch-1
 *
 * on the chip's matrix cores (MFMA), with fp16/bf16 inputs and fp32
 * accumulation, an fp16-output ("fp16 accumulate") variant, an int8 -> int32
 * variant and FP8 e4m3 inputs with fp32 accumulation.
 *
 * Sources for the operation and its conventions:
 *   - "Tensor Cores, CUTLASS and CuTe", section 2.1 (one matrix instruction is
 *     D = A*B + C with low-precision inputs and an fp32/int32 accumulator; the
 *     table of input/accumulator type pairs, including fp16 accumulation and
 *     int8 -> int32 and e4m3 -> fp32), section 4.1 (the 4096^3 bf16 problem: bf16 in, fp32
 *     accumulate, bf16 out; "TN" = A row-major M x K, B stored N x K row-major),
 *     section 4.4 (the host entry point checks device, type, rank and
 *     contiguity before it reinterprets untyped pointers) and section 7 (the
 *     strided-batched BLAS form alpha*A*B + beta*C); section 6.5 (FP8 GEMMs:
 *     a K-tile of 128 one-byte values moves the bytes of 64 bf16 values).
 *   - "hgemm_mma_m16n8k16_mma2x4_warp4x4_kernel" walkthrough, section 1.1
 *     (C = A x B with A M x K and B K x N, both row-major: "NN").
 *   - Layout-experiment post (KingOfEgg, RTX 5080), section 3 (D = A x B + C;
 *     an fp32 accumulator is the floor for long sums).
 *
 * Every entry point is a plain C function on plain pointers and sizes.  Device
 * buffers are owned by the caller; the library allocates no device memory,
 * keeps no pointer after a call returns, and has no mutable global state other
 * than a thread-local error message.  All entry points are thread-safe.
 */
#ifndef DMU_H
#define DMU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum {
    DMU_F16 = 1,  /* IEEE binary16                       */
    DMU_BF16 = 2, /* bfloat16 (upper half of a binary32) */
    DMU_F32 = 3,  /* IEEE binary32                       */
    DMU_I8 = 4,   /* signed 8-bit integer                */
    DMU_I32 = 5,  /* signed 32-bit integer               */
    DMU_E4M3 = 6  /* FP8 e4m3: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
                     no infinities, S.1111.111 is NaN, largest finite 448   */
} dmu_dtype;

/* Storage order of a logical matrix X(r, c) with leading dimension ld (elements):
 *   DMU_ROW_MAJOR: X(r, c) is at r*ld + c,   ld >= max(1, cols)
 *   DMU_COL_MAJOR: X(r, c) is at r + c*ld,   ld >= max(1, rows)            */
typedef enum { DMU_ROW_MAJOR = 0, DMU_COL_MAJOR = 1 } dmu_layout;

/* Return codes.  Argument errors are reported before any HIP call is made. */
typedef enum {
    DMU_OK = 0,
    DMU_ERR_INVALID_ARG = -1, /* bad size, pointer, leading dimension, stride or overlap */
    DMU_ERR_UNSUPPORTED = -2, /* a type/variant the library does not implement          */
    DMU_ERR_HIP = -3          /* the HIP runtime reported an error for a launch         */
} dmu_status;

/*
 * One (optionally strided-batched) product.
 *
 *  M, N, K, batch   sizes, each >= 0.  M, N or batch == 0: nothing is done.
 *                   K == 0: D = C (or 0 when C is NULL).
 *  in_type          type of A and B: DMU_F16, DMU_BF16, DMU_I8 or DMU_E4M3.
 *  acc_type         accumulator: DMU_F32 (fp16/bf16/e4m3 in), DMU_F16 (fp16
 *                   in, "fp16 accumulate") or DMU_I32 (int8 in).
 *  out_type         type of C and D.  Supported (in, acc, out) triples:
 *                     (F16,F32,F32) (F16,F32,F16) (F16,F16,F16)
 *                     (BF16,F32,BF16) (BF16,F32,F32) (I8,I32,I32)
 *                     (I8,I32,F32) (I8,I32,F16) (I8,I32,BF16)
 *                     (E4M3,F32,F32) (E4M3,F32,F16) (E4M3,F32,BF16)
 *                   The last three dequantise: the int32 sum is converted
 *                   to fp32 (round to nearest even), goes through the
 *                   optional epilogue of dmu_gemm_ex in fp32, and is rounded
 *                   to the output type.
 *                   For acc_type == DMU_F16 the matrix cores still sum the
 *                   exact products in fp32 and the result is rounded once to
 *                   fp16 (gfx950 has no fp16-accumulating matrix
 *                   instruction); this is at least as accurate as a true fp16
 *                   accumulation.
 *  layout_a/_b      storage order of A (logical M x K) and B (logical K x N).
 *                   Row-major B is the "NN" case, column-major B (B stored as
 *                   an N x K row-major array) the "TN" case.
 *  A, lda, stride_a device pointer, leading dimension and batch stride, in
 *  B, ldb, stride_b elements.  Strides >= 0 (0 broadcasts one matrix to every
 *                   batch).  Any element-aligned pointer and any leading
 *                   dimension satisfying the layout rule is accepted; the
 *                   library picks the widest legal vector access.
 *  C, ldc, stride_c optional addend (NULL => 0), row-major M x N of out_type,
 *                   ldc >= N.  C may be the same buffer as D with the same ldc
 *                   and stride (in-place accumulate), but may not partially
 *                   overlap it.
 *  D, ldd, stride_d output, row-major M x N of out_type, ldd >= N.  For
 *                   batch > 1, stride_d >= (M-1)*ldd + N so batches do not
 *                   overlap.  D may not overlap A or B.
 *
 * Rounding: fp32 -> fp16/bf16 output conversion is round-to-nearest-even;
 * subnormal inputs and outputs are kept (not flushed).  int32 results wrap
 * modulo 2^32 (no overflow is possible for K <= 2^17).
 * M, N, K and batch must each be below 2^31 (larger: DMU_ERR_UNSUPPORTED).
 */
typedef struct dmu_gemm_args {
    int64_t M, N, K, batch;
    int32_t in_type, acc_type, out_type; /* dmu_dtype  */
    int32_t layout_a, layout_b;          /* dmu_layout */
    const void *A;
    int64_t lda, stride_a;
    const void *B;
    int64_t ldb, stride_b;
    const void *C;
    int64_t ldc, stride_c;
    void *D;
    int64_t ldd, stride_d;
} dmu_gemm_args;

/*
 * D = A*B + C as described above, enqueued on `stream` (a hipStream_t; NULL is
 * the default stream).  Asynchronous: returns once the kernel is launched.
 * Errors: DMU_ERR_INVALID_ARG / DMU_ERR_UNSUPPORTED before any HIP call (the
 * message is in dmu_last_error()); DMU_ERR_HIP if the launch fails.  Nothing
 * is written to D when an error is returned before the launch.
 */
int dmu_gemm(const dmu_gemm_args *args, void *stream);

/*
 * Fused epilogue ("Tensor Cores, CUTLASS and CuTe", section 5: the scaled-mm
 * epilogue multiplies the accumulator by a per-column and a per-row scale
 * before the output conversion, as for int8 dequantisation; section 7: the
 * bias + activation epilogue of a fused linear layer).  With P the product sum
 * (the fp32 accumulator, or the int32 one converted to fp32):
 *
 *     D[b](i,j) = round_out( act( rs[b](i) * cs[b](j) * P + bias[b](j) + C[b](i,j) ) )
 *
 * evaluated in fp32 in that order and rounded once to the output type.
 *
 *  row_scale        M floats per batch slice (NULL: 1); slice b starts at
 *                   row_scale + b * stride_row_scale (stride >= 0, 0 shares
 *                   one vector across batches).
 *  col_scale        N floats per batch slice (NULL: 1), likewise.
 *  bias             N floats per batch slice (NULL: 0), likewise.
 *  act              DMU_ACT_NONE, DMU_ACT_RELU (x > 0 ? x : +0) or
 *                   DMU_ACT_GELU_TANH (0.5 x (1 + tanh(sqrt(2/pi)(x + 0.044715 x^3)))).
 *
 * Vectors are device pointers aligned to 4 bytes, read only, and may not
 * overlap D.  int32 output takes no epilogue (DMU_ERR_UNSUPPORTED).
 */
enum { DMU_ACT_NONE = 0, DMU_ACT_RELU = 1, DMU_ACT_GELU_TANH = 2 };

typedef struct dmu_epilogue {
    const float *row_scale;
    int64_t stride_row_scale;
    const float *col_scale;
    int64_t stride_col_scale;
    const float *bias;
    int64_t stride_bias;
    int32_t act;
} dmu_epilogue;

/*
 * D = epilogue(A*B + C) as described above, on `stream`; `ep` may be NULL (then
 * exactly dmu_gemm).  Errors as for dmu_gemm, plus DMU_ERR_INVALID_ARG for a bad
 * activation, a negative stride, a misaligned vector or one that overlaps D.
 */
int dmu_gemm_ex(const dmu_gemm_args *args, const dmu_epilogue *ep, void *stream);

/* Validate `args` and `ep` exactly as dmu_gemm_ex does, without touching the GPU. */
int dmu_gemm_ex_check(const dmu_gemm_args *args, const dmu_epilogue *ep);

/*
 * Persistent stream-K schedule of the same product ("Tensor Cores, CUTLASS and
 * CuTe", section 6.5: a persistent tile scheduler launches a fixed number of
 * blocks that loop over the work, instead of one block per output tile;
 * section 4.5 lists the one-block-per-tile dispatch among its kernel's gaps).
 *
 * One workgroup per compute unit ("worker") shares the tiles x K-tiles
 * multiply-accumulate iterations of the tiled kernel evenly, so that a tile
 * count that does not fill the compute units (or leaves a partial last wave)
 * still keeps every unit busy.  A tile split between workers is completed by
 * the worker that holds its last K-tile, which adds the others' fp32/int32
 * partial sums in a fixed order: results are reproducible launch to launch,
 * and equal to dmu_gemm_ex's within the accumulation-order tolerance (bit for
 * bit for int8 and for exactly representable sums).
 *
 *  args, ep        as for dmu_gemm_ex (same validation, same results).
 *  workspace       device memory of at least dmu_gemm_streamk_workspace_size
 *                  bytes, 256-byte aligned, owned by the caller, not overlapping
 *                  any operand.  It must be zero-filled before its first use;
 *                  every call leaves its flag words zero again, so one
 *                  workspace serves any number of calls in stream order.  Calls
 *                  that overlap in time (several streams) need separate
 *                  workspaces.  Layout: an error word (the first 32-bit word;
 *                  bytes 0-255 are reserved for it), one 32-bit flag per
 *                  worker from byte 256, then one slot of partial sums per
 *                  worker from the next multiple of 256 bytes.  Each wait of a
 *                  worker for another is bounded; a wait that runs past its
 *                  limit (not expected: every worker is resident) sets the
 *                  error word and the kernel completes with a WRONG result.
 *                  The launch itself still returns DMU_OK (it is
 *                  asynchronous): query dmu_gemm_streamk_error after the
 *                  call; when it reports a failure, discard D and zero-fill
 *                  the workspace again before its next use.
 *  workspace_bytes its size.
 * The schedule is used where it pays: when the data-parallel kernel's tiles
 * fill less than 80 % of its waves of one workgroup per compute unit (60 %
 * where its tiles are 64 x 128, which already spread few tiles over more
 * units; few tiles, long K).  Otherwise -- and for products that only the fallback kernel
 * can read, and K == 0 -- the call runs the data-parallel kernel and uses no
 * workspace (its size is then 0).  The environment variable DMU_STREAMK=always
 * or =never overrides the choice.
 * Returns DMU_ERR_INVALID_ARG for a missing, misaligned, small or overlapping
 * workspace, and DMU_ERR_HIP if the device cannot be queried or the launch
 * fails; otherwise as dmu_gemm_ex.
 */
int dmu_gemm_streamk(const dmu_gemm_args *args, const dmu_epilogue *ep, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Whether a wait inside an earlier dmu_gemm_streamk call on `workspace` ran
 * past its limit (so that call's D is wrong).  Waits for `stream` (the stream
 * of those calls; NULL is the default stream), then reads the workspace's
 * error word: *failed = 1 if it is set, else 0.  The word stays set until the
 * caller zero-fills the workspace.  `workspace` is a device pointer, 256-byte
 * aligned, or NULL for the library scratch of dmu_gemm_streamk_noalloc on the
 * current device (the last such call's word); `failed` a host pointer owned
 * by the caller.  Returns DMU_OK, DMU_ERR_INVALID_ARG for a NULL `failed` or a
 * misaligned workspace (before any HIP call), or DMU_ERR_HIP if the copy or
 * the synchronisation fails.
 */
int dmu_gemm_streamk_error(const void *workspace, void *stream, int *failed);

/*
 * dmu_gemm_streamk without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * schedule's error word, flags and partial sums live in a scratch array that
 * the library holds in device memory, DMU_STREAMK_SCRATCH_BYTES on each GPU it
 * runs on, until the process ends.  Same arguments, validation, choice of
 * schedule and results as dmu_gemm_streamk (bit for bit: the same kernels on
 * the same workspace layout).  Each call first clears the scratch's error word
 * and flags with a small kernel on `stream` (no hipMemsetAsync, so the call can
 * be captured), then runs the schedule.  The first call on a device asks the
 * runtime for that device's address of the array.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (several streams, several host threads) race and give wrong
 * results; serialise them (one stream) or use dmu_gemm_streamk with separate
 * workspaces.  dmu_gemm_streamk_error(NULL, stream, &failed) reports whether
 * the last call's waits gave up.
 * Returns DMU_ERR_UNSUPPORTED when the schedule would need more than
 * DMU_STREAMK_SCRATCH_BYTES (more than 256 workers of 256 x 128 tiles); no
 * memory is allocated on any path.  Otherwise as dmu_gemm_streamk.
 */
#define DMU_STREAMK_SCRATCH_BYTES (33u * 1024u * 1024u)
int dmu_gemm_streamk_noalloc(const dmu_gemm_args *args, const dmu_epilogue *ep, void *stream);

/* Workspace bytes dmu_gemm_streamk needs for these arguments on the current
 * device (the worker count is the device's compute-unit count, at most the
 * number of iterations).  *bytes = 0 when none is needed.  Validation as for
 * dmu_gemm_check; DMU_ERR_HIP if the device cannot be queried. */
int dmu_gemm_streamk_workspace_size(const dmu_gemm_args *args, size_t *bytes);

/*
 * Validate `args` exactly as dmu_gemm does, without touching the GPU.
 * Returns DMU_OK or the error dmu_gemm would return before launching.
 */
int dmu_gemm_check(const dmu_gemm_args *args);

/*
 * Attention forward, fused on the matrix cores: for every batch slice b,
 *
 *     O[b] = softmax(scale * Q[b] K[b]^T) V[b]      (softmax over each row)
 *
 * The pages move the two products of this computation onto the matrix units
 * and keep P = softmax(S) in registers between them (layout-experiment post,
 * sections 1-2; "Tensor Cores, CUTLASS and CuTe", part 3 section 2: the
 * accumulator of S = Q K^T feeds O = P V, with each row's max and sum taken
 * across the lanes that share the row).  Here S never leaves the chip: each
 * workgroup walks the keys in blocks with a running row maximum and sum (the
 * online softmax), P is rounded to the input type for the P V product.
 *
 *  batch, seq_q, seq_k  sizes; batch and seq_q >= 0 (0: nothing is done),
 *                   seq_k >= 1.  Each below 2^31.
 *  head_dim         d of Q, K and V; 128 is supported.
 *  in_type          DMU_F16 or DMU_BF16 (Q, K, V).
 *  out_type         DMU_F32, DMU_F16 or DMU_BF16 (O); rounded once (RNE).
 *  scale            softmax scale (e.g. 1/sqrt(head_dim)), fp32.
 *  Q, ldq, stride_q row-major seq_q x head_dim, leading dimension and batch
 *  K, ldk, stride_k stride in elements (seq_k x head_dim for K and V);
 *  V, ldv, stride_v pointers and leading dimensions 16-byte aligned (ld a
 *                   multiple of 8 elements), strides >= 0.
 *  O, ldo, stride_o row-major seq_q x head_dim of out_type; rows 16-byte
 *                   aligned; may not overlap Q, K or V, nor its own batches.
 *
 * Errors as for dmu_gemm: DMU_ERR_INVALID_ARG / DMU_ERR_UNSUPPORTED before any
 * HIP call, DMU_ERR_HIP for a failed launch.  Asynchronous on `stream`.
 */
typedef struct dmu_attention_args {
    int64_t batch, seq_q, seq_k, head_dim;
    int32_t in_type, out_type; /* dmu_dtype */
    float scale;
    const void *Q;
    int64_t ldq, stride_q;
    const void *K;
    int64_t ldk, stride_k;
    const void *V;
    int64_t ldv, stride_v;
    void *O;
    int64_t ldo, stride_o;
} dmu_attention_args;

int dmu_attention(const dmu_attention_args *args, void *stream);

/* Validate `args` exactly as dmu_attention does, without touching the GPU. */
int dmu_attention_check(const dmu_attention_args *args);

/*
 * Name of the kernel variant dmu_gemm would launch for `args` -- in the manner
 * of the walkthrough's kernel name ("hgemm_mma_m16n8k16_mma2x4_warp4x4_kernel",
 * opening listing: the instruction shape, the instruction tiles per warp and
 * the warp tiles are spelled out in the name) -- as a static
 * string: "mfma_<tile>_<A mode>_<B mode>_<in>_<out>", e.g.
 * "mfma_256x256_k16_t16_bf16_bf16" -- 256 x 256 tiles, A K-contiguous with
 * 16-byte rows, B M/N-contiguous 16-bit -- or "mfma_generic64_any_any_f16_f32"
 * for the fallback; operand modes: k16 K-contiguous with 16-byte rows, kd
 * K-contiguous with 4-byte rows, t16 M/N-contiguous 16-bit, t8 M/N-contiguous
 * 8-bit), or NULL if the arguments are invalid or the call would
 * launch nothing.  The tile is 256 x 128 when N <= 128 < M; otherwise, when
 * 240 or more 256 x 256 tiles cover the problem, 256 x 256 if K spans more
 * than two 128-byte K-tiles and 256 x 128 if it spans at most two; 128 x 128
 * for smaller problems, and 64 x 128 when at most 128 tiles of 128 x 128
 * cover the problem (all batch slices) and A is K-contiguous (twice the
 * workgroups for few tiles); e4m3 never takes 256 x 256.  The environment
 * variable DMU_FORCE_KERNEL=256x256 | 256x256w4 | 256x128 | 128x128 | 64x128 |
 * generic overrides the choice ("256x256w4": the 256 x 256 tile on four
 * wavefronts of 128 x 128 with AGPR accumulators, 16-bit inputs -- int8 takes
 * 256x256 instead; never chosen by default; "64x128" applies to K-contiguous
 * A only).  Host-only; no GPU access.
 */
const char *dmu_gemm_kernel_name(const dmu_gemm_args *args);

/*
 * Phase log (diagnostics).  The layout-experiment post (KingOfEgg, section 1)
 * backs a kernel claim with profiler evidence that includes its duration, and
 * "Tensor Cores, CUTLASS and CuTe" section 4.5 explains its kernel's distance
 * from peak by where the time goes; this log says where one launch's time goes
 * per workgroup.  While a log is set, every launch of the process (dmu_gemm,
 * dmu_gemm_ex, dmu_gemm_streamk, dmu_gemm_streamk_noalloc, dmu_attention) has
 * thread 0 of each workgroup write one record of 8 uint64_t into it:
 *   [0] start, [1] end of the main loop (attention: of the last key block),
 *       [2] end of the stream-K partial sums (persistent kernel: after the
 *       next tile's first loads are issued; = [1] for the other kernels),
 *       [3] end of the epilogue or of the
 *       stream-K partial store -- the chip's 100 MHz constant clock
 *       (s_memrealtime); for a stream-K worker with several tiles, [1] and
 *       [2] are those of its last tile;
 *   [4] start, [5] end -- the shader clock counter (s_memtime);
 *   [6] HW_ID register (low 32 bits) and XCC_ID register (high 32 bits);
 *   [7] workgroup id (low 32 bits) and the K-tiles (attention: key blocks)
 *       of the record (high 32).
 * Records: one per workgroup of the one-workgroup-per-tile kernel (index =
 * workgroup id), one per tile of the persistent kernel (index = tile number),
 * one per worker of stream-K (index = worker number), one per workgroup of
 * the attention kernel; the fallback kernel writes none.  `device_log` is a device buffer of `records` x 64 bytes,
 * 8-byte aligned, owned by the caller, which must keep it alive while launches
 * that write it may run; NULL with 0 turns the log off (the default).  A launch
 * that would write more records than the log holds fails with
 * DMU_ERR_INVALID_ARG before any HIP call.  The setting is process-wide and
 * not synchronised with launches on other threads: a diagnostic for a single
 * caller.  Returns DMU_OK, or DMU_ERR_INVALID_ARG for a buffer without a
 * count, a count without a buffer, or a misaligned buffer.  Host-only.
 */
int dmu_phase_log(void *device_log, size_t records);

/*
 * Records the last launch wrote into the phase log (*records; 0 when the
 * log was off, the problem empty or the kernel the fallback) and how they are
 * indexed (*kind: 0 none, 1 one per workgroup of the one-per-tile kernel, 2
 * one per tile of the persistent kernel, 3 one per stream-K worker, 4 one per
 * workgroup of the attention kernel).  Both are
 * host pointers owned by the caller; DMU_ERR_INVALID_ARG if either is NULL.
 * Host-only.
 */
int dmu_phase_log_last(size_t *records, int *kind);

/*
 * Compute units and peak shader clock (kHz) of HIP device `device`, as the
 * runtime reports them -- the inputs of a dense peak derived on the machine
 * itself (compute units x clock x multiply-adds per clock and unit), the
 * derivation "Tensor Cores, CUTLASS and CuTe" makes in its opening section for
 * its own GPU (multiprocessors x tensor-core FMAs per clock x 2 x clock).  Both
 * outputs are host pointers owned by the caller.  Returns DMU_OK;
 * DMU_ERR_INVALID_ARG for a NULL output or a negative device (message in
 * dmu_last_error()); DMU_ERR_HIP when the runtime cannot answer (no such
 * device).  Initialises the HIP runtime; launches nothing.
 */
int dmu_device_info(int device, int *compute_units, int *max_clock_khz);

/* Static description of a return code.  The host entry point of "Tensor Cores,
 * CUTLASS and CuTe" section 4.4 rejects a bad call with a message before any
 * kernel runs; across a C ABI that is a status code (dmu_status) plus the
 * message below.  Host-only; no GPU access. */
const char *dmu_status_string(int status);

/* Detail of the last failing call on this thread ("" if none), the message
 * part of the error reporting described at dmu_status_string.  The pointer
 * stays valid until the next call into the library on this thread. */
const char *dmu_last_error(void);

/*
 * Single-wavefront layout probes (test support).
 *
 * The layout experiment (KingOfEgg, sections 4-7) pins the matrix
 * instruction's fragment ownership and the shared-memory fragment-load
 * protocol with one warp and hand-made data before they go into a big
 * kernel.  These probes do the same for the gfx950 instructions and the LDS
 * tile format the GEMM kernels use; each runs one wavefront of 64 lanes:
 *
 *  variant                  in0 (device)          in1 (device)       out (device)
 *  DMU_PROBE_MFMA_*         A, m x k row-major    B^T, n x k         raw accumulators,
 *                           (in_type bits)        row-major          [64 lanes][regs] 32-bit
 *  DMU_PROBE_LDS_READ_B128  LDS image, 4096 B     int32 byte         [64][16 bytes]
 *  DMU_PROBE_LDS_READ_TR16  LDS image, 4096 B     address per lane   [64][8 bytes]
 *  DMU_PROBE_LDS_READ_TR8   LDS image, 4096 B     address per lane   [64][8 bytes]
 *  DMU_PROBE_LDS_FRAG       32 x 128-byte tile,   unused             [64][2 row blocks][2 K-steps]
 *                           row-major (logical)                      [16 bytes]
 *  DMU_PROBE_LDS_FRAG_T     64 x 128 16-bit tile, unused             [64][8 column blocks][2 K-steps]
 *                           row-major (logical)                      [8 16-bit values]
 *  DMU_PROBE_LANE_SWAP      uint32[64]            unused             [64][4] 32-bit words
 *  DMU_PROBE_CVT_BF16/_F16  float32[256]          unused             [256] 16-bit patterns
 *
 *  MFMA_*: lane l loads its operand fragments straight from in0/in1 with the
 *    hypothesised mapping (X[row = l % m][k = (16 bytes / element) * (l / m) + s])
 *    and issues one MFMA with a zero accumulator; the caller checks every
 *    (lane, register) against the product.  MFMA_16x16x128_E4M3 takes 32 bytes
 *    per lane, the GEMM kernels' two 16-byte fragments of a 128-byte row: bytes
 *    16 (l / 16) .. +15 and 64 + 16 (l / 16) .. +15 of row l % 16.
 *  LDS_READ_*: the image is copied to LDS; lane l reads at in1[l] (masked to
 *    an aligned in-bounds address) with ds_read_b128 / ds_read_b64_tr_b16 /
 *    ds_read_b64_tr_b8.
 *  LDS_FRAG: the tile is stored with the tiled kernel's staging writes of a
 *    K-contiguous operand and read back with its fragment reads (rows 16 b +
 *    l % 16, bytes 64 ks + 16 (l / 16) .. +15).
 *  LDS_FRAG_T: the tile (K-rows x values) is stored with the tiled kernel's
 *    staging writes of an M/N-contiguous operand and read back with its
 *    transposing fragment reads (column 16 b + l % 16, k = 32 ks + 8 (l / 16)
 *    + 0..7).
 *  LANE_SWAP: lane l passes in0[l] as both operands of v_permlane16_swap and
 *    of v_permlane32_swap and writes the two results of each (the attention
 *    kernel's row max reads the pair as {value of lane l, of lane l^16 / l^32}).
 *  CVT_*: the GEMM epilogue's fp32 -> bf16 / fp16 conversion.
 * dmu_probe_info() reports m, n, k, the input type and the number of 32-bit
 * output words per lane.  `stream` as for dmu_gemm.
 */
enum {
    DMU_PROBE_MFMA_32x32x16_BF16 = 1,
    DMU_PROBE_MFMA_32x32x16_F16 = 2,
    DMU_PROBE_MFMA_16x16x32_BF16 = 3,
    DMU_PROBE_MFMA_16x16x32_F16 = 4,
    DMU_PROBE_MFMA_32x32x32_I8 = 5,
    DMU_PROBE_MFMA_16x16x64_I8 = 6,
    DMU_PROBE_MFMA_16x16x128_E4M3 = 7,
    DMU_PROBE_LDS_READ_B128 = 10,
    DMU_PROBE_LDS_READ_TR16 = 11,
    DMU_PROBE_LDS_FRAG = 12,
    DMU_PROBE_LDS_FRAG_T = 13,
    DMU_PROBE_LANE_SWAP = 14,
    DMU_PROBE_LDS_READ_TR8 = 15,
    DMU_PROBE_CVT_BF16 = 30,
    DMU_PROBE_CVT_F16 = 31
};

int dmu_probe(int variant, const void *in0, const void *in1, void *out, void *stream);

/*
 * Matrix-core ceiling (diagnostics): the rate this chip sustains for the GEMM
 * kernels' 16 x 16 matrix instructions when nothing else runs, the practical
 * counterpart of the dense peak that "Tensor Cores, CUTLASS and CuTe" derives
 * in its opening section (units x instructions per clock x clock), measured
 * rather than multiplied out.  Launches `workgroups` workgroups of 8
 * wavefronts (two per SIMD, as the tiled kernels run); every wavefront issues
 * rounds x 32 independent instructions of `in_type` (DMU_BF16, DMU_F16:
 * 16x16x32; DMU_I8: 16x16x64) on register operands of fixed pseudo-random
 * finite values, with no memory traffic.  With 256 workgroups and 128 rounds
 * the launch does the 2 x 4096^3 FLOP of the 4096^3 product.  `stamps` (device,
 * caller-owned, 8-byte aligned, or NULL) receives 4 uint64_t per workgroup:
 * the 100 MHz constant clock and the shader clock counter at start, then both
 * at end, from thread 0.  The caller times the launch (HIP events on
 * `stream`).  DMU_ERR_INVALID_ARG for rounds or workgroups < 1 or a misaligned
 * `stamps`; DMU_ERR_UNSUPPORTED for another type; DMU_ERR_HIP if the launch
 * fails.
 */
int dmu_mfma_ceiling(int in_type, int rounds, int workgroups, void *stamps, void *stream);

/* Shape of a probe variant: instruction m, n, k, input dmu_dtype and the
 * number of 32-bit output registers per lane.  Host-only. */
int dmu_probe_info(int variant, int *m, int *n, int *k, int *in_type, int *regs_per_lane);

#ifdef __cplusplus
}
#endif

#endif /* DMU_H */
