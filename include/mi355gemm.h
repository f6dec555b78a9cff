/*
 * mi355gemm -- tiled dense GEMM for one AMD Instinct MI355X (gfx950).
 *
 * C ABI of libmi355gemm.so.  Every entry point takes plain device pointers,
 * sizes in elements and a HIP stream; it validates its arguments on the host
 * (before any HIP call), enqueues its kernels on `stream` and returns without
 * synchronising.  The library allocates no memory and keeps no state besides
 * a read-only configuration table and the process-wide override set by
 * mg_set_config().
 *
 * Common rules
 *  - Element types: fp16 or bf16 in, the same type out.  Products are exact
 *    and are accumulated in fp32 ("Triton study notes", section 2.1: always
 *    accumulate in fp32); the fp32 result is rounded once, to nearest even,
 *    to the output type.  mg_gemm, mg_gemm_bias_relu and mg_conv2d also
 *    take fp32 (MG_F32 in and out, see mg_gemm).
 *  - Layout: matrices with one unit stride.  Leading strides are in
 *    elements, must be >= the row length and span 16 bytes a whole number
 *    of times (a multiple of 8 for 16-bit types, of 4 for fp32), so every
 *    row starts on a 16-byte boundary; base pointers must be 16-byte
 *    aligned.  Where a transposed operand is accepted, the entry point says.
 *  - Ownership: the caller owns every buffer.  Outputs must not overlap
 *    inputs.  Buffers must stay valid until the enqueued work has finished.
 *  - Errors: a non-MG_OK status means nothing was enqueued, except
 *    MG_ERR_HIP, which reports a failed launch (hipGetLastError).
 *  - Sizes: M == 0 or N == 0 is a no-op returning MG_OK; K == 0 yields the
 *    empty sum (zeros, or ReLU(bias) for the fused epilogue).
 *  - Concurrency: calls are independent and may be issued from several host
 *    threads; mg_set_config() is process-wide and meant for benchmarking.
 */
#ifndef MI355GEMM_H
#define MI355GEMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MG_OK = 0,
    MG_ERR_INVALID_ARG = 1,        /* null pointer with a nonzero extent, negative size, bad count */
    MG_ERR_UNSUPPORTED_DTYPE = 2,  /* dtype not fp16/bf16, or input and output types differ        */
    MG_ERR_UNSUPPORTED_LAYOUT = 3, /* no unit stride, leading stride shorter than a row, or a
                                      transposed operand on a shape the direct kernels cannot take  */
    MG_ERR_MISALIGNED = 4,         /* base pointer not 16-byte aligned or leading stride % 8 != 0   */
    MG_ERR_HIP = 5,                /* the HIP runtime reported an error when launching               */
    MG_ERR_BAD_CONFIG = 6          /* unknown configuration id, or a BK the configuration cannot use */
} mg_status;

typedef enum { MG_F16 = 0, MG_BF16 = 1, MG_F32 = 2 } mg_dtype;

/* Human-readable name of a status code (static storage). */
const char* mg_status_string(mg_status status);

/*
 * C[M,N] = A[M,K] * B[K,N].
 *
 * The tiled product of the pages' minimal kernel ("Using Triton to optimise
 * GEMM across chips", section 2.1; Gluon matmul example): the output is cut
 * into BM x BN tiles, each tile accumulates BK-wide slices of A and B.
 * A: M x K, element (m, k) at A + m*stride_am + k*stride_ak: either
 *    stride_ak == 1 (row-major) or stride_am == 1 (A given transposed,
 *    stored K x M with row stride stride_ak).
 * B: K x N, element (k, n) at B + k*stride_bk + n*stride_bn: either
 *    stride_bn == 1 (row-major) or stride_bk == 1 (B given transposed,
 *    stored N x K with row stride stride_bn).
 * C: M x N, row stride stride_cm, inner stride stride_cn (must be 1).
 * Strides are in elements; a transposed view is a swap of the two strides
 * (the strided 2-D view of "Triton study notes", section 1.2).  The stored
 * row stride of each operand must be a multiple of 8 and at least its row
 * length; any other stride pattern is MG_ERR_UNSUPPORTED_LAYOUT.  Any M, N
 * and K are accepted in either layout (the direct-to-LDS kernels zero-fill
 * a K tail and mask the N tail).  A transposed operand is refused
 * (MG_ERR_UNSUPPORTED_LAYOUT) in two cases.  The first is a configuration,
 * forced with mg_set_config(), that has no direct-to-LDS kernel.  The
 * second is a row stride so large (about 2^24 elements or more) that a
 * 64-row span of the operand passes the direct-to-LDS kernel's 31-bit
 * load offsets.  Row-major operands with such strides run on the general
 * kernel.  The output tiles of one call (BM x BN each, counted over every
 * batch entry or split where the entry point has them) must number below
 * 2^31, else MG_ERR_INVALID_ARG.
 *
 * fp32 (in_dtype == out_dtype == MG_F32; the 4096^3 fp32 row of the FlagOS
 * cross-chip page's benchmark table, section 3.4): fp32 inputs on the fp32
 * matrix cores, fp32 accumulation and output.  Row-major A and B only,
 * K % 16 == 0 and N % 4 == 0, else MG_ERR_UNSUPPORTED_LAYOUT; leading
 * strides multiples of 4.  Not available in the batched, split-K, grouped
 * or prepacked entry points (MG_ERR_UNSUPPORTED_DTYPE there).
 */
mg_status mg_gemm(const void* A, const void* B, void* C,
                  int64_t M, int64_t N, int64_t K,
                  int64_t stride_am, int64_t stride_ak,
                  int64_t stride_bk, int64_t stride_bn,
                  int64_t stride_cm, int64_t stride_cn,
                  mg_dtype in_dtype, mg_dtype out_dtype, hipStream_t stream);

/*
 * C[M,N] = ReLU(A[M,K] * B[K,N] + bias[N]) in one kernel.
 *
 * The fused epilogue of "Using Triton to optimise GEMM across chips",
 * section 3.4: bias and activation are applied to the fp32 accumulator in
 * registers before the single rounding, so the product never makes an extra
 * trip through memory.  bias: N contiguous elements of out_dtype.  ReLU of a
 * non-positive value is +0.0.  Other arguments as mg_gemm.
 */
mg_status mg_gemm_bias_relu(const void* A, const void* B, const void* bias, void* C,
                            int64_t M, int64_t N, int64_t K,
                            int64_t stride_am, int64_t stride_ak,
                            int64_t stride_bk, int64_t stride_bn,
                            int64_t stride_cm, int64_t stride_cn,
                            mg_dtype in_dtype, mg_dtype out_dtype, hipStream_t stream);

/*
 * Batched GEMM in one launch: C_b = A_b * B_b for b = 0 .. batch-1, where
 * entry b of each operand starts batch_stride_{a,b,c} elements after entry
 * b-1 (the batched shapes of "Using Triton to optimise GEMM across chips",
 * section 4.3).  Every entry has the layout mg_gemm() accepts, transposed
 * operands included.  A stride of 0 repeats one A or B for every entry; C
 * entries must not overlap (batch_stride_c >= M * stride_cm), otherwise
 * MG_ERR_UNSUPPORTED_LAYOUT.  Batch strides are multiples of 8 (16-byte
 * aligned entries), else MG_ERR_MISALIGNED; batch < 0 is MG_ERR_INVALID_ARG,
 * batch == 0 does nothing.  Workgroups take the tiles of one entry after
 * another, so one launch fills the GPU with many small products.
 */
mg_status mg_gemm_batched(const void* A, const void* B, void* C, int64_t batch,
                          int64_t M, int64_t N, int64_t K,
                          int64_t stride_am, int64_t stride_ak,
                          int64_t stride_bk, int64_t stride_bn,
                          int64_t stride_cm, int64_t stride_cn,
                          int64_t batch_stride_a, int64_t batch_stride_b, int64_t batch_stride_c,
                          mg_dtype in_dtype, mg_dtype out_dtype, hipStream_t stream);

/*
 * Split-K GEMM for outputs too small to fill the GPU (tall-skinny or large-K
 * shapes, "Using Triton to optimise GEMM across chips", section 4.3): the K
 * slices are cut into `splits` contiguous runs, one set of output tiles per
 * run writes fp32 partial products to the caller's workspace
 * ([splits][M][N] fp32, mg_splitk_workspace_bytes() bytes, 16-byte aligned,
 * device memory the call only writes and reads), and a second kernel adds
 * the partials in split order (deterministic) and rounds once into C.  Both
 * kernels run on `stream`; the workspace must not be used by another call
 * until they have finished.  Operands as for mg_gemm(), transposed ones
 * included, any K; N must be a multiple of 8 (the partials are summed 8
 * columns at a time), else MG_ERR_UNSUPPORTED_LAYOUT.  splits in [1, 4096];
 * a workspace that is null or too small is MG_ERR_INVALID_ARG.
 */
size_t mg_splitk_workspace_bytes(int64_t M, int64_t N, int64_t splits);
/* A split count for mg_gemm_splitk() (1 means: use mg_gemm()): for a shape
 * the offline sweep timed, the count that measured fastest on MI355X;
 * otherwise the count of least time in the library's time model.  Host
 * only; no HIP call. */
int64_t mg_splitk_choose(int64_t M, int64_t N, int64_t K);
mg_status mg_gemm_splitk(const void* A, const void* B, void* C, void* workspace, size_t workspace_bytes,
                         int64_t splits, int64_t M, int64_t N, int64_t K,
                         int64_t stride_am, int64_t stride_ak,
                         int64_t stride_bk, int64_t stride_bn,
                         int64_t stride_cm, int64_t stride_cn,
                         mg_dtype in_dtype, mg_dtype out_dtype, hipStream_t stream);

/*
 * mg_gemm_splitk without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The fp32
 * partials go to a fixed scratch array inside the library: one per GPU, of
 * mg_splitk_noalloc_max_bytes() bytes (32 MiB), created when the library is
 * first used on that GPU and held until the process ends.  A problem whose
 * partials (splits * M * N * 4 bytes) exceed it is MG_ERR_INVALID_ARG;
 * everything else as mg_gemm_splitk().  The call makes no hipMalloc, hipFree
 * or other allocating call; its only HIP calls besides the launches are
 * hipGetDevice and, on the first call on a device, hipGetSymbolAddress.
 * Every call on one GPU shares that GPU's array and overwrites the part it
 * uses before reading it: calls on one GPU must not overlap in time (calls
 * on one stream never do; calls on different streams race).
 */
size_t mg_splitk_noalloc_max_bytes(void);
mg_status mg_gemm_splitk_noalloc(const void* A, const void* B, void* C, int64_t splits,
                                 int64_t M, int64_t N, int64_t K,
                                 int64_t stride_am, int64_t stride_ak,
                                 int64_t stride_bk, int64_t stride_bn,
                                 int64_t stride_cm, int64_t stride_cn,
                                 mg_dtype in_dtype, mg_dtype out_dtype, hipStream_t stream);

/*
 * Grouped GEMM for the expert layer of a mixture-of-experts model, in one
 * launch: for every expert e,
 *     Y[o_e : o_{e+1}, :] = X[o_e : o_{e+1}, :] * W[e]
 * with o = expert_offsets (the yfxerp page, section 2.3, on the dozens of
 * GEMMs one MoE layer chains).
 * X: T x K token rows sorted by expert, row stride stride_xm.
 * W: E matrices K x N; W[e] starts stride_we elements after W[e-1]; row
 *    stride stride_wk.  stride_we must be a multiple of 8.
 * Y: T x N, row stride stride_ym.
 * expert_offsets: DEVICE array of E+1 int32 with o_0 = 0, o_E = T and
 *    o_e <= o_{e+1}.  It is read by the kernel and is not validated.  As
 *    the kernel reads the offsets, it clamps each into [0, T] and raises
 *    it to at least the previous one.  Offsets that break the rules
 *    therefore leave some rows of Y unspecified, but never cause an access
 *    outside X, W and Y.  Experts with no rows write nothing.
 * dtype is both the input and the output type.  T and E must be below 2^31,
 * and so must the tiles the launch is sized for, (ceil(T / BM) + E) times
 * the column tiles (else MG_ERR_INVALID_ARG).
 */
mg_status mg_grouped_gemm(const void* X, const void* W, void* Y, const int32_t* expert_offsets,
                          int64_t E, int64_t T, int64_t N, int64_t K,
                          int64_t stride_xm, int64_t stride_we, int64_t stride_wk, int64_t stride_ym,
                          mg_dtype dtype, hipStream_t stream);

/*
 * Blocked re-layout of A ("layout planner", "Using Triton to optimise GEMM
 * across chips", section 3.2): A[M,K] -> Ap[ceil(K/BK), M, BK], i.e. element
 * (m, k) moves to ((k / BK) * M + m) * BK + k % BK, and the last K block is
 * zero-padded.  Each BM x BK tile of A then is one contiguous run.
 * Ap must hold mg_prepacked_bytes(M, K, BK, dtype) bytes, 16-byte aligned.
 * BK must be a BK of some configuration (see mg_config_bk).
 */
size_t mg_prepacked_bytes(int64_t M, int64_t K, int64_t BK, mg_dtype dtype);
mg_status mg_prepack_a(const void* A, void* Ap, int64_t M, int64_t K, int64_t stride_am, int64_t BK,
                       mg_dtype dtype, hipStream_t stream);

/* The BK that mg_gemm_prepacked will use for this problem (the selected
 * configuration's K step); pack A with exactly this BK. */
int64_t mg_config_bk(int64_t M, int64_t N, int64_t K, mg_dtype dtype);

/* C = A * B with A given in the blocked layout produced by mg_prepack_a with
 * the same BK.  Returns MG_ERR_BAD_CONFIG if BK differs from the selected
 * configuration's.  B and C as in mg_gemm. */
mg_status mg_gemm_prepacked(const void* Ap, int64_t BK, const void* B, void* C,
                            int64_t M, int64_t N, int64_t K,
                            int64_t stride_bk, int64_t stride_bn,
                            int64_t stride_cm, int64_t stride_cn,
                            mg_dtype dtype, hipStream_t stream);

/*
 * The layout planner's cost/benefit test ("Using Triton to optimise GEMM
 * across chips", section 3.2: re-lay A out only when the gain exceeds the cost
 * of the copy).  For an M x N x K GEMM on the row the table selects: the
 * number of GEMMs that must share one blocked A (mg_prepack_a) before the
 * blocking copy has paid for itself, from the packed/plain time ratio and
 * the copy rate that the offline sweep measured; -1 when the blocked layout
 * is not faster on that row (then prepacking never pays).  Host only.
 */
int64_t mg_prepack_uses_to_pay(int64_t M, int64_t N, int64_t K, mg_dtype dtype);

/* ---- GEMM consumers ------------------------------------------------------- */

/*
 * Shape of a 2-D convolution (cross-correlation with zero padding, as deep-
 * learning frameworks define it).  Input NHWC [batch, height, width,
 * in_channels]; output NHWC [batch, OH, OW, out_channels] with
 *     OH = (height + 2*pad_h - dilation_h*(kernel_h - 1) - 1) / stride_h + 1
 * (floor) and OW likewise.
 */
typedef struct {
    int64_t batch, height, width, in_channels, out_channels;
    int64_t kernel_h, kernel_w;
    int64_t stride_h, stride_w;
    int64_t pad_h, pad_w;
    int64_t dilation_h, dilation_w;
} mg_conv2d_shape;

/* Output height and width of `shape`; MG_ERR_INVALID_ARG for a negative size,
 * a stride, dilation or kernel extent below 1, or an empty output. */
mg_status mg_conv2d_output_hw(const mg_conv2d_shape* shape, int64_t* out_h, int64_t* out_w);

/*
 * im2col (FlagOS cross-chip page, section 5.3: a convolution becomes a GEMM
 * through im2col): cols is [M = batch*OH*OW, ld_cols] row-major; row
 * m = (n*OH + oh)*OW + ow holds at column k = (kh*kernel_w + kw)*in_channels
 * + c the input element x[n, oh*stride_h - pad_h + kh*dilation_h,
 * ow*stride_w - pad_w + kw*dilation_w, c], or zero where that position is
 * outside the image.  Columns K = kernel_h*kernel_w*in_channels ..
 * ld_cols-1 are written as zero.  x: dense NHWC, 16-byte aligned.  ld_cols
 * >= K and a whole number of 16-byte chunks (else MG_ERR_UNSUPPORTED_LAYOUT
 * / MG_ERR_MISALIGNED).  Bit copies: any of the three dtypes.  Limits (else
 * MG_ERR_UNSUPPORTED_LAYOUT): M < 2^31, ld_cols < 2^27, kernel_h*kernel_w
 * <= 65535, height + 2*pad_h and width + 2*pad_w < 2^30.
 */
mg_status mg_im2col(const mg_conv2d_shape* shape, const void* x, void* cols, int64_t ld_cols,
                    mg_dtype dtype, hipStream_t stream);

/*
 * Workspace that mg_conv2d needs for `shape`: the im2col matrix
 * [batch*OH*OW, ld] with ld = K rounded up to whole 16-byte chunks, or 0
 * when the convolution runs without one:
 *  - a 1x1 kernel with unit stride and no padding whose channel rows are
 *    whole 16-byte chunks (the input itself is then the GEMM's A);
 *  - implicit GEMM: fp16/bf16, an image batch below 2^31 bytes and an
 *    in_channels count that the selected configuration's K slice divides
 *    (every multiple of 64 qualifies).  The GEMM kernel then gathers each
 *    slice of its A operand straight from the image, zero-filling taps
 *    outside it, and im2col never reaches memory.
 * 0 also for an invalid shape.  The answer depends on the configuration
 * table, so an mg_set_config() override applies to it as to mg_conv2d.
 */
size_t mg_conv2d_workspace_bytes(const mg_conv2d_shape* shape, mg_dtype dtype);

/*
 * 2-D convolution as a GEMM over the im2col matrix (FlagOS cross-chip page,
 * section 5.3), gathered by the GEMM's loads (implicit GEMM) or written by
 * the im2col kernel into the workspace first (see mg_conv2d_workspace_bytes):
 *     y[n,oh,ow,o] = sum_{kh,kw,c} x[n, ih, iw, c] * w(k = (kh*kernel_w + kw)*in_channels + c, o)
 * then, when bias is not null, ReLU(y + bias[o]) (the fused epilogue of
 * mg_gemm_bias_relu).  x: dense NHWC, 16-byte aligned.  w: the K x
 * out_channels GEMM operand, element (k, o) at w + k*stride_wk +
 * o*stride_wn: HWIO weights ([kh][kw][c][o], stride_wk = out_channels,
 * stride_wn = 1) or OHWI weights ([o][kh][kw][c], stride_wk = 1, stride_wn
 * = K; the transposed-B layout of mg_gemm, 16-bit types only).  y: dense
 * NHWC; its row length out_channels must span whole 16-byte chunks.
 * workspace: at least mg_conv2d_workspace_bytes() bytes of device memory,
 * 16-byte aligned (may be null when that is 0), used by this call's kernels
 * only until they finish.  The kernels run in order on `stream`.  Errors as mg_im2col and mg_gemm; a short workspace is
 * MG_ERR_INVALID_ARG.  batch == 0 or out_channels == 0 does nothing.
 */
mg_status mg_conv2d(const mg_conv2d_shape* shape, const void* x, const void* w, int64_t stride_wk,
                     int64_t stride_wn, const void* bias, void* y, void* workspace, size_t workspace_bytes,
                     mg_dtype dtype, hipStream_t stream);

/*
 * Attention scores S_h = Q_h * K_h^T for every head h in one launch (FlagOS
 * cross-chip page, section 5.3: the QK^T of attention is a GEMM; scaling and
 * softmax are not part of it).  Q_h: Lq x d rows (row stride stride_qm,
 * head stride stride_qh), K_h: Lk x d rows (stride_kn, stride_kh), S_h: Lq x
 * Lk (stride_sm, stride_sh).  The batched GEMM with K_h as a transposed B
 * operand; fp16 or bf16; any Lq, Lk and d; strides multiples of 8.
 */
mg_status mg_attention_scores(const void* Q, const void* K, void* S, int64_t heads, int64_t Lq, int64_t Lk,
                              int64_t d, int64_t stride_qh, int64_t stride_qm, int64_t stride_kh,
                              int64_t stride_kn, int64_t stride_sh, int64_t stride_sm, mg_dtype dtype,
                              hipStream_t stream);

/* ---- configuration table (offline-tuned; read-only) ---------------------- */

typedef struct {
    int id;
    int bm, bn, bk;           /* output tile and K step                    */
    int waves_m, waves_n;     /* wavefront grid of one workgroup           */
    int stages;               /* LDS buffers in the K pipeline             */
    int mfma_m, mfma_n, mfma_k;
    int group_m;              /* tile rows visited together (L2 reuse)     */
    int xcd_remap;            /* 1: consecutive tiles stay on one XCD      */
    int lds_bytes;            /* shared memory of one workgroup            */
    int direct_lds;           /* 1: has a direct-to-LDS kernel: the
                                 pipelined kernel takes every shape, the
                                 K-split one (direct_ksplit > 1) dense
                                 row-major problems with K % direct_bk == 0
                                 and N % 8 == 0                            */
    int direct_bk;            /* K slice of the direct-to-LDS kernel       */
    int direct_stages;        /* LDS ring slots of the direct kernel       */
    int direct_lds_bytes;     /* shared memory of the direct kernel        */
    int direct_ksplit;        /* waves that split K inside the workgroup,
                                 each with its own LDS ring (1: none)      */
    const char* name;
} mg_config_desc;

int mg_num_configs(void);
mg_status mg_config_info(int id, mg_config_desc* out);
/* Force configuration `id` for every following call in this process (-1
 * restores the table's choice).  For benchmarking and tuning sweeps. */
mg_status mg_set_config(int id);
/* Override the tile raster of every following dense call in this process:
 * group_m tile rows visited together (the GROUP_M of the Gluon matmul
 * example; -1 restores the table's, 1..256 otherwise) and the XCD
 * renumbering of workgroups (1 on, 0 off, -1 the table's).  For the sweep's
 * measurements; anything else is MG_ERR_INVALID_ARG. */
mg_status mg_set_raster(int group_m, int xcd_remap);
/* Configuration id used by the most recent successful call in this process. */
int mg_last_config(void);
/* Kernel family of the most recent successful 16-bit GEMM launch in this
 * process: 0 = general register-staged kernel, 1 = direct-to-LDS pipelined
 * kernel, 2 = direct-to-LDS K-split kernel; -1 before any launch. */
int mg_last_kernel(void);
/* Configuration the table selects for a problem of this shape: dense when
 * `grouped` is 0 (a batched product of `batch` entries of M x N x K when
 * batch > 1, as mg_gemm_batched and mg_attention_scores launch it), else a
 * grouped problem of `grouped` experts over M = T rows (batch ignored).  The
 * table's model and its per-shape cache are generated by the offline sweep
 * (mg_rates.h from profiles/table_sweep.json). */
int mg_select_config(int64_t M, int64_t N, int64_t K, mg_dtype dtype, int grouped, int64_t batch);

#ifdef __cplusplus
}
#endif

#endif /* MI355GEMM_H */
