/*
 * na2d.h -- C ABI of libna2d: forward pass of 2D (dilated) Neighborhood
 * Attention on AMD Instinct MI355X (gfx950).
 *
 * The operator (NAT model doc, Overview; NAT repository README,
 * introduction; DiNAT walk-through blog, section "What is DiNAT"):
 * every query pixel attends to a k x k window of key pixels taken every d
 * pixels (dilation d).  The window is placed inside the query's residue class
 * (the pixels with the same row mod d and column mod d), centred on the query
 * and shifted inward at the borders, so every query keeps exactly k*k
 * neighbours.  Scores are q.k / sqrt(D) plus a per-head relative-position
 * bias looked up by the key-minus-query offset counted in steps of d; a
 * softmax over the k*k neighbours follows, then the probability-weighted sum
 * of the value rows.  The blog's module code shows the decomposition this
 * header mirrors: natten2dqkrpb -> softmax(dim=-1) -> natten2dav.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates no memory and keeps no mutable global state (the one
 *    exception: na2d_backward_noalloc's fixed device array and the
 *    once-per-device record of its address, described there).
 *  - q, k, v and out are dense [B, heads, H, W, D] (D fastest) in `dtype`.
 *  - rpb is dense [heads, 2k-1, 2k-1] in `dtype`; entry [h][dy+k-1][dx+k-1]
 *    is the bias of a key dy window-steps below and dx steps right of the
 *    query.  rpb == NULL means a zero bias.
 *  - attn (the unfused path's score / probability tensor) is always fp32,
 *    dense [B, heads, H, W, k*k]; neighbour slot n = a*k + c is window row a,
 *    window column c.
 *  - Work is enqueued on `stream` (NULL = the null stream) and the call
 *    returns without waiting.  A fault inside a kernel is reported by the
 *    caller's next synchronisation, not by the return value.
 *  - Outputs must not overlap inputs (except na2d_softmax, which may run in
 *    place with attn_in == attn_out).
 *  - Every argument check runs before any HIP call.  Calls are thread-safe.
 *
 * Status codes
 * ------------
 *  NA2D_ERROR_INVALID_VALUE: a size < 1; kernel_size even or < 1;
 *    dilation < 1; H or W smaller than kernel_size * dilation (the caller must
 *    pad such maps, as the DiNAT module's maybe_pad does); a required pointer
 *    NULL or not 16-byte aligned; dtype or algorithm not in its enum;
 *    overlapping output and input; B*heads*H*W*max(D, k*k) beyond 2^60.
 *  NA2D_ERROR_NOT_SUPPORTED: a valid problem this build does not implement:
 *    D != 32, kernel_size > 13, more than 2^31-1 workgroups, or (na2d_qkrpb,
 *    na2d_av) a (batch, head) plane of 2^31 pixels or more.
 *  NA2D_ERROR_LAUNCH_FAILURE: the HIP runtime refused a launch.
 */
#ifndef NA2D_H
#define NA2D_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NA2D_DTYPE_F32 = 0,
    NA2D_DTYPE_BF16 = 1,
    NA2D_DTYPE_F16 = 2
} na2d_dtype_t;

typedef enum {
    NA2D_SUCCESS = 0,
    NA2D_ERROR_INVALID_VALUE = 1,
    NA2D_ERROR_NOT_SUPPORTED = 2,
    NA2D_ERROR_LAUNCH_FAILURE = 3,
    NA2D_ERROR_WORKSPACE_LIMIT = 4  /* na2d_backward_noalloc: problem needs more
                                       workspace than its fixed array holds */
} na2d_status_t;

/* Kernel family used by na2d_forward_algo. */
typedef enum {
    NA2D_ALGO_AUTO = 0, /* MFMA for bf16/fp16, FMA for fp32 */
    NA2D_ALGO_FMA = 1,  /* one lane per query, scalar fp32 FMA, any dtype */
    NA2D_ALGO_MFMA = 2, /* matrix-core kernels (the library's choice), bf16/fp16 only */
    NA2D_ALGO_MFMA_TILED = 3 /* the block-tiled matrix-core kernel only (never the
                                row-streaming one): for comparisons and tests */
} na2d_algo_t;

/*
 * Fused forward pass: out = softmax(q.k/sqrt(D) + rpb) . v over each query's
 * dilated k x k window, in one kernel; the attention weights never reach
 * memory.  Accumulation is fp32; out is rounded once to `dtype` (RNE).
 */
na2d_status_t na2d_forward(const void *q, const void *k, const void *v, const void *rpb,
                           void *out, int B, int heads, int H, int W, int D,
                           int kernel_size, int dilation, na2d_dtype_t dtype,
                           hipStream_t stream);

/* na2d_forward with an explicit kernel family.  NA2D_ALGO_MFMA returns
 * NA2D_ERROR_NOT_SUPPORTED for fp32 data and for (batch, head) planes that
 * span more than 2^31 bytes (H*W > 2^25 pixels at 16 bits); NA2D_ALGO_AUTO
 * sends such planes to the FMA kernel. */
na2d_status_t na2d_forward_algo(const void *q, const void *k, const void *v, const void *rpb,
                                void *out, int B, int heads, int H, int W, int D,
                                int kernel_size, int dilation, na2d_dtype_t dtype,
                                na2d_algo_t algo, hipStream_t stream);

/*
 * na2d_forward that also writes each query's log-sum-exp: the natural log of
 * the softmax's denominator over its k*k window,
 *   lse[b,h,i,j] = ln sum_n exp(q[b,h,i,j].k[neighbour n] / sqrt(D) + rpb[h][offset of n]),
 * the score row of the blog's natten2dqkrpb step (DiNAT walk-through blog,
 * "What is DiNAT") reduced the way its softmax(dim=-1) normalises it.  With
 * it the softmax weights exp(score - lse) are recoverable from q, k and rpb
 * alone, which is what a gradient pass needs.
 *
 *   lse  written, fp32, dense [B, heads, H, W]; device memory, 16-byte
 *        aligned; must not overlap out or any input
 *
 * lse is computed in fp32 from the same scores as out (the matrix-core
 * kernels take the weights' fp32 sum before they are rounded for the value
 * product).  out is bit-identical to na2d_forward's.  Other arguments, rules
 * and status codes as na2d_forward (kernel family NA2D_ALGO_AUTO).
 */
na2d_status_t na2d_forward_lse(const void *q, const void *k, const void *v, const void *rpb,
                               void *out, float *lse, int B, int heads, int H, int W, int D,
                               int kernel_size, int dilation, na2d_dtype_t dtype,
                               hipStream_t stream);

/*
 * na2d_forward on strided views: the same operator, with q, k, v and out
 * addressed as [B, heads, H, W, D] views whose element (b, h, i, j, e) sits
 * at  b*s[0] + h*s[1] + i*s[2] + j*s[3] + e  (D channels contiguous).  This
 * reads channels-last hidden states as the NAT/DiNAT encoders keep them
 * ([B, H, W, heads*D]: s = {H*W*heads*D, D, W*heads*D, heads*D}; DiNAT
 * walk-through blog, encoder section, and the blog's attention module, which
 * splits the channels into heads) and writes out in that layout, with no
 * permute around the call; a fused QKV buffer [B, H, W, 3*heads*D] passes
 * q, k, v as three base pointers with shared strides.
 *
 *   in_strides   4 element strides (batch, head, row, column) shared by q,
 *                k and v; host memory, read during the call only
 *   out_strides  4 element strides of out; host memory
 *
 * Strides must be >= 0 with every stride times the element size a multiple
 * of 16 bytes; out's strides must not map two elements to one address; out's
 * footprint (first to last element it touches) must not overlap q's, k's,
 * v's or rpb's.  Violations return NA2D_ERROR_INVALID_VALUE before any HIP
 * call.  Kernel family as NA2D_ALGO_AUTO; dense strides take exactly the
 * na2d_forward path.  Other conventions as na2d_forward.
 */
na2d_status_t na2d_forward_strided(const void *q, const void *k, const void *v,
                                   const void *rpb, void *out, int B, int heads, int H, int W,
                                   int D, int kernel_size, int dilation,
                                   const int64_t *in_strides, const int64_t *out_strides,
                                   na2d_dtype_t dtype, hipStream_t stream);

/*
 * Forward pass on a map that may be smaller than the dilated window, as the
 * DiNAT layer runs it (maybe_pad: a feature map smaller than
 * kernel_size * dilation is padded, attended and cropped back; DiNAT
 * walk-through blog, layer organisation).  The operator runs on an
 * Hp x Wp map, Hp = max(H, k*d) and Wp = max(W, k*d), padded below and to
 * the right: a padded pixel has key pad_k[h] and value pad_v[h], the
 * projection of a zero feature (the key/value projection biases; NULL =
 * zeros, i.e. no bias).  Windows are clamped inside the padded map.
 *
 *   q, k, v, out  dense [B, heads, H, W, D] at the real size; out receives
 *                 the H x W queries (the crop)
 *   pad_k, pad_v  [heads, D] in dtype, 16-byte aligned, or NULL
 *
 * H, W >= 1 (no k*d minimum); maps that need no padding run exactly
 * na2d_forward (the pad vectors are unused).  Other rules as na2d_forward;
 * out must not overlap q, k, v, rpb or the pad vectors.
 */
na2d_status_t na2d_forward_padded(const void *q, const void *k, const void *v, const void *rpb,
                                  const void *pad_k, const void *pad_v, void *out, int B,
                                  int heads, int H, int W, int D, int kernel_size,
                                  int dilation, na2d_dtype_t dtype, hipStream_t stream);

/*
 * Linear projection of channels-last features: y[m, n] = sum_k x[m, k] *
 * w[n, k] + b[n] (w in the [out, in] layout of a Linear layer), the
 * projections the attention module wraps around the operator (DiNAT
 * walk-through blog, "What is DiNAT": query/key/value projections with bias,
 * the configuration's qkv_bias).  fp32 accumulation, y rounded once.
 *
 *   x [M, K], w [N, K], b [N] (NULL = no bias), y [M, N]: dense, 16-byte
 *   aligned, y overlapping none of the others.
 * N % 16 == 0 and K % 32 == 0 (else NA2D_ERROR_NOT_SUPPORTED).
 */
na2d_status_t na2d_linear(const void *x, const void *w, const void *b, void *y, int64_t M,
                          int N, int K, na2d_dtype_t dtype, hipStream_t stream);

/* Bytes of scratch na2d_block_forward needs: B*H*W*4*C elements (the
 * q|k|v projection and the attention output); 0 for invalid sizes. */
size_t na2d_block_workspace_size(int B, int H, int W, int C, int heads, na2d_dtype_t dtype);

/*
 * The attention block around the operator, on channels-last features:
 *   qkv = x w_qkv^T + b_qkv;  ctx = NA(q, k, v) per head;  y = ctx w_out^T + b_out
 * (the NAT/DiNAT attention module: q/k/v projections with bias, then
 * natten2dqkrpb, softmax and natten2dav -- DiNAT walk-through blog, "What is
 * DiNAT" -- closed by the output projection).  Maps smaller than
 * kernel_size * dilation are padded as the layer does (maybe_pad): the
 * padded features project to the key/value biases.
 *
 *   x, y        [B, H, W, C] channels-last, C = heads * 32
 *   w_qkv       [3C, C] (rows: query, key, value projections); b_qkv [3C] or NULL
 *   w_out       [C, C]; b_out [C] or NULL
 *   rpb         [heads, 2k-1, 2k-1] or NULL
 *   workspace   >= na2d_block_workspace_size(...) bytes of device scratch;
 *               its content on return is unspecified
 * On `stream`: one fused kernel where it applies (see na2d_block_path_t),
 * else three launches (the q|k|v projection written as three dense
 * [B, heads, H, W, D] tensors, the attention, the output projection).  y and
 * workspace must overlap none of the inputs nor each other.  D = C / heads != 32 returns
 * NA2D_ERROR_NOT_SUPPORTED; other rules as na2d_forward_padded.
 */
na2d_status_t na2d_block_forward(const void *x, const void *w_qkv, const void *b_qkv,
                                 const void *rpb, const void *w_out, const void *b_out,
                                 void *y, void *workspace, size_t workspace_bytes, int B, int H,
                                 int W, int C, int heads, int kernel_size, int dilation,
                                 na2d_dtype_t dtype, hipStream_t stream);

/* Kernel plan of the attention block. */
typedef enum {
    NA2D_BLOCK_AUTO = 0,     /* the fused kernel where it applies, else three launches */
    NA2D_BLOCK_UNFUSED = 1,  /* projection, attention, projection: three launches */
    NA2D_BLOCK_FUSED = 2     /* one kernel: bf16/fp16, C = 64 in 2 heads, k in {3, 5, 7},
                                dilation 1, H, W >= k (no padding), H*W <= 2^24;
                                elsewhere NA2D_ERROR_NOT_SUPPORTED */
} na2d_block_path_t;

/*
 * na2d_block_forward with an explicit kernel plan.  The fused kernel keeps
 * q, k, v and the attention output on chip (each rounded to `dtype` as the
 * three-launch path stores them) and reads no workspace: with
 * NA2D_BLOCK_FUSED, workspace may be NULL and workspace_bytes 0.  AUTO and
 * UNFUSED validate the workspace as na2d_block_forward does, whichever path
 * then runs.  Invalid `path` returns NA2D_ERROR_INVALID_VALUE.
 */
na2d_status_t na2d_block_forward_path(const void *x, const void *w_qkv, const void *b_qkv,
                                      const void *rpb, const void *w_out, const void *b_out,
                                      void *y, void *workspace, size_t workspace_bytes, int B,
                                      int H, int W, int C, int heads, int kernel_size,
                                      int dilation, na2d_dtype_t dtype, na2d_block_path_t path,
                                      hipStream_t stream);

/*
 * Unfused step 1 (the blog's natten2dqkrpb): attn[b,h,i,j,n] =
 * q[b,h,i,j].k[neighbour n] / sqrt(D) + rpb[h][offset of n], in fp32.
 */
na2d_status_t na2d_qkrpb(const void *q, const void *k, const void *rpb, float *attn,
                         int B, int heads, int H, int W, int D, int kernel_size,
                         int dilation, na2d_dtype_t dtype, hipStream_t stream);

/*
 * Unfused step 2 (softmax over the last axis): each row of k*k fp32 scores is
 * replaced by exp(s - max) / sum.  attn_in == attn_out runs in place.
 */
na2d_status_t na2d_softmax(const float *attn_in, float *attn_out, int B, int heads, int H,
                           int W, int kernel_size, hipStream_t stream);

/*
 * Unfused step 3 (the blog's natten2dav): out[b,h,i,j,:] =
 * sum_n attn[b,h,i,j,n] * v[neighbour n, :], accumulated in fp32 and rounded
 * once to `dtype`.
 */
na2d_status_t na2d_av(const float *attn, const void *v, void *out, int B, int heads, int H,
                      int W, int D, int kernel_size, int dilation, na2d_dtype_t dtype,
                      hipStream_t stream);

/*
 * Backward pass: gradients of sum(out * dout) with respect to q, k, v and the
 * bias table, for the operator na2d_forward computes (the chain rule through
 * the DiNAT module's natten2dqkrpb -> softmax -> natten2dav; DiNAT
 * walk-through blog, "What is DiNAT").
 *
 *   q, k, v, rpb  the forward inputs (rpb may be NULL: zero bias); the
 *                 probabilities are recomputed from them
 *   dout          gradient of the loss with respect to the forward output
 *   dq, dk, dv    written, [B, heads, H, W, D] in `dtype`, rounded once (RNE)
 *   drpb          written when not NULL: fp32 [heads, 2k-1, 2k-1], the bias
 *                 table's gradient summed over batch and pixels; NULL skips it
 *   workspace     caller-owned device memory of at least
 *                 na2d_backward_workspace_size(...) bytes, 16-byte aligned;
 *                 its contents are scratch (nothing needs to be zeroed)
 *
 * All accumulation is fp32 and every sum runs in a fixed order: repeated
 * calls give identical results.  Layouts, dtypes and status codes are those
 * of na2d_forward; outputs must not overlap each other, the inputs or the
 * workspace.  Work is enqueued on `stream`.
 */
na2d_status_t na2d_backward(const void *q, const void *k, const void *v, const void *rpb,
                            const void *dout, void *dq, void *dk, void *dv, float *drpb,
                            void *workspace, size_t workspace_bytes, int B, int heads, int H,
                            int W, int D, int kernel_size, int dilation, na2d_dtype_t dtype,
                            hipStream_t stream);

/* Workspace bytes na2d_backward needs (with_bias_grad: drpb != NULL); 0 for
 * an invalid or unsupported problem. */
size_t na2d_backward_workspace_size(int B, int heads, int H, int W, int D, int kernel_size,
                                    int dilation, int with_bias_grad);

/*
 * na2d_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, results and status codes are
 * na2d_backward's; the gradients are bit-identical to its.
 *
 * The workspace is a fixed device array of na2d_backward_noalloc_limit()
 * bytes (64 MiB) inside the library, one copy per GPU, present from the
 * library's first use on that GPU until the process ends.  Its device address
 * is looked up on the first call on each device (the device of `stream`, or
 * the current one for the null stream) and kept for later calls.  The call
 * allocates nothing and calls no allocating routine.
 *
 *  - A problem whose workspace (na2d_backward_workspace_size) exceeds the
 *    limit returns NA2D_ERROR_WORKSPACE_LIMIT before any HIP call; every
 *    configuration of the NAT/DiNAT layers up to 200x336 maps at k = 13 fits.
 *  - Every call on one GPU uses the same array.  Calls whose work overlaps in
 *    time on one GPU (different streams, or several host threads without
 *    ordering) race on it and give undefined results; calls ordered on one
 *    stream are safe.  The kernels write every workspace entry they read
 *    first, so nothing needs clearing between calls.
 */
na2d_status_t na2d_backward_noalloc(const void *q, const void *k, const void *v,
                                    const void *rpb, const void *dout, void *dq, void *dk,
                                    void *dv, float *drpb, int B, int heads, int H, int W, int D,
                                    int kernel_size, int dilation, na2d_dtype_t dtype,
                                    hipStream_t stream);

/* Bytes of na2d_backward_noalloc's device array. */
size_t na2d_backward_noalloc_limit(void);

/* Static, NUL-terminated description of a status code. */
const char *na2d_status_string(na2d_status_t status);

/* Library version as major*10000 + minor*100 + patch. */
int na2d_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NA2D_H */
