/*
 * mm.h -- C ABI of libmm.so, a bf16 matrix-multiply library for one AMD
 * MI355X (gfx950) GPU.
 *
 * The operations are the two op forms the pages centre on -- the MatmulOp
 * form out = A.B and the LinearOp form out = x.W^T + bias (issue "Automate
 * performant Hopper matmul", section "Persistent matmul"; PR "Implement
 * persistent matmul scheduling", description) -- with a fused elementwise
 * epilogue (the MLP forward epilogue fusion of that PR's description) and the
 * Llama-FFN horizontal fusion of two GEMMs that share x (PR "Translate MmaOp
 * patterns properly on Hopper", commit list: "Fix llama ffn horizontal
 * fusion", "Fixes the horizontal fusion tests").  The contraction is the
 * broadcast-multiply-sum of the _BroadcastInputs tests that PR "Implement
 * persistent matmul scheduling" describes (fusedMultiplySum): bf16 inputs,
 * fp32 accumulation, one rounding of the epilogue result to the output type.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE memory owned by the caller.  The library
 *     never allocates, frees or keeps a pointer past the return of a call.
 *   - Each successful call with M > 0 and N > 0 enqueues its work on `stream`
 *     (a hipStream_t; NULL means the default stream): one kernel, or two for a
 *     split-K call (the pieces, then their reduction), and returns without
 *     synchronizing.  Errors in execution surface on the stream.
 *   - Matrices are dense and row-major in their stored shape (the last
 *     dimension is contiguous); a transposed operand is described by the
 *     layout letters, never copied.
 *   - Argument errors are detected on the host before any HIP call, return a
 *     status and have no side effects; mm_last_error() then describes them.
 *   - M == 0 or N == 0 is a successful no-op.  K == 0 is the empty sum: every
 *     accumulator is 0, so the output is the epilogue of 0 (+ bias): bias[n],
 *     gelu(bias[n]) or 0, and 0 for the FFN forms (act(0) * 0); the operands
 *     are then never read and may be null.
 *   - Alignment: A, B (and W_gate/W_up) must be 16-byte aligned and the
 *     contiguous extent of each of them a multiple of 8 elements; bias must be
 *     2-byte aligned; out must be aligned to its element size.  Otherwise
 *     MM_ERR_MISALIGNED.  (The output may have any N, e.g. N = 3001.)
 *   - `out` must not overlap any input (MM_ERR_INVALID_VALUE).
 *   - Sizes: 0 <= M, N, K < 2^31; individual operands may hold more than 2^31
 *     elements (addresses are formed in 64 bits), each below 2^60 over all
 *     batch entries (else MM_ERR_UNSUPPORTED).
 *   - Thread safety: calls may be made from several host threads; the only
 *     process-wide state is a per-device attribute cache, the configuration
 *     override (mm_set_config), the thread-local last-error string and the
 *     static split-K scratch of mm_matmul_noalloc (see there).
 */
#ifndef MM_H_
#define MM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MM_OK = 0,
  MM_ERR_INVALID_VALUE = 1, /* null pointer, negative size, overlap, bad enum */
  MM_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement */
  MM_ERR_MISALIGNED = 3,    /* pointer or contiguous extent not aligned      */
  MM_ERR_HIP = 4            /* a HIP runtime call failed (see mm_last_error) */
} mm_status;

/* Operand layouts: the letters say whether op(A) and op(B) are the stored
 * matrix (N) or its transpose (T); op(A) is [M,K] and op(B) is [K,N].  These
 * are the axis mappings that distinguish the MatmulOp and LinearOp forms
 * (issue "Automate performant Hopper matmul", section "Persistent matmul":
 * AxisMapping).
 *   MM_NN  A stored [M][K], B stored [K][N]
 *   MM_NT  A stored [M][K], B stored [N][K]  (the LinearOp weight W [N][K])
 *   MM_TN  A stored [K][M], B stored [K][N]
 *   MM_TT  A stored [K][M], B stored [N][K]                                 */
typedef enum { MM_NN = 0, MM_NT = 1, MM_TN = 2, MM_TT = 3 } mm_layout;

/* Epilogues applied to the fp32 accumulator before the single rounding:
 *   NONE: y = acc;   BIAS: y = acc + bias[n];
 *   GELU_TANH: y = gelu(acc);   BIAS_GELU_TANH: y = gelu(acc + bias[n]),
 * with gelu(t) = 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))).  The bias
 * is one bf16 value per output column, broadcast over rows. */
typedef enum {
  MM_EPI_NONE = 0,
  MM_EPI_BIAS = 1,
  MM_EPI_GELU_TANH = 2,
  MM_EPI_BIAS_GELU_TANH = 3
} mm_epilogue;

typedef enum { MM_OUT_BF16 = 0, MM_OUT_F32 = 1 } mm_out_dtype;

/* Gate activations of the horizontally fused FFN: y = act(g) * u.
 *   SILU: act(g) = g / (1 + exp(-g))   (the Llama FFN)
 *   IDENTITY: act(g) = g               (bilinear GLU; its products of small
 *                                       integers are exact, which lets the
 *                                       gate/up index mapping be checked
 *                                       bit for bit)                       */
typedef enum { MM_GLU_SILU = 0, MM_GLU_IDENTITY = 1 } mm_glu_act;

/* MatmulOp form: out[M][N] = op(A) . op(B), written as bf16 (RNE) or fp32.
 *   A, B    bf16 operands in the storage given by `layout`
 *   out     [M][N] row-major, element type `out_dtype`
 *   stream  hipStream_t (NULL = default stream)                             */
mm_status mm_matmul(const void* A, const void* B, void* out, int64_t M, int64_t N, int64_t K,
                    mm_layout layout, mm_out_dtype out_dtype, void* stream);

/* LinearOp form: out[M][N] = epi(op(x) . op(W) + bias), bf16 output (RNE).
 *   x       activations; [M][K] for MM_NN/MM_NT, [K][M] for MM_TN/MM_TT
 *   W       weight; [N][K] for MM_NT/MM_TT (the usual linear layer), [K][N]
 *           for MM_NN/MM_TN
 *   bias    [N] bf16; required for MM_EPI_BIAS and MM_EPI_BIAS_GELU_TANH,
 *           ignored (may be NULL) otherwise                                  */
mm_status mm_linear(const void* x, const void* W, const void* bias, void* out, int64_t M,
                    int64_t N, int64_t K, mm_layout layout, mm_epilogue epi, void* stream);

/* LinearOp with two epilogue outputs (issue "Automate performant Hopper
 * matmul", section "Epilogue", TMA store: staging memory reused when a
 * fusion has several outputs; here the pre-activation beside the activation,
 * which a backward pass of GELU needs):
 *   preact[M][N] = op(x) . op(W) + bias          (the bias term for
 *                                                 MM_EPI_BIAS_GELU_TANH only)
 *   out[M][N]    = GELU_tanh(preact), computed from the fp32 value before
 *                  preact is rounded
 * both bf16 (RNE), written by the same kernel from the same accumulators.
 *   epi     MM_EPI_GELU_TANH or MM_EPI_BIAS_GELU_TANH; any other returns
 *           MM_ERR_INVALID_VALUE
 *   preact  caller-owned device memory, element aligned, not overlapping x, W,
 *           bias or out (else MM_ERR_INVALID_VALUE / MM_ERR_MISALIGNED)
 * Other arguments, alignment rules and errors as for mm_linear.              */
mm_status mm_linear_preact(const void* x, const void* W, const void* bias, void* out, void* preact,
                           int64_t M, int64_t N, int64_t K, mm_layout layout, mm_epilogue epi,
                           void* stream);

/* Batched forms (the pages' BMNK operands: PR "Implement persistent matmul
 * scheduling", description -- inputs canonicalized to batch, M, N, K
 * dimensions, broadcast inputs through fusedMultiplySum):
 *   out[b] = op(A[b]) . op(B[b])          (mm_matmul_batched)
 *   out[b] = epi(op(x[b]) . op(W[b]) + bias)   (mm_linear_batched)
 * for b < batch, in one kernel.  Entry b of an operand starts stride_*
 * elements after entry 0; a stride of 0 broadcasts that operand to every
 * entry (e.g. one weight for all batch entries).  Each entry is laid out as
 * the unbatched call's operand (`layout` as for mm_matmul / mm_linear).
 * bias [N] is shared by all entries.
 *   stride_a / stride_x, stride_b / stride_w   >= 0, multiples of 8 when
 *                              batch > 1 (entries stay 16-byte aligned)
 *   stride_out   >= M * N when batch > 1 (entries must not overlap)
 * With batch == 1 the strides are ignored and the calls equal the unbatched
 * ones.  Errors as for mm_matmul, plus MM_ERR_INVALID_VALUE for batch < 1,
 * negative strides, or output entries that would overlap.                  */
mm_status mm_matmul_batched(const void* A, const void* B, void* out, int64_t batch, int64_t M,
                            int64_t N, int64_t K, int64_t stride_a, int64_t stride_b,
                            int64_t stride_out, mm_layout layout, mm_out_dtype out_dtype,
                            void* stream);
mm_status mm_linear_batched(const void* x, const void* W, const void* bias, void* out, int64_t batch,
                            int64_t M, int64_t N, int64_t K, int64_t stride_x, int64_t stride_w,
                            int64_t stride_out, mm_layout layout, mm_epilogue epi, void* stream);

/* Split-K workspace (PR "Implement persistent matmul scheduling", review
 * notes: splitting the K loop over workgroups, split-K and stream-K, named
 * there and left out of the persistent scheduler).  When a single-weight
 * product -- mm_matmul, or mm_linear with any epilogue, any layout, K >= 128
 * -- has fewer 256 x 256 (256 x 192, 256 x 128) output tiles than the GPU
 * has resident workgroups (at most half as many) and a cost model of the
 * kernels finds a split faster than the best unsplit run (chunks of at least
 * 8 x 64 of K), the _ws entry points below cut each tile's K loop into chunks
 * and deal the chunks of all tiles to the resident workgroups (one chunk
 * each, or equal contiguous ranges: stream-K); each piece leaves its fp32
 * partial tile in this workspace (one 256 KiB slot per workgroup, two per
 * stream-K workgroup), and a second kernel on the same stream adds them in k
 * order and applies the epilogue once.  Products of at most 32 rows (the
 * skinny kernel, see mm_describe_config) use it for fp32 partial outputs of
 * S slices of K (S x M x N x 4 bytes), added in k order the same way.
 *   form    0 matmul/linear, 1 FFN (never uses a workspace)
 *   bytes   receives the size a call of this shape on the current device may
 *           use; 0 = the shape runs without one.  Queries the device (CU
 *           count, occupancy); launches nothing.
 * Workspace contract: device memory, 256-byte aligned, any contents (every
 * byte a call reads it has written first), reusable by later calls on the
 * same stream; two calls in flight at once must not share it.             */
mm_status mm_workspace_size(int form, int64_t M, int64_t N, int64_t K, mm_layout layout,
                            int64_t* bytes);

/* mm_matmul / mm_linear with a workspace (see mm_workspace_size).  With a NULL
 * workspace, or a shape that needs none, they behave exactly as mm_matmul /
 * mm_linear.  A workspace smaller than reported returns MM_ERR_INVALID_VALUE;
 * one that overlaps an operand or the output returns MM_ERR_INVALID_VALUE.
 * A split call enqueues two kernels (the pieces, then their sum); a tile's
 * partial sums are added in k order, so results are reproducible run to run
 * (they differ from the unsplit kernel's by fp32 rounding order only).  For
 * mm_linear_ws the second kernel applies the epilogue (bias, GELU) to the
 * summed value, then rounds once.                                          */
mm_status mm_matmul_ws(const void* A, const void* B, void* out, int64_t M, int64_t N, int64_t K,
                       mm_layout layout, mm_out_dtype out_dtype, void* workspace,
                       int64_t workspace_bytes, void* stream);
mm_status mm_linear_ws(const void* x, const void* W, const void* bias, void* out, int64_t M,
                       int64_t N, int64_t K, mm_layout layout, mm_epilogue epi, void* workspace,
                       int64_t workspace_bytes, void* stream);

/* mm_matmul_ws for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the split-K partial tiles go to a static device array inside the library
 * instead of a caller's workspace.  The array holds 64 MiB (one 256 x 256
 * fp32 slot per workgroup of a chunk-major split on 256 CUs; the automatic
 * split never needs more there); each GPU the library runs on holds its own
 * copy from the first call on it until the process ends.  Arguments, results
 * and errors as for mm_matmul; in addition a shape whose split needs more
 * scratch than the array holds (a forced stream-K configuration) returns
 * MM_ERR_UNSUPPORTED before any launch.  The call itself allocates nothing:
 * no hipMalloc / hipFree, no allocating library routine.
 * All calls on one GPU share its array, and a call reads only slots it has
 * written itself, so calls made one after the other (on one stream, or
 * synchronized) need no clearing between them; calls whose kernels may run
 * at the same time on one GPU (two streams, two host threads) race on the
 * array and must not be made.                                               */
mm_status mm_matmul_noalloc(const void* A, const void* B, void* out, int64_t M, int64_t N,
                            int64_t K, mm_layout layout, mm_out_dtype out_dtype, void* stream);

/* Llama-FFN horizontal fusion in one kernel:
 *   out[M][N] = SiLU(x . W_gate^T) * (x . W_up^T), bf16 output (RNE),
 * x [M][K], W_gate and W_up [N][K].  Each x tile is loaded once and feeds
 * both products; the two accumulators meet only in the epilogue. */
mm_status mm_ffn_swiglu(const void* x, const void* W_gate, const void* W_up, void* out,
                        int64_t M, int64_t N, int64_t K, void* stream);

/* As mm_ffn_swiglu with a selectable gate activation. */
mm_status mm_ffn_glu(const void* x, const void* W_gate, const void* W_up, void* out, int64_t M,
                     int64_t N, int64_t K, mm_glu_act act, void* stream);

/* Tile configuration override, parsed from a string such as
 *   "BM=256,BN=256,WM=2,WN=2,G=8,XCD=1,KALT=1,GRID=0"
 * (BM/BN: output tile; WM/WN: wave grid; G: grouped-swizzle band height in
 * tiles; XCD: XCD-aware workgroup remap on/off; KALT: alternate the K
 * direction per persistent tile (1), never (0) or automatically (2);
 * GRID: persistent grid size, 0 = one wave of resident workgroups; PIPE:
 * preferred kernel family, 5 two-group ping-pong over alternate tiles and
 * 4 wave-specialized producer/consumer (both with BM=256,BN=128,WM=2,WN=4),
 * 3 whole-line slab ring, 2 split-phase on one tile, 1 32-k pipeline,
 * 0 basic (64 x 64 tiles of K <= 256 otherwise take the kernel that holds
 * all of K in LDS); SK: stream-K chunks per tile when a workspace is given,
 * 0 automatic, 1 never, n >= 2 forced; BSTAGE=1: linear forms with a bias
 * take the slab instance that brings the bias into LDS under the K loop).  The
 * heuristic is replaced for every later call in the process, in the manner
 * of the pages' heuristic plugin (PR "Translate MmaOp patterns properly on
 * Hopper", review of MatmulSchedulerPluginTest).  NULL or "" restores the
 * heuristic.  An invalid or unsupported string returns MM_ERR_UNSUPPORTED
 * and leaves the current setting unchanged.  The environment variable
 * MM_FORCE_CONFIG, read on the first call, sets the same override.  Not
 * thread-safe with respect to concurrent GEMM calls. */
mm_status mm_set_config(const char* spec);

/* Describes the configuration the next call of this shape would use, for
 * logging and tests: writes a string like the one mm_set_config accepts;
 * for a plain product that a split-K workspace would split on the current
 * device, SPLIT=<chunks per tile>x<tile width> (that part queries the device
 * and is left out when there is none); and last KERNEL=<family>.  The tile
 * and KERNEL parts describe a call without a workspace; with SPLIT present,
 * a call given a workspace (mm_matmul_ws, mm_linear_ws, mm_matmul_noalloc)
 * runs the slab kernel on 256 x <tile width> tiles instead.  Products of at
 * most 32 rows against at least 8 MiB of weights (layout MM_NT, one weight,
 * no forced configuration, K at most 2^23) name gemm_skinny, with
 * SPLIT=<k slices>x64 (64 weight rows per workgroup) when a workspace would
 * cut K (no device query).  K = 0 names empty_k_fill.  form: 0
 * matmul/linear, 1 FFN.  Returns MM_ERR_INVALID_VALUE for bad args. */
mm_status mm_describe_config(int form, int64_t M, int64_t N, int64_t K, mm_layout layout,
                             char* buf, int64_t buflen);

/* Host-only description of the persistent tile order, for inspection and
 * tests; launches nothing and makes no HIP call.  For a grid of `grid`
 * workgroups (capped at the tile count) it lists, in each workgroup's visit
 * order, five int32 per visited tile: hardware workgroup id, its local tile
 * index, tile row, tile column, and 1 if that tile's K loop runs from the
 * last k-step down.  Writes at most `cap` entries and stores the full count
 * in *count.  form: 0 matmul/linear, 1 FFN. */
mm_status mm_debug_schedule(int form, int64_t M, int64_t N, int64_t K, mm_layout layout,
                            int64_t grid, int32_t* out, int64_t cap, int64_t* count);

/* Static description of a status code (never NULL). */
const char* mm_status_string(mm_status s);

/* Thread-local detail of the last non-OK status returned on this thread
 * ("" if none).  Valid until the next call on the same thread. */
const char* mm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MM_H_ */
