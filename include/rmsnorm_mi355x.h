/*
 * rmsnorm_mi355x.h -- C ABI of the MI355X (gfx950) RMSNorm library.
 *
 * Operations (all rows are independent; normalisation is over the last axis):
 *
 *   rmsnorm_fwd            y = x * rsqrt(mean(x^2) + eps) * (weight_bias + w)
 *       The reference expression of the MLX pull request "RMSNormVJP backward
 *       writes a full {n_rows, D} gw_temp intermediate" (section POC), with
 *       the weight_bias offset of mlxcel issue "Fused residual-add RMSNorm and
 *       fused RoPE + KV-append decode kernels" (FusedAddRMSNorm bullet):
 *       weight_bias = 1 gives Gemma's (1 + w) convention, 0 the plain one.
 *
 *   fused_add_rmsnorm_fwd  new_residual = x + residual,
 *                          normed = rmsnorm(x + residual)
 *       Same mlxcel issue, FusedAddRMSNorm bullet and the paragraph on the
 *       two-output constraint: two separate outputs (which may also be placed
 *       over the inputs, see "In place" below).  The sum is formed once in
 *       fp32 and normalised unrounded; new_residual is that sum rounded to the
 *       storage dtype.
 *
 *   rmsnorm_vjp            dx, dw for an upstream gradient dy of y
 *       MLX pull request above, sections "Proposed changes" and "POC": the
 *       backward recomputes the row statistic from x, and the weight gradient
 *       is summed across rows inside the library, never through an
 *       intermediate of the input's size.  With g = weight_bias + w,
 *       r = rsqrt(mean(x^2) + eps), S = sum_j dy_j g_j x_j:
 *           dx_j = r g_j dy_j - x_j r^3 S / D,     dw_j = sum_rows dy_j x_j r.
 *
 *   fused_add_rmsnorm_vjp  dh = VJP(h; dy) + d_new_residual, dw
 *       Training-side backward of the fused form: h = x + residual (the saved
 *       new_residual) feeds both the normalised output and the next residual
 *       stream, so the gradient reaching h -- and through the sum both x and
 *       residual -- is the VJP for dy plus the residual-stream gradient.
 *
 *   rmsnorm_fwd_vjp        y, dx and dw from one pass over x and dy
 *       The grad call the MLX pull request's POC times (section POC: a
 *       gradient evaluation is the forward recompute plus the VJP), done in
 *       one launch: x and dy are read once, y and dx written once.
 *
 *   rmsnorm_backward       the three backward forms above through one call,
 *                          with dw in fp32 or in the weight dtype
 *
 *   silu_gate              y = silu(x[:, :d]) * x[:, d:2d],  silu(a) = a / (1 + e^-a)
 *       The gated activation of the same mlxcel issue's candidate-fusion
 *       list, with 16-byte loads: x is [rows, 2d] (the two halves of each row
 *       side by side), y is [rows, d].  fp32 arithmetic, one rounding.
 *
 *   silu_gate_vjp          dx = [da | db] for an upstream gradient dy of y:
 *                          db = dy * a * s,  da = dy * b * s * (1 + a * (1 - s)),
 *                          s = sigmoid(a) (the derivative of the gate above)
 *
 * Conventions shared by every entry point:
 *   - Layout: row-major, contiguous [rows, D] tensors; w is [D].  x,
 *     residual, w, dy, y, normed, new_residual and dx all have the dtype
 *     `dt`; dw is fp32 (rmsnorm_backward can also return it in `dt`).
 *     Arithmetic is fp32 throughout, rounded once (to nearest, ties to even)
 *     on store.
 *   - Pointers: device pointers owned by the caller; the library allocates
 *     no device memory and keeps no pointer after the call returns (the one
 *     fixed array it holds is the scratch of rmsnorm_vjp_noalloc).  Each
 *     pointer must be aligned to its element size.  Row vectors are read and
 *     written at element alignment, so the load width (16 bytes where D *
 *     itemsize is a multiple of 16) does not depend on the pointers'
 *     alignment.
 *   - In place: a [rows, D] output may be the very buffer of a [rows, D]
 *     input of the same call (same address, same extent) -- y over x;
 *     normed or new_residual over x or residual; dx (dh) or y over x (h), dy
 *     or d_new_residual; silu_gate_vjp's dx over x.  Any other overlap --
 *     partial, between two outputs, with w, dw or the workspace, any overlap
 *     for silu_gate -- returns RMSN_E_OVERLAP.
 *   - Execution: asynchronous on `hip_stream` (a hipStream_t; NULL is the
 *     null stream).  No call synchronises.  The functions are thread-safe;
 *     one workspace must not serve two calls in flight at once.
 *   - Device: the calling thread's current device (hipSetDevice) must hold
 *     every pointer and `hip_stream`; the launch configuration (from its
 *     compute-unit count) and rmsnorm_vjp_noalloc's scratch are that
 *     device's.
 *   - Errors: a status is returned, nothing is thrown.  Arguments are checked
 *     before any launch; launch failures return RMSN_E_HIP.
 *   - rows == 0 is valid: nothing is written, except that the backward
 *     entry points set dw to zero (the empty sum).  Pointers other than w
 *     and dw may then be NULL.
 */
#ifndef RMSNORM_MI355X_H
#define RMSNORM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RMSN_F32 = 0,
    RMSN_F16 = 1,
    RMSN_BF16 = 2
} rmsn_dtype_t;

typedef enum {
    RMSN_OK = 0,
    RMSN_E_NULLPTR = -1,   /* a required pointer is NULL */
    RMSN_E_SHAPE = -2,     /* rows < 0, D (or d) < 1, beyond its maximum, or sizes overflow */
    RMSN_E_DTYPE = -3,     /* unknown dtype, or a dw dtype other than fp32 and dt */
    RMSN_E_WORKSPACE = -4, /* workspace NULL or smaller than required */
    RMSN_E_OVERLAP = -5,   /* an output range overlaps another argument */
    RMSN_E_HIP = -6,       /* the HIP runtime reported an error */
    RMSN_E_ALIGN = -7,     /* a pointer is not aligned to its element size */
    RMSN_E_CONFIG = -8     /* an explicit kernel configuration cannot serve the shape */
} rmsn_status_t;

/* Largest D served (elements). */
#define RMSN_MAX_D ((int64_t)1 << 24)
/* Largest half width d served by silu_gate (elements). */
#define RMSN_MAX_GATE_D ((int64_t)1 << 28)

/* Kernel configuration.  Zero in a field means "choose automatically".
 * Only the *_cfg entry points take one; the plain entry points always choose
 * automatically.  An explicit choice that cannot serve the shape returns
 * RMSN_E_CONFIG. */
typedef struct {
    int32_t lanes_per_row;  /* threads cooperating on one row: a power of two, 1..1024,
                               or 64 W with W = 3, 5, 6, 7, 9, 10, 11, 12, 13, 14 or 15
                               ("wave rows": 16-byte vectors, vecs_per_lane 1 or 2, rows
                               of exactly lanes_per_row * vecs_per_lane vectors, 1, 2 or
                               4 rows per block; for the backward forms only where the
                               instance exists: 16-bit rows of 13 to 15 waves with 2
                               vectors per lane do not); the VJP of 16-bit rows also
                               takes 384, 448 or 512 lanes with 4 vectors per lane,
                               the grad call and fused backward 448 or 512, and every backward form of fp32
                               rows 512 lanes with 4, one row per block; the backward forms
                               also take wave rows with more vector slots than the row has
                               vectors (at most twice as many; the slots past the row's end
                               redo slots inside it); on rows that are not a whole number of
                               16-byte vectors (the last one overlapped) the forward forms
                               take wave rows with vecs_per_lane 1, 2 or 0 (the fewest that
                               hold the row) and at least as many slots as vectors, the slots
                               past the row's end masked, at most 1024 vectors per row */
    int32_t vecs_per_lane;  /* vectors each thread holds per row: 1, 2, 4 or 8;
                               -1 selects the streaming (looped) kernel; -2 the
                               column-split backward forms (backward entry points
                               only; lanes_per_row 0, block_threads 0 or 256,
                               num_blocks the row chunks, at most 1024, each of at
                               most 512 rows; rows at most 65535) */
    int32_t vec_bytes;      /* bytes per load/store: 16, 8, 4 or the element size */
    int32_t block_threads;  /* threads per block: 64..1024, multiple of lanes_per_row */
    int32_t num_blocks;     /* grid size (for rmsnorm_vjp also the number of dw partial rows) */
} rmsn_config_t;

/* y[rows, D] = rmsnorm(x) * (weight_bias + w).  See the file header. */
int rmsnorm_fwd(const void *x, const void *w, void *y,
                int64_t rows, int64_t D, int dt,
                float eps, float weight_bias, void *hip_stream);

/* new_residual = x + residual; normed = rmsnorm(x + residual) * (weight_bias + w). */
int fused_add_rmsnorm_fwd(const void *x, const void *residual, const void *w,
                          void *normed, void *new_residual,
                          int64_t rows, int64_t D, int dt,
                          float eps, float weight_bias, void *hip_stream);

/* Bytes of workspace rmsnorm_vjp (and every backward entry point, including
 * rmsnorm_backward with dw in the weight dtype) needs for this shape on the
 * current device: fp32 dw partials, [num_blocks, D] with num_blocks bounded
 * independently of rows and below the rows whenever there are two or more
 * (at least one row); for few rows of a wide D (the column-split plan),
 * also the rows' statistics, two floats per row and slice of 1024 vectors,
 * ahead of the partial rows.  0 for invalid arguments.  Never more than
 * 2048 * D * 4 + 256. */
size_t rmsnorm_vjp_workspace_bytes(int64_t rows, int64_t D, int dt);

/* dx[rows, D] (dtype dt) and dw[D] (fp32, overwritten).  `workspace` is
 * device memory of at least rmsnorm_vjp_workspace_bytes(rows, D, dt) bytes,
 * 16-byte aligned (RMSN_E_ALIGN otherwise); its contents on entry do not
 * matter and are left undefined. */
int rmsnorm_vjp(const void *x, const void *w, const void *dy,
                void *dx, float *dw, void *workspace, size_t workspace_bytes,
                int64_t rows, int64_t D, int dt,
                float eps, float weight_bias, void *hip_stream);

/* Bytes of the library's own device scratch used by rmsnorm_vjp_noalloc
 * (one array per GPU, held until the process ends). */
#define RMSN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* rmsnorm_vjp without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same operation,
 * kernels and results as rmsnorm_vjp (dx and dw bit-identical for the same
 * arguments); the dw partial rows live in a file-scope device array of
 * RMSN_NOALLOC_SCRATCH_BYTES bytes inside the library.  The first call on a
 * device looks up that array's device address once (hipGetSymbolAddress);
 * no call allocates or frees memory.  Shapes whose workspace
 * (rmsnorm_vjp_workspace_bytes) exceeds RMSN_NOALLOC_SCRATCH_BYTES (e.g.
 * num_blocks * D * 4 bytes of partial rows for D above 2^14 with 256
 * partial rows) return RMSN_E_WORKSPACE before any launch.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in
 * time on one GPU (two streams, two threads) race and must be serialised by
 * the caller.  Nothing in the scratch needs to start at any value. */
int rmsnorm_vjp_noalloc(const void *x, const void *w, const void *dy,
                        void *dx, float *dw,
                        int64_t rows, int64_t D, int dt,
                        float eps, float weight_bias, void *hip_stream);

/* Grad call: y (as rmsnorm_fwd), dx and dw (as rmsnorm_vjp) from one pass
 * over x and dy.  Same workspace rule as rmsnorm_vjp; y may be x or dy in
 * place (not dx), like dx. */
int rmsnorm_fwd_vjp(const void *x, const void *w, const void *dy,
                    void *y, void *dx, float *dw, void *workspace, size_t workspace_bytes,
                    int64_t rows, int64_t D, int dt,
                    float eps, float weight_bias, void *hip_stream);

/* Backward of fused_add_rmsnorm_fwd: dh[rows, D] = VJP of rmsnorm at h (the
 * new_residual the forward returned) for dy, plus d_new_residual; dw as
 * rmsnorm_vjp.  dh is the gradient of both x and residual.  Same workspace
 * rule as rmsnorm_vjp. */
int fused_add_rmsnorm_vjp(const void *h, const void *w, const void *dy, const void *d_new_residual,
                          void *dh, float *dw, void *workspace, size_t workspace_bytes,
                          int64_t rows, int64_t D, int dt,
                          float eps, float weight_bias, void *hip_stream);

/* Gated activation: y[rows, d] = silu(x[:, :d]) * x[:, d:2d] for x[rows, 2d]
 * (x and y of dtype dt, row-major, contiguous).  y must not overlap x.  No
 * workspace.  Errors: RMSN_E_SHAPE for rows < 0, d < 1, d > RMSN_MAX_GATE_D
 * or a size that overflows; the usual pointer, alignment and dtype codes.
 * First-half elements below -88.7 give silu = -0 (true magnitude < 6e-37). */
int silu_gate(const void *x, void *y, int64_t rows, int64_t d, int dt, void *hip_stream);

/* Backward of silu_gate: dx[rows, 2d] (gradient of the first half, then of
 * the second) for x[rows, 2d] and the upstream gradient dy[rows, d], all of
 * dtype dt.  dx may be x itself (in place); it must not overlap dy.  fp32
 * arithmetic, one rounding per output; errors as silu_gate. */
int silu_gate_vjp(const void *x, const void *dy, void *dx, int64_t rows, int64_t d, int dt,
                  void *hip_stream);

/* General backward, one entry point for the three backward forms and the
 * weight-gradient dtype: the VJP (y and d_new_residual NULL), the grad call
 * (y non-NULL, as rmsnorm_fwd_vjp) or the fused backward (d_new_residual
 * non-NULL, as fused_add_rmsnorm_vjp; x is then h).  dw has dtype dw_dt:
 * RMSN_F32, or dt -- the weight's dtype, the fp32 sum rounded once to
 * nearest even (the MLX pull request above prices its gw temporary at the
 * input's itemsize in "Proposed changes", i.e. its gw is in the storage
 * dtype).  y and d_new_residual together return
 * RMSN_E_CONFIG; another dw_dt returns RMSN_E_DTYPE.  Workspace: at least
 * rmsnorm_vjp_workspace_bytes(rows, D, dt) (or, with cfg, num_blocks * D * 4,
 * and D * 4 for a one-block grid with dw in the weight dtype).  cfg may be
 * NULL. */
int rmsnorm_backward(const void *x, const void *w, const void *dy, const void *d_new_residual,
                     void *y, void *dx, void *dw, int dw_dt,
                     void *workspace, size_t workspace_bytes,
                     int64_t rows, int64_t D, int dt, float eps, float weight_bias,
                     const rmsn_config_t *cfg, void *hip_stream);

/* The same operations with an explicit kernel configuration (NULL =
 * automatic).  For rmsnorm_vjp_cfg the workspace must hold
 * num_blocks * D * 4 bytes for the configuration actually used. */
int rmsnorm_fwd_cfg(const void *x, const void *w, void *y,
                    int64_t rows, int64_t D, int dt, float eps, float weight_bias,
                    const rmsn_config_t *cfg, void *hip_stream);
int fused_add_rmsnorm_fwd_cfg(const void *x, const void *residual, const void *w,
                              void *normed, void *new_residual,
                              int64_t rows, int64_t D, int dt, float eps, float weight_bias,
                              const rmsn_config_t *cfg, void *hip_stream);
int rmsnorm_vjp_cfg(const void *x, const void *w, const void *dy,
                    void *dx, float *dw, void *workspace, size_t workspace_bytes,
                    int64_t rows, int64_t D, int dt, float eps, float weight_bias,
                    const rmsn_config_t *cfg, void *hip_stream);
int rmsnorm_fwd_vjp_cfg(const void *x, const void *w, const void *dy,
                        void *y, void *dx, float *dw, void *workspace, size_t workspace_bytes,
                        int64_t rows, int64_t D, int dt, float eps, float weight_bias,
                        const rmsn_config_t *cfg, void *hip_stream);
int fused_add_rmsnorm_vjp_cfg(const void *h, const void *w, const void *dy,
                              const void *d_new_residual, void *dh, float *dw,
                              void *workspace, size_t workspace_bytes,
                              int64_t rows, int64_t D, int dt, float eps, float weight_bias,
                              const rmsn_config_t *cfg, void *hip_stream);
/* For silu_gate_cfg: lanes_per_row must be 0; vecs_per_lane (1, 2, 4, 8) is
 * the number of output vectors each thread handles per chunk; num_blocks is
 * the grid (the kernel loops over chunks of block_threads * vecs_per_lane
 * output vectors). */
int silu_gate_cfg(const void *x, void *y, int64_t rows, int64_t d, int dt,
                  const rmsn_config_t *cfg, void *hip_stream);
int silu_gate_vjp_cfg(const void *x, const void *dy, void *dx, int64_t rows, int64_t d, int dt,
                      const rmsn_config_t *cfg, void *hip_stream);

/* Operation ids for rmsn_query_config. */
#define RMSN_OP_FWD 0
#define RMSN_OP_FUSED 1
#define RMSN_OP_VJP 2
#define RMSN_OP_GRAD 3
#define RMSN_OP_FUSED_VJP 4
#define RMSN_OP_GATE 5      /* D is the half width d */

/* Fill *out with the configuration the automatic choice makes for `op` on
 * this shape.  `align_bytes` (a power of two: the alignment of the
 * pointers) is validated but does not change the choice, which depends on
 * the shape, the dtype and the current device's compute-unit count only
 * (persistent grids; forward calls on no more rows than compute units take
 * one row per block).  Returns RMSN_OK or an argument error.  For the backward forms
 * the library additionally picks, per call, between two row loops of the same
 * geometry and arithmetic: a software-pipelined one (rows of exactly
 * lanes_per_row * vecs_per_lane vectors; power-of-two rows in blocks of at
 * most 256 threads or as one 512-lane row per block; wave rows and
 * four-vector rows always; the grad call only where an instance with the
 * lanes fixed exists) and the plain one; the choice does not change any
 * result. */
int rmsn_query_config(int op, int64_t rows, int64_t D, int dt, int align_bytes,
                      rmsn_config_t *out);

/* Static text for a status code. */
const char *rmsn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MI355X_H */
