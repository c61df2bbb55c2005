/*
 * mb.h -- C ABI of the fused Transformer epilogue kernels for AMD MI355X (gfx950).
 *
 * The operations are the memory-bound epilogues that Megatron-LM fuses, as
 * described by the wmrh.cn article on Megatron-LM's megatron/core/fusions
 * package (wmrh.cn/news/51426), cited here as [fusions §N] for its section N.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout:   tensors are row-major and contiguous. "tokens" (T) is the number
 *           of rows, "hidden" (H) the number of columns. A bias has H entries
 *           and is broadcast over the rows.
 * Pointers: every pointer is a DEVICE pointer, owned by the caller. The
 *           library allocates nothing, keeps no state between calls and never
 *           synchronizes: work is enqueued on the caller's stream `s` and the
 *           call returns at once. Calls are thread-safe.
 * dtypes:   `dt` is the storage type of the inputs and outputs; arithmetic is
 *           fp32 in registers and each output is rounded once, to nearest
 *           even. Bias and weight gradients are always fp32.
 * Shapes:   T >= 0; H > 0; H * sizeof(dt) must be a multiple of 16 bytes
 *           (H % 8 == 0 for bf16/fp16, H % 4 == 0 for fp32), because every
 *           lane moves whole 16-byte vectors (residual add + LayerNorm states
 *           its own rule).
 * Alignment: tensor and bias pointers must be 16-byte aligned; fp32 gradient
 *           outputs 4-byte aligned; workspaces 16-byte aligned.
 * Aliasing: only the exact aliases listed per entry point are allowed; any
 *           other overlap of two buffers is rejected.
 * Errors:   arguments are validated on the host before any HIP call; a bad
 *           argument returns an error code and enqueues nothing. After the
 *           launches, a pending HIP error is returned as MB_ERR_HIP. Nothing
 *           throws across the ABI.
 * Empty:    T == 0 enqueues nothing, except that a requested bias gradient is
 *           written as zeros.
 * Reductions: bias, weight and LayerNorm parameter gradients are fixed-order
 *           sums with no atomic accumulation. Their grouping of rows follows
 *           the shape and the device's compute-unit count, so repeated calls
 *           on one device give the same bits; devices with another CU count
 *           (a partitioned one, say) round differently within the stated
 *           tolerance.
 */
#ifndef MB_H
#define MB_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* The last two enumerators only widen the type's range to every 32-bit int, so
 * that an unknown value from a caller is a value the library can check and
 * refuse (MB_ERR_DTYPE) rather than an out-of-range enum in C++. */
typedef enum {
  MB_F32 = 0,
  MB_F16 = 1,
  MB_BF16 = 2,
  MB_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  MB_DTYPE_RANGE_MAX_ = 2147483647
} mb_dtype_t;

typedef enum {
  MB_OK = 0,
  MB_ERR_NULL = 1,      /* a required pointer is NULL */
  MB_ERR_SHAPE = 2,     /* T < 0, H <= 0, H*sizeof(dt) % 16 != 0, or size overflow */
  MB_ERR_DTYPE = 3,     /* unknown or unsupported dtype combination */
  MB_ERR_ALIGN = 4,     /* a pointer is not aligned as required */
  MB_ERR_ALIAS = 5,     /* two buffers overlap in a way the entry point forbids */
  MB_ERR_PROB = 6,      /* dropout probability NaN or outside [0, 1]; LayerNorm eps not finite or < 0 */
  MB_ERR_WORKSPACE = 7, /* workspace missing or smaller than the query returned */
  MB_ERR_HIP = 8,       /* the HIP runtime reported an error for the launches */
  MB_ERR_SCRATCH = 9    /* needs more than the static scratch of mb_bias_gelu_bwd_noalloc */
} mb_status_t;

/* Human-readable name of a status code (static storage). */
const char* mb_status_string(mb_status_t status);

/* ABI version. 1: dropout keep word = Philox4x32-10 word (i mod 4) of block
 * counter (i/4, offset), key seed, one 32-bit word per element. */
int mb_abi_version(void);

/* ---------------------------------------------------------------------------
 * Bias + GeLU, tanh approximation [fusions §4.2, §4.3]
 *   z   = y + bias
 *   out = 0.5 z (1 + tanh(0.79788456 z (1 + 0.044715 z^2)))
 * y [T,H], bias [H] (NULL: no bias), out [T,H]; out may equal y (in place).
 * ------------------------------------------------------------------------- */
mb_status_t mb_bias_gelu_fwd(const void* y, const void* bias, void* out, int64_t tokens,
                             int64_t hidden, mb_dtype_t dt, hipStream_t s);

/* Bytes of workspace mb_bias_gelu_bwd needs for the bias gradient (0 when
 * with_dbias = 0 or tokens = 0). */
size_t mb_bias_gelu_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dbias);

/* Backward of bias + GeLU [fusions §4.2, §4.3]:
 *   dgrad = g * gelu'(y + bias),
 *   gelu'(z) = 0.5 (1 + t) + 0.5 z (1 - t^2)(0.79788456 + 0.1070322243 z^2),
 *   t = tanh(0.79788456 z (1 + 0.044715 z^2));
 *   dbias[j] = sum over rows of the fp32 dgrad[:, j] (before rounding).
 * g, y, dgrad [T,H]; bias [H] (NULL: none); dbias [H] fp32 (NULL: not computed).
 * dgrad may equal g or y. The reduction is deterministic and atomic-free: a
 * second launch sums per-row-group partials kept in the workspace `ws`
 * (ws_bytes >= mb_bias_gelu_bwd_workspace(...); unused when dbias is NULL). */
mb_status_t mb_bias_gelu_bwd(const void* g, const void* y, const void* bias, void* dgrad,
                             float* dbias, void* ws, size_t ws_bytes, int64_t tokens,
                             int64_t hidden, mb_dtype_t dt, hipStream_t s);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): mb_bias_gelu_bwd
 * without a workspace argument. It calls no allocating routine; the bias
 * gradient's partial rows go to a static device array of the library, 16 MiB
 * per GPU, held from the first call on that GPU
 * until the process ends. Same arguments, results and errors as
 * mb_bias_gelu_bwd: dgrad is bit for bit the same; dbias is the same column
 * sum taken over fewer, larger row groups (the scratch bounds them to
 * min(512, 16 MiB / (4 hidden)) rows), so it can differ in the last bits.
 * MB_ERR_SCRATCH when dbias != NULL and one fp32 row of hidden values does
 * not fit the scratch (hidden > 4194304). Limits: every call on one GPU shares
 * that GPU's scratch, so calls that overlap in time on one GPU (different
 * streams, or threads) race and must be serialized by the caller; the first
 * call on each GPU looks up the scratch address and should not be made under
 * graph capture. The scratch keeps the last call's contents; nothing in it
 * needs to start at zero. */
mb_status_t mb_bias_gelu_bwd_noalloc(const void* g, const void* y, const void* bias, void* dgrad,
                                     float* dbias, int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                     hipStream_t s);

/* Exact GeLU [fusions §4.2, the erf definition with its printed constants]:
 *   out = 0.5 z (1 + erf(0.70710678 z)),  z = y + bias;
 * same arguments, aliasing and errors as mb_bias_gelu_fwd. erfc is evaluated
 * to 2e-7 relative for fp32 outputs (and in the backward) and to 3.5e-5
 * relative for bf16/fp16 outputs, well inside half an output ulp. */
mb_status_t mb_bias_gelu_erf_fwd(const void* y, const void* bias, void* out, int64_t tokens,
                                 int64_t hidden, mb_dtype_t dt, hipStream_t s);

/* Workspace bytes for mb_bias_gelu_erf_bwd (its own launch shape). */
size_t mb_bias_gelu_erf_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                      int with_dbias);

/* Backward of the exact GeLU:
 *   dgrad = g * (0.5 (1 + erf(0.70710678 z)) + z * 0.3989423 * exp(-z^2 / 2)),
 *   dbias as for mb_bias_gelu_bwd; the workspace is sized by
 *   mb_bias_gelu_erf_bwd_workspace. */
mb_status_t mb_bias_gelu_erf_bwd(const void* g, const void* y, const void* bias, void* dgrad,
                                 float* dbias, void* ws, size_t ws_bytes, int64_t tokens,
                                 int64_t hidden, mb_dtype_t dt, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Bias + dropout + residual add [fusions §3.2, §3.3]
 *   r'  = residual rounded to dt when residual_dt != dt (the mixed-precision
 *         cast of the residual to x's dtype), else residual;
 *   z   = x + bias;
 *   train: out = r' + (keep ? z * s : 0),  s = (float)(1 / (1 - p));
 *   infer: out = r' + z  (dropout is the identity at inference).
 * x, out [T,H] dtype dt; bias [H] dtype dt (NULL: none); residual [T,H] of
 * dtype residual_dt, which is dt or MB_F32. out may equal x, or residual when
 * residual_dt == dt (in place).
 * keep: element i = t*H + j is kept iff word >= floor(p * 2^32), where word is
 * 32-bit word (i mod 4) of Philox4x32-10 (Salmon et al., SC'11) applied to the
 * counter (lo32(i/4), hi32(i/4), lo32(offset), hi32(offset)) with the key
 * (lo32(seed), hi32(seed)). The mask is therefore a pure function of
 * (seed, offset, element index): it is reproducible and independent of the
 * launch shape. p in [0, 1]; p = 0 keeps all, p = 1 drops all.
 * ------------------------------------------------------------------------- */
mb_status_t mb_bias_dropout_add_train(const void* x, const void* bias, const void* residual,
                                      mb_dtype_t residual_dt, void* out, int64_t tokens,
                                      int64_t hidden, mb_dtype_t dt, float p, uint64_t seed,
                                      uint64_t offset, hipStream_t s);

mb_status_t mb_bias_dropout_add_infer(const void* x, const void* bias, const void* residual,
                                      mb_dtype_t residual_dt, void* out, int64_t tokens,
                                      int64_t hidden, mb_dtype_t dt, hipStream_t s);

/* Bytes of workspace mb_bias_dropout_add_bwd needs for the bias gradient
 * (0 when with_dbias = 0 or tokens = 0). */
size_t mb_bias_dropout_add_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dbias);

/* Backward of mb_bias_dropout_add_train for the same (p, seed, offset): with
 * g = d loss / d out [T,H] (dtype dt),
 *   dx[t, j]        = g * s where the element was kept, 0 where dropped
 *                     (the keep decisions are regenerated, nothing is stored);
 *   dresidual[t, j] = g in the residual's dtype residual_dt (dt or MB_F32):
 *                     the cast of the residual passes the gradient through;
 *                     NULL skips it (with residual_dt == dt it equals g);
 *   dbias[j]        = sum over rows of the fp32 dx[:, j] (NULL: skip; the bias
 *                     gradient equals that of x summed over tokens [fusions §4.3]).
 * dx may equal g (in place); dresidual may equal g only when residual_dt == dt.
 * The reduction is deterministic and atomic-free (second launch over partials
 * in ws, ws_bytes >= mb_bias_dropout_add_bwd_workspace(...)). Needs p in [0, 1]. */
mb_status_t mb_bias_dropout_add_bwd(const void* g, void* dx, void* dresidual, mb_dtype_t residual_dt,
                                    float* dbias, void* ws, size_t ws_bytes, int64_t tokens, int64_t hidden,
                                    mb_dtype_t dt, float p, uint64_t seed, uint64_t offset, hipStream_t s);

/* The keep decisions mb_bias_dropout_add_train makes for (T, H, p, seed,
 * offset), as bits: bit (i mod 8) of byte i/8 is element i = t*H + j
 * (1 = kept). bits holds ceil(T*H/8) bytes; unused high bits of the last byte
 * are 0. Needs H % 4 == 0. Lets a backward pass or a test regenerate the mask. */
mb_status_t mb_dropout_mask(uint8_t* bits, int64_t tokens, int64_t hidden, float p, uint64_t seed,
                            uint64_t offset, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Bias + gated linear units [fusions §2, §9]
 * The input row has 2H columns: a = in[t, 0:H] + bias[0:H] goes through the
 * activation, b = in[t, H:2H] + bias[H:2H] is the linear half.
 *   SwiGLU: out = silu(a) * b (* w[t] when weights are given),
 *           silu(a) = a / (1 + exp(-a));
 *   GEGLU:  out = gelu_tanh(a) * b.
 * `hidden` is H, the output width. in [T,2H], bias [2H] (NULL: none),
 * weights [T] of dtype weights_dt (dt or MB_F32; NULL: unweighted), out [T,H].
 * out must not overlap in.
 * ------------------------------------------------------------------------- */
mb_status_t mb_bias_swiglu_fwd(const void* in, const void* bias, const void* weights,
                               mb_dtype_t weights_dt, void* out, int64_t tokens, int64_t hidden,
                               mb_dtype_t dt, hipStream_t s);

mb_status_t mb_bias_geglu_fwd(const void* in, const void* bias, void* out, int64_t tokens,
                              int64_t hidden, mb_dtype_t dt, hipStream_t s);

/* Workspace bytes for the gated backward passes. */
size_t mb_bias_glu_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dbias,
                                 int with_dweights);

/* Backward of bias + SwiGLU (weighted when weights != NULL):
 *   da = g * w * b * silu'(a),  silu'(a) = sigmoid(a) (1 + a (1 - sigmoid(a)))
 *   db = g * w * silu(a)
 *   din[t, 0:H] = da, din[t, H:2H] = db          (dtype dt)
 *   dbias[c]    = sum over rows of fp32 din[:, c] (fp32 [2H], NULL: skip)
 *   dweights[t] = sum over j of g * silu(a) * b   (fp32 [T], NULL: skip;
 *                                                  needs weights)
 * g [T,H], in and din [T,2H]; din may equal in (in place); g must not
 * overlap din. The reductions are deterministic and atomic-free (second
 * launch over partials in ws). */
mb_status_t mb_bias_swiglu_bwd(const void* g, const void* in, const void* bias, const void* weights,
                               mb_dtype_t weights_dt, void* din, float* dbias, float* dweights,
                               void* ws, size_t ws_bytes, int64_t tokens, int64_t hidden,
                               mb_dtype_t dt, hipStream_t s);

/* Backward of bias + GEGLU: da = g * b * gelu_tanh'(a), db = g * gelu_tanh(a),
 * with gelu_tanh' as in mb_bias_gelu_bwd; din, dbias as for SwiGLU. */
mb_status_t mb_bias_geglu_bwd(const void* g, const void* in, const void* bias, void* din,
                              float* dbias, void* ws, size_t ws_bytes, int64_t tokens,
                              int64_t hidden, mb_dtype_t dt, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Weighted squared ReLU for MoE experts [fusions §2 and §8 name the fused op
 * and its switch, §9 its unit test; no formula is printed]. Read as the
 * weighted-SwiGLU pattern of §9 (the unweighted activation times the
 * per-token weight) applied to the squared ReLU:
 *   out[t, j] = relu(x)^2 * w[t]
 * relu passes NaN through. weights [T] of weights_dt (fp32, fp16 or bf16) or
 * NULL for the plain squared ReLU. x, out [T,H] dt; out may equal x (in
 * place). Errors as for mb_bias_gelu_fwd; weights must be aligned to their
 * element size. */
mb_status_t mb_weighted_squared_relu_fwd(const void* x, const void* weights, mb_dtype_t weights_dt,
                                         void* out, int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                         hipStream_t s);

/* Workspace bytes for the weights gradient of mb_weighted_squared_relu_bwd. */
size_t mb_weighted_squared_relu_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                              int with_dweights);

/* Backward:
 *   dx[t, j]    = g * w[t] * 2 relu(x)              (dtype dt; may equal g or x)
 *   dweights[t] = sum over j of g * relu(x)^2        (fp32 [T], NULL: skip;
 *                                                    needs weights)
 * The weights gradient is deterministic and atomic-free: per-strip row
 * partials in ws, then an ordered sum over the strips. */
mb_status_t mb_weighted_squared_relu_bwd(const void* g, const void* x, const void* weights,
                                         mb_dtype_t weights_dt, void* dx, float* dweights, void* ws,
                                         size_t ws_bytes, int64_t tokens, int64_t hidden,
                                         mb_dtype_t dt, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Residual add + LayerNorm [fusions §5.1-§5.4: the fused LayerNorm that
 * Megatron-LM wraps, its eps (default 1e-5) in the denominator, and the
 * zero-centred gamma applied as weight + 1], fused with the residual add that
 * precedes it on a layer's residual path. The normalisation is the standard
 * one over the hidden dimension with the biased (1/H) variance:
 *   h[t, j] = x + residual'     residual' = residual cast to dt when it is fp32
 *                               (as in the dropout-add); h rounded to dt
 *   mean_t  = (1/H) sum_j h,  var_t = (1/H) sum_j (h - mean_t)^2
 *   rstd_t  = 1 / sqrt(var_t + eps)
 *   y[t, j] = (h - mean_t) * rstd_t * gamma'_j + beta_j
 *   gamma'  = gamma + 1 when zero_centered_gamma != 0, else gamma
 * computed in fp32 from the ROUNDED h.
 *
 * x, y, h_out [T,H] dt; residual [T,H] residual_dt (= dt, or MB_F32 beside
 * fp16/bf16); gamma [H] dt (required), beta [H] dt or NULL (0); h_out NULL
 * skips storing h; mean, rstd [T] fp32, both or neither (the backward needs
 * them). hidden: a multiple of 8 elements for fp16/bf16 rows (4 with an fp32
 * residual, and for fp32) and at most 65536 fp16/bf16 or 32768 fp32 (or
 * fp16/bf16 with an fp32 residual) elements. eps: finite, >= 0.
 * Aliasing: h_out and y may each equal x or residual exactly (same dtype),
 * never each other; nothing else may overlap. Errors: MB_ERR_DTYPE,
 * MB_ERR_SHAPE, MB_ERR_NULL, MB_ERR_ALIGN (16-byte tensors, 4-byte mean/rstd),
 * MB_ERR_ALIAS, MB_ERR_PROB (eps out of range), MB_ERR_HIP. */
mb_status_t mb_add_layer_norm_fwd(const void* x, const void* residual, mb_dtype_t residual_dt,
                                  const void* gamma, const void* beta, float eps,
                                  int zero_centered_gamma, void* h_out, void* y, float* mean,
                                  float* rstd, int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                  hipStream_t s);

/* Workspace bytes for mb_add_layer_norm_bwd: rows of more than 2048 16-byte
 * vectors (over 16384 fp16/bf16 elements, over 8192 fp32 or beside an fp32
 * residual) keep their row sums there (a pair of fp32 partial sums per row
 * and block of the row when a row is split over up to 8 blocks, else two
 * fp32 sums per row); with parameter gradients it also holds their partial
 * rows. 0 when neither applies (and for tokens 0). */
size_t mb_add_layer_norm_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                       mb_dtype_t residual_dt, int with_param_grads);

/* Backward of residual add + LayerNorm, from the forward's h, mean and rstd.
 * With a = dy * gamma' and xhat = (h - mean) * rstd:
 *   dh[t, j]  = rstd * (a - (1/H) sum_j a - xhat (1/H) sum_j a xhat) + dh_in
 *   dx        = dh in dt;  dresidual = dh in residual_dt (NULL: skip)
 *   dgamma[j] = sum_t dy * xhat,  dbeta[j] = sum_t dy   (fp32 [H], NULL: skip)
 * dh_in [T,H] residual_dt or NULL: the gradient reaching h from its use as the
 * next residual. dx may equal dy or h exactly; dresidual may equal dh_in, or
 * dy or h when residual_dt == dt. The parameter gradients are deterministic
 * and atomic-free (partials in ws, sized by mb_add_layer_norm_bwd_workspace,
 * then ordered column sums). Rows of 2049-8192 vectors are split over teams
 * of blocks that exchange their partial row sums through ws (agent-scope
 * atomic stores and loads; a block that waits in vain past a bound leaves the
 * row to a second pass that recomputes the sums the same way, so results do
 * not depend on timing). With an output over an input such rows take two
 * passes over dy and h instead: the same values within the stated bound, not
 * bit for bit those of the out-of-place call. Errors as for the forward, plus
 * MB_ERR_WORKSPACE. */
mb_status_t mb_add_layer_norm_bwd(const void* dy, const void* h, const void* gamma,
                                  const float* mean, const float* rstd, int zero_centered_gamma,
                                  const void* dh_in, mb_dtype_t residual_dt, void* dx,
                                  void* dresidual, float* dgamma, float* dbeta, void* ws,
                                  size_t ws_bytes, int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                  hipStream_t s);

/* Test-only. Rows of 2049-8192 vectors are split over a team of blocks that
 * exchange their partial row sums [fusions §5.3: the widest hidden sizes];
 * a block polls for a partner's sums at most `polls` times (negative: the
 * default, 4096) and then computes them itself, with the same arithmetic,
 * so outputs do not depend on it: a test sets 0 to run every row through
 * that path and compares. Applies to later calls in this process. */
void mb_set_layer_norm_team_wait(int polls);

#ifdef __cplusplus
}
#endif

#endif /* MB_H */
