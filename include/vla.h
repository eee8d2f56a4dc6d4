/*
 * vla.h - C ABI of the MI355X (gfx950) Variational Linear Attention scan.
 *
 * The library exports these compute entry points:
 *
 *   vla_scan_forward  the VLA recurrence scan over a sequence, per (batch, head)
 *   vla_scan_step     one token per chain with the state updated in place
 *                     (streaming decode)
 *   vla_scan_forward_fused  the scan from raw q, k and W_u (feature map and
 *                     projection fused in)
 *   vla_scan_backward the gradients of the scan (additive update)
 *   vla_project_u     the learned penalty directions u = normalize(W_u k_raw)
 *
 * plus parameter, workspace and status helpers.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers (memory on the current HIP device)
 *   unless a comment says otherwise.  The caller owns every buffer; the library
 *   never allocates, frees or retains device memory.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Work is enqueued asynchronously on it; no call synchronises the host,
 *   except vla_scan_forward with `validate` set (documented there).  The
 *   chunked schedule also runs part of its work on a side stream the library
 *   owns (one per device, default priority, created on first use and kept):
 *   that work is ordered after what `stream` already holds and joined back
 *   into `stream` with events before the call returns, so whatever is
 *   enqueued on `stream` later sees all of it.
 * - Layouts are row-major with the feature dimension contiguous.
 * - Errors: every argument and shape check happens before anything is
 *   launched.  A failed check returns VLA_EINVAL or VLA_EUNSUPPORTED and
 *   writes nothing.  A failed launch returns VLA_EHIP.  Faults inside a kernel
 *   surface at the caller's next synchronisation, as usual for HIP.  No C++
 *   exception crosses this interface.  vla_last_error() gives a thread-local
 *   message for the last failure on the calling thread.
 * - Calls are thread-safe; calls on different streams may overlap.
 */
#ifndef VLA_H_
#define VLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VLA_ABI_VERSION 3

typedef enum {
  VLA_OK = 0,
  VLA_EINVAL = 1,        /* bad argument (null pointer, negative size, inconsistent shape) */
  VLA_EUNSUPPORTED = 2,  /* well-formed but outside the supported set (d, r, dtype) */
  VLA_EWORKSPACE = 3,    /* workspace missing or smaller than vla_scan_workspace_size() */
  VLA_ENONFINITE = 4,    /* validate was set and an input holds NaN or Inf */
  VLA_EHIP = 5           /* a HIP runtime call failed */
} vla_status_t;

typedef enum { VLA_F32 = 0, VLA_BF16 = 1 } vla_dtype_t;

typedef enum {
  VLA_SCHEDULE_AUTO = 0,        /* library picks */
  VLA_SCHEDULE_SEQUENTIAL = 1,  /* one workgroup owns a (batch, head) chain for the whole sequence */
  VLA_SCHEDULE_CHUNKED = 2      /* time-parallel inverse pass over chunks, then a per-chain state
                                   pass (d = 64; needs workspace; see vla_scan_forward) */
} vla_schedule_t;

/* The state step of the recurrence.  ADDITIVE is the update of "Mathematical
 * Primitives", section 5 (S += v alpha_hat^T, alpha_hat = alpha / max(|alpha|, 1)).
 * RESIDUAL is the recursive update rule of "Variational Linear Attention:
 * Stable Associative Memory for Long-Context Transformers", technical summary
 * 2.3: k_hat = k / |k|, alpha_hat = A_t k_hat / |A_t k_hat| (unit), and
 * S += (v - S k_hat) alpha_hat^T with the prediction S k_hat taken before the
 * update; normalisations divide by max(|x|, 1e-12). */
typedef enum {
  VLA_UPDATE_ADDITIVE = 0,
  VLA_UPDATE_RESIDUAL = 1
} vla_update_t;

/* Parameters of one scan call.  Fill with vla_scan_params_init() first. */
typedef struct {
  int32_t B, H;          /* batch and heads: B*H independent chains */
  int32_t T;             /* tokens in this call (0 copies the state through) */
  int32_t d;             /* head dimension: 16, 32, 64 or 128 */
  int32_t r;             /* penalty directions per token (Woodbury rank): 1..4 */
  int32_t in_dtype;      /* vla_dtype_t: storage of q, k, v, u and of the output o */
  float eps;             /* guard threshold and nudge size (default 1e-6) */
  int32_t nudge_period;  /* eps*I added to A every nudge_period tokens; 0 = off */
  float s_cap;           /* Frobenius cap on S; <= 0 or +inf = off */
  float den_eps;         /* readout denominator epsilon (default 1e-6) */
  int64_t t0;            /* global index of this call's first token (nudge phase, resume) */
  int64_t stride_b;      /* element strides of q, k and v (shared) over batch, head and */
  int64_t stride_h;      /* token; the feature dimension is contiguous.  All three 0 means */
  int64_t stride_t;      /* the contiguous [B, H, T, d] layout (see vla_scan_forward) */
  int32_t schedule;      /* vla_schedule_t */
  int32_t validate;      /* nonzero: synchronous NaN/Inf pre-check of the inputs */
  int32_t chunk_len;     /* tokens per chunk of the chunked schedule; 0 = library picks */
  int32_t segment_blocks; /* chunked schedule: blocks of 64 tokens per state-pass
                             segment, rounded up to a multiple of 4 and to at
                             most 16 segments; the first is five eighths as
                             long and a remainder under half a segment is
                             shared with the one before (the chain kernel runs
                             one segment while a side stream preps the next
                             and reads out the last); 0 = library picks (256),
                             < 0 = one segment */
  int32_t update;        /* vla_update_t (both schedules) */
  int32_t para_segments; /* chunked schedule, additive update: the per-chain state
                            pass cut into this many segments (2..16) that run in
                            parallel from guessed starts, corrected by sweeps
                            until the starts stop moving; 1 = one pass per chain
                            (the segmented pipeline above); 0 = library picks
                            (min(16, 256 / chains, blocks / 32), blocks of 64
                            tokens per chain; below 2 means one pass); an
                            explicit count is capped at blocks / 2 */
} vla_scan_params_t;

/* Defaults: B = H = T = 0, d = 64, r = 1, f32, eps = 1e-6, no nudge, no cap,
 * den_eps = 1e-6, t0 = 0, contiguous q, k, v (strides 0), automatic schedule,
 * no validation, chunk_len = 0, segment_blocks = 0, additive update,
 * para_segments = 0.  Host pointer. */
void vla_scan_params_init(vla_scan_params_t* p);

/* Bytes of device workspace vla_scan_forward needs for these parameters
 * (host pointers in and out), for the schedule the call would use.  Zero for
 * the sequential schedule with contiguous q, k, v and without validation. */
vla_status_t vla_scan_workspace_size(const vla_scan_params_t* p, size_t* bytes);

/*
 * vla_scan_forward: the VLA recurrence, sequential over tokens, independent
 * per (batch, head) chain.
 *
 * Sources: "Mathematical Primitives" (VLA documentation), section 2
 * (Sherman-Morrison rank-1 inverse tracking: z = A u, delta = 1 + u.z, the
 * |delta| < eps guard that injects eps*I, A <- A - z z^T / delta, periodic
 * eps*I spectrum stabilisation), section 3 (rank r as r sequential rank-1
 * updates), section 4 (alpha_t = A_t k_t), section 5 (S_t = S_{t-1} + v alpha^T
 * and Frobenius renormalisation of S); "Variational Linear Attention (VLA)"
 * README, v3 notes (ELU+1 features applied upstream, normalised alpha, z.q
 * readout denominator).
 *
 * Per chain, for each token t (tau = t0 + t + 1, 1-based):
 *   for i = 1..r:  z = A u_{t,i};  delta = 1 + u_{t,i}.z
 *                  if |delta| < eps:  A += eps*I  (update skipped, counted)
 *                  else:              A -= z z^T / delta
 *   if nudge_period > 0 and tau % nudge_period == 0:  A += eps*I
 *   alpha = A k_t;  alpha_hat = alpha / max(|alpha|_2, 1)
 *   S += v_t alpha_hat^T                      (S is [value, key])
 *     (update = RESIDUAL instead: k_hat = k_t / |k_t|,
 *      alpha_hat = A k_hat / |A k_hat|, S += (v_t - S k_hat) alpha_hat^T)
 *   if cap on and |S|_F > s_cap:  S *= s_cap / |S|_F   (counted)
 *   n += k_t;  o_t = S q_t / (n.q_t + den_eps)
 *
 * Arguments (device pointers):
 *   q, k, v  [B, H, T, d] in in_dtype.  q and k are the positive (ELU+1)
 *            features; the library does not apply the feature map.  With the
 *            strides all 0 the three are contiguous.  Otherwise element
 *            (b, h, t, i) of each sits at element b*stride_b + h*stride_h +
 *            t*stride_t + i of its pointer (e.g. q, k, v sliced from one
 *            packed [B, T, H, 3d] projection: stride_b = T*H*3d, stride_h = 3d,
 *            stride_t = H*3d); each stride must be >= 0, stride_t >= d, and
 *            stride * element size a multiple of 16 bytes.  Strided inputs are
 *            first gathered into the workspace by a copy kernel, so the
 *            kernels of both schedules read them contiguously.
 *   u        [B, H, T, r, d] in in_dtype, contiguous; u[..., t, i, :] is the
 *            i-th direction of token t, applied in index order.
 *   A0, S0   [B, H, d, d] float32, n0 [B, H, d] float32: initial state.  Each
 *            may be NULL, meaning I, 0 and 0 respectively.
 *   o        [B, H, T, d] in in_dtype (written).
 *   A_T, S_T [B, H, d, d] float32 and n_T [B, H, d] float32: final state
 *            (written).  They may alias A0, S0, n0 exactly (in-place state
 *            carry); no other aliasing is allowed.
 *   stats    [B, H, 4] int32 or NULL: guard fires, cap fires, non-finite flag
 *            (1 if any output or final state of the chain is NaN/Inf), and the
 *            0-based index of the first cap fire in this call (-1 if none).
 *   workspace, workspace_bytes: device scratch of at least
 *            vla_scan_workspace_size() bytes (may be NULL when that is 0).
 * State is float32 throughout; products accumulate in float32.
 *
 * Schedules.  SEQUENTIAL runs each chain in one workgroup, token after token.
 * CHUNKED (d = 64; or d = 128 with bf16 storage, the additive update and no
 * cap) splits the tokens into chunks of chunk_len: while no guard fires, A_t
 * is the inverse of the accumulated penalty M_t = A0^{-1} + sum u u^T
 * ("Mathematical Primitives", section 2), so each chunk's starting inverse
 * follows in parallel from per-chunk Gram matrices (in float64, carrying the
 * nudges exactly), the inverse recurrence of every chunk runs in parallel
 * (at d = 128 a workgroup may carry A over a span of consecutive chunks),
 * and a state pass applies the state update, cap and readout.  A chain where
 * the guard fires, or whose chunk-start inverse is not positive definite, is
 * recomputed sequentially in the same call, so the result does not depend on
 * the schedule beyond float32 rounding.  At d = 64 the state pass runs either
 * parallel in time (para_segments segments of every chain at once from
 * guessed starts, corrected by per-chain sweeps until they stop moving) or
 * per chain in segments of segment_blocks blocks of 64 tokens, a segment's
 * chain kernel overlapping the next segment's preparation and the previous
 * one's readout on the side stream; at d = 128, without the cap, it is a
 * prefix sum over chunks with a chunked readout.  CHUNKED needs chunk_len to
 * divide nudge_period (when nonzero) and t0; AUTO uses it when there are few
 * chains and long sequences.
 *
 * With update = RESIDUAL the chunked schedule's inverse pass writes the unit
 * gates, and the state pass uses that, inside a block of 64 tokens, the
 * prediction errors solve a unit lower-triangular system, so each block maps
 * its starting state affinely, S -> S (I + N) + Q, with N and Q computed for
 * all blocks in parallel; a per-chain pass chains those maps, and a parallel
 * readout recovers every token's state and output.  A chain with a token
 * whose state exceeds s_cap is recomputed sequentially with the cap applied.
 *
 * With validate != 0 the call first checks q, k, v, u for NaN/Inf on the
 * stream (after the gather of strided inputs), synchronises the stream, and
 * returns VLA_ENONFINITE (having launched nothing else) if any is found.
 */
vla_status_t vla_scan_forward(const vla_scan_params_t* p,
                              const void* q, const void* k, const void* v, const void* u,
                              const float* A0, const float* S0, const float* n0,
                              void* o, float* A_T, float* S_T, float* n_T, int32_t* stats,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * vla_scan_step: one decode step, T = 1 token per chain, with the recurrent
 * state read and written in place.
 *
 * Source: "Variational Linear Attention: Stable Associative Memory for
 * Long-Context Transformers", technical summary (streaming inference with a
 * constant-size state and no growing cache); README, v3 notes item 5 (the
 * readout at decode time).  The token's arithmetic is vla_scan_forward's,
 * with tau = t0 + 1 for the nudge.
 *
 *   p        parameters as for vla_scan_forward; p->T must be 1 (VLA_EINVAL
 *            otherwise); p->t0 is the global index of this token
 *   q, k, v  [B, H, 1, d] in in_dtype (strides as in vla_scan_forward)
 *   u        [B, H, 1, r, d] in in_dtype
 *   A, S     [B, H, d, d] float32 and n [B, H, d] float32: the state before
 *            the token, overwritten with the state after it (non-NULL)
 *   o        [B, H, 1, d] in in_dtype (written); stats as in vla_scan_forward
 *   workspace as for vla_scan_forward (zero bytes unless strided or validated)
 */
vla_status_t vla_scan_step(const vla_scan_params_t* p,
                           const void* q, const void* k, const void* v, const void* u,
                           float* A, float* S, float* n, void* o, int32_t* stats,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * vla_scan_forward_fused: the scan with its prologue fused in: the feature
 * map and the penalty directions are computed from the raw inputs.
 *
 * Source: "Variational Linear Attention (VLA)" README, v3 notes items 1-2
 * (Q, K = ELU(.) + 1; u_t = normalize(W_u k_t^raw)).  Equivalent to
 *   q = ELU(q_raw) + 1, k = ELU(k_raw) + 1      (float32, ELU with alpha 1)
 *   u = normalize(W_u[i] k_raw)                 (vla_project_u)
 * each stored in in_dtype (bfloat16: round to nearest even), followed by
 * vla_scan_forward(q, k, v, u, ...) with the same parameters.
 *
 * When the call takes the sequential schedule with d <= 64 and more than
 * 16 tokens, the scan kernel itself streams q_raw, k_raw, v and builds each
 * token's features and u in LDS on the matrix cores (u never exists in
 * HBM; no workspace).  Otherwise a prologue pass writes q, k and u into the
 * workspace and the scan reads them there.
 *
 *   q_raw, k_raw, v [B, H, T, d] and W_u [r, d, d] in in_dtype (device,
 *   contiguous, 16-byte aligned); the rest as in vla_scan_forward.
 *   workspace: at least vla_scan_fused_workspace_size() bytes.
 * Strides must be 0 and validate 0 (VLA_EUNSUPPORTED otherwise); every other
 * error as in vla_scan_forward.
 */
vla_status_t vla_scan_fused_workspace_size(const vla_scan_params_t* p, size_t* bytes);
vla_status_t vla_scan_forward_fused(const vla_scan_params_t* p,
                                    const void* q_raw, const void* k_raw, const void* v, const void* W_u,
                                    const float* A0, const float* S0, const float* n0,
                                    void* o, float* A_T, float* S_T, float* n_T, int32_t* stats,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * vla_scan_backward: gradients of the scan with the ADDITIVE update.
 *
 * Source: "Variational Linear Attention (VLA)" README, v3 notes item 2 (the
 * scan keeps full gradient flow) and "Running the Sub-Tests" (gradient
 * checks); "Mathematical Primitives" section 5 (a stable backward pass).  The
 * pages give only the forward recurrence of vla_scan_forward; this call
 * returns its exact derivative (up to float32 rounding) for the loss
 *   L = sum_t <g_o[t], o_t> + <g_AT, A_T> + <g_ST, S_T> + <g_nT, n_T>
 * with respect to q, k, v, u, A0, S0 and n0, at the same parameters.  The
 * derivative follows the forward's branches: a rank-1 step the guard skipped
 * passes no gradient to its direction, and the cap contributes only on the
 * tokens where it fired.
 *
 *   p        as for vla_scan_forward; supported: d in {16, 32, 64}, r 1..4,
 *            f32 or bf16 storage, update = ADDITIVE, contiguous inputs (all
 *            strides 0); the schedule field is ignored (one workgroup per
 *            chain runs the forward again with a tape, then the reverse)
 *   q..n0    the forward's inputs (A0, S0, n0 nullable: I, 0, 0)
 *   g_o      [B, H, T, d] float32 (may be NULL only when T = 0)
 *   g_AT, g_ST [B, H, d, d], g_nT [B, H, d] float32, each nullable (zero)
 *   g_q, g_k, g_v [B, H, T, d], g_u [B, H, T, r, d], g_A0, g_S0 [B, H, d, d],
 *   g_n0 [B, H, d]: float32 gradients (written; all non-NULL, none may
 *            overlap an input or another output)
 *   workspace at least vla_scan_backward_workspace_size() bytes, 256-byte
 *            aligned: the tape (per token the r rank-1 steps' z and delta,
 *            alpha_hat, |alpha|, the cap scale) and A, S, n every 32 tokens
 * Errors as for vla_scan_forward: VLA_EUNSUPPORTED outside the supported set.
 */
vla_status_t vla_scan_backward_workspace_size(const vla_scan_params_t* p, size_t* bytes);
vla_status_t vla_scan_backward(const vla_scan_params_t* p,
                               const void* q, const void* k, const void* v, const void* u,
                               const float* A0, const float* S0, const float* n0,
                               const float* g_o, const float* g_AT, const float* g_ST, const float* g_nT,
                               float* g_q, float* g_k, float* g_v, float* g_u,
                               float* g_A0, float* g_S0, float* g_n0,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * vla_scan_forward_noalloc: vla_scan_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It takes no workspace argument: the
 * scratch that vla_scan_forward would take from its workspace (the chunked
 * schedule's buffers, the gather of strided inputs, the validation flag)
 * comes from a static device array of VLA_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device it runs on until the process ends.  Its
 * device address is looked up once per device, on the first call with that
 * device current.
 *
 * Arguments, layouts, results and errors are those of vla_scan_forward.  A
 * call whose vla_scan_workspace_size() exceeds VLA_NOALLOC_SCRATCH_BYTES is
 * refused with VLA_EWORKSPACE before anything is launched (e.g. the chunked
 * schedule on 16 chains of 65536 tokens, about 1.2 GB); the caller can then
 * use vla_scan_forward with its own workspace.  The call allocates nothing
 * (no hipMalloc or hipFree, no allocating library routine).  Every call on a
 * device shares that device's array, and each call overwrites what the last
 * one left there (the kernels initialise whatever they read back): calls that
 * overlap in time on one device, on different streams or from different
 * threads, race on it and must be serialised by the caller.
 */
#define VLA_NOALLOC_SCRATCH_BYTES (256ull << 20)
vla_status_t vla_scan_forward_noalloc(const vla_scan_params_t* p,
                                      const void* q, const void* k, const void* v, const void* u,
                                      const float* A0, const float* S0, const float* n0,
                                      void* o, float* A_T, float* S_T, float* n_T, int32_t* stats,
                                      void* stream);

/*
 * vla_project_u: learned penalty directions, u_{row, i} = normalize(W_u[i] k_raw[row]).
 *
 * Source: "Variational Linear Attention (VLA)" README, v3 notes item 2
 * (u_t = normalize(W_u k_t^raw)).  normalize(x) = x / max(|x|_2, 1e-12).
 *
 *   rows      number of key rows (e.g. B*H*T), >= 0
 *   d         head dimension (16, 32, 64 or 128); r directions (1..4)
 *   in_dtype  storage of W_u and k_raw; out_dtype storage of u
 *   W_u       [r, d, d] device pointer, row-major; applied as W_u[i] @ k_raw
 *   k_raw     [rows, d] device pointer
 *   u         [rows, r, d] device pointer (written)
 * Products accumulate in float32 on the matrix cores; the norm, the scale and
 * the final cast are float32.
 */
vla_status_t vla_project_u(int64_t rows, int32_t d, int32_t r, int32_t in_dtype,
                           int32_t out_dtype, const void* W_u, const void* k_raw,
                           void* u, void* stream);

/*
 * Measurement hook for the dominant kernel: the state-chain kernel of the
 * chunked schedule (the sequential S/cap recursion, one workgroup per chain).
 * Not part of the method; it serves benchmarks that must time that kernel on
 * the stream it runs on.
 *
 * vla_timing_enable(1) creates VLA_TIMING_SLOTS pairs of HIP events on the
 * device current at that moment and makes each following vla_scan_forward
 * that runs the chunked schedule record one pair on its stream, immediately
 * before and after each launch of that kernel (one per segment), until the
 * slots are used up (later launches are not recorded).  vla_timing_enable(0) stops recording and releases the
 * events.  vla_timing_collect waits for the recorded events, writes up to
 * `cap` durations in milliseconds to `ms` (oldest first), stores how many it
 * wrote in *n and clears the record; recording continues if enabled.
 *
 * Errors: VLA_EINVAL for a NULL `ms` or `n` or a negative `cap`; VLA_EHIP if
 * an event call fails.  The calls take a process-wide lock.
 */
#define VLA_TIMING_SLOTS 256
vla_status_t vla_timing_enable(int32_t enable);
vla_status_t vla_timing_collect(float* ms, int32_t cap, int32_t* n);

/* Static string naming a status code. */
const char* vla_status_string(vla_status_t s);

/* Thread-local detail of the last failed call on this thread ("" if none). */
const char* vla_last_error(void);

/* VLA_ABI_VERSION of the built library. */
int vla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VLA_H_ */
