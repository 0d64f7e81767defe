/*
 * fibattn.h - C ABI of libfibattn.so: depth-staggered Fibonacci-offset sparse self-attention,
 * forward and backward, on AMD Instinct MI355X (gfx950).
 *
 * The operation is defined in "Depth-Staggered Fibonacci Spacing for Sparse Attention: Static
 * Schedules Beat Learned Dilation and Extrapolate Where Dense Attention Fails" (C. A. Capps,
 * arXiv 2606.28560). Section references below are to that paper.
 *
 * What is computed (§2 "Attended set"). Query i of head h attends to
 *   - the dense causal window of distances {0, 1, ..., W} (self included), and
 *   - one slot per base rung f_k at distance d_k = alpha * f_k, read by linear interpolation:
 *       key = (1 - t) * krot[i - a] + t * krot[i - a - 1],  a = floor(d_k),  t = d_k - a,
 *     and likewise for the value row (values are not rotated).
 * q and k are rotated by RoPE at their own (integer) positions before the gather, with
 * half-split pairs (j, j + D/2) and frequency rope_theta^(-2j/D). Scores are scaled by 1/sqrt(D),
 * softmax runs over the valid slots, and query head h reads key-value head h / (Hq / Hkv) (GQA,
 * §3 "Models and training").
 *
 * Slot rules where the paper leaves the detail open (the offset plan, fibattn_plan):
 *   - d_k is computed in double; if |d_k - rint(d_k)| <= 1e-9 it is snapped to rint(d_k);
 *   - an integral d_k <= W is DUP: dropped, the window already holds that distance;
 *   - an integral d_k > W is INT: row i - d_k, valid for i >= d_k;
 *   - otherwise INTERP: valid for i >= floor(d_k) + 1 (the farther row exists).
 * The kernels never read a row before 0 or at or beyond L.
 *
 * Layout: every tensor is contiguous [B, H, L, D] (H = Hq for q, o, do, dq; Hkv for k, v, dk,
 * dv). lse is [B, Hq, L] float32 (natural log). D must be 64.
 * Storage types: FIBATTN_F32 (float32 everywhere) or FIBATTN_BF16 (bfloat16 q, k, v, o, do, dq,
 * dk, dv; dot products take fp16-rounded operands - rotated q and k, values, softmax weights,
 * do - with float32 accumulation, and the softmax, its gradient and every reduction run in
 * float32; decode computes in float32 throughout). Every finite bf16 input is accepted: rows
 * that fp16 does not hold well as they are (an element of 2^15 or more, or a nonzero row whose
 * largest element is below 2^-10) are either carried scaled by a power of two, which the kernels
 * undo exactly in float32 (q, do and the backward's hand-off of dS), or, for keys and values,
 * make every tile that reads them compute in float32 from the caller's bf16 rows.
 *
 * Ownership and execution. All buffers belong to the caller. Device pointers must stay valid
 * until the stream reaches the work. `offsets` is a host array, read during the call and not
 * kept. The library keeps no allocation and no state between calls (except the device array of
 * the allocation-free forward, fibattn_fwd_noalloc); calls are asynchronous on `stream` (a
 * hipStream_t; NULL is the null stream) and are re-entrant. Outputs are overwritten, never
 * accumulated.
 *
 * Errors. Arguments are checked on the host before anything is launched; on error no work is
 * queued and an error status is returned. fibattn_last_error() gives the calling thread's last
 * error text. Nothing aborts or throws across this boundary.
 */
#ifndef FIBATTN_H
#define FIBATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FIBATTN_OK = 0,
    FIBATTN_ERR_INVALID = 1,      /* an argument is out of its domain */
    FIBATTN_ERR_UNSUPPORTED = 2,  /* valid, but not implemented here (e.g. D != 64, W > 31) */
    FIBATTN_ERR_WORKSPACE = 3,    /* workspace pointer missing or smaller than required */
    FIBATTN_ERR_HIP = 4           /* a HIP call or kernel launch failed */
} fibattn_status_t;

typedef enum { FIBATTN_F32 = 0, FIBATTN_BF16 = 1 } fibattn_dtype_t;

typedef enum { FIBATTN_DUP = 0, FIBATTN_INT = 1, FIBATTN_INTERP = 2 } fibattn_offset_kind_t;

typedef enum { FIBATTN_BASE_FIB = 0, FIBATTN_BASE_POW2 = 1 } fibattn_base_t;

typedef enum {
    FIBATTN_SCHEDULE_FIXED = 0,
    FIBATTN_SCHEDULE_LINEAR = 1,
    FIBATTN_SCHEDULE_COPRIME = 2
} fibattn_schedule_t;

/* Largest window W and number of base rungs K the kernels take. */
#define FIBATTN_MAX_W 31
#define FIBATTN_MAX_K 32

/* Text of a status code (static storage). */
const char* fibattn_status_string(fibattn_status_t status);

/* The calling thread's last error message ("" if none). Valid until the thread's next call. */
const char* fibattn_last_error(void);

/*
 * Base rungs (§2 "Attended set" for the Fibonacci list 1, 2, 3, 5, ..., 987, K = 15; §2 "Control
 * base" for the power-of-two control 1, 2, 4, ..., up to pow2_max inclusive).
 * out: host int32[capacity]; *count receives K. pow2_max is ignored for the Fibonacci base.
 * Errors: INVALID for a NULL pointer, an unknown base, pow2_max < 1, or capacity < K.
 */
fibattn_status_t fibattn_base_offsets(int32_t base, int32_t pow2_max, int32_t* out,
                                      int32_t capacity, int32_t* count);

/*
 * Per-layer alpha of a static schedule (§2 "Per-layer scalar"): fixed 1; linear
 * 0.5 + layer / (n_layers - 1); coprime: the linear value of layer (7 * layer mod n_layers).
 * Errors: INVALID for NULL alpha, an unknown schedule, n_layers < 2, layer outside
 * [0, n_layers), or (coprime) n_layers sharing a factor with 7.
 */
fibattn_status_t fibattn_alpha_schedule(int32_t schedule, int32_t layer, int32_t n_layers,
                                        double* alpha);

/*
 * Learned schedule (§2 "Per-layer scalar"): alpha = 0.5 + sigmoid(theta), and the factor
 * dalpha/dtheta = sigmoid(theta) (1 - sigmoid(theta)) that turns d(alpha) into d(theta).
 * Either output may be NULL. Errors: INVALID for a non-finite theta.
 */
fibattn_status_t fibattn_alpha_from_theta(double theta, double* alpha, double* dalpha_dtheta);

/*
 * Rounded-integer stagger (§2 "Implementation note": the fixed and staggered variants have integer
 * offsets and can run on the integer path, numerically the same as a boolean-mask attention):
 * d_k = alpha * offsets[k] rounded to the nearest integer, ties to even, after snapping 2 d_k to an
 * integer within 1e-9 (so that a ramp value such as 0.5 + 5/15 times 3 is the tie 2.5). Writes the
 * distinct d_k >= 1, increasing, to out (host, capacity entries) and their number to count; pass
 * them as the offsets of fibattn_fwd / fibattn_bwd with alpha = 1 (d(alpha) is then UNSUPPORTED:
 * the offsets are integral). Errors: INVALID for NULL pointers, bad alpha or offsets (as
 * fibattn_plan) or a capacity below the count; UNSUPPORTED if some alpha * f_k exceeds 2^30.
 */
fibattn_status_t fibattn_round_offsets(double alpha, const int32_t* offsets, int32_t K, int32_t* out,
                                       int32_t capacity, int32_t* count);

/*
 * Offset plan: the slot table the kernels use, host-only and GPU-free (§2 "Attended set").
 * For each rung k: kind_out[k] (fibattn_offset_kind_t), floor_out[k] = a, t_out[k] = t rounded
 * to float32 (0 for INT and DUP), reach_out[k] = first query index at which the slot is valid.
 * All outputs are host arrays of K entries. Errors: INVALID for NULL pointers (when K > 0),
 * K outside [0, 32], W < 0, a non-finite or non-positive alpha, or offsets not strictly
 * increasing from >= 1; UNSUPPORTED if some alpha * f_k exceeds 2^30.
 */
fibattn_status_t fibattn_plan(double alpha, int32_t W, const int32_t* offsets, int32_t K,
                              uint8_t* kind_out, int32_t* floor_out, float* t_out,
                              int32_t* reach_out);

/* Bytes of device workspace fibattn_fwd needs (staged rotated keys and values). */
size_t fibattn_fwd_workspace_bytes(int32_t B, int32_t L, int32_t Hkv, int32_t D, int32_t dtype);

/*
 * Forward pass (§2 "Attended set", "Implementation note"; shapes §3 "Models and training").
 * q: device [B, Hq, L, D]; k, v: device [B, Hkv, L, D]; all of storage type `dtype`.
 * o: device [B, Hq, L, D] of `dtype` (written). lse: device float32 [B, Hq, L] (written) or
 * NULL when no backward pass will follow.
 * workspace: device, >= fibattn_fwd_workspace_bytes(...) bytes, scratch for this call only.
 * Queues two kernels on `stream`: fibattn_fwd_prep, then fibattn_fwd_attend.
 * Arithmetic: float32 for FIBATTN_F32. For FIBATTN_BF16, rotated keys and values are staged as
 * fp16, and the matrix-core kernels also round the rotated q and the softmax weights to fp16 for
 * their products (each operand within 2^-11 relative); products accumulate in float32, and the
 * interpolation weight t is applied in float32 (to scores and weights on the matrix cores, to
 * the staged rows in the general kernels). The prep flags blocks of key and value rows that
 * fp16 does not hold well (see Storage types above); a tile that reads a flagged row, or whose
 * own q row (times 1/sqrt(D)) lies outside fp16's range, is computed in float32 from the
 * caller's bf16 rows instead, so any finite input is handled.
 * Errors: INVALID (NULL pointers, B/L/Hq/Hkv < 1, Hq % Hkv != 0, W < 0, K outside [0, 32],
 * bad alpha, bad offsets, unknown dtype, rope_theta not finite and > 0), UNSUPPORTED (D != 64,
 * W > 31, L > 2^20), WORKSPACE, HIP.
 */
fibattn_status_t fibattn_fwd(const void* q, const void* k, const void* v, double alpha,
                             int32_t W, const int32_t* offsets, int32_t K, int32_t B, int32_t L,
                             int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype, double rope_theta,
                             void* o, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * First stage of fibattn_fwd, exposed so that each kernel can be timed on its own: rotate every
 * key row at its position once (RoPE before the gather, §2 "Attended set") into the workspace.
 * For FIBATTN_F32 the rotated keys are stored as float32; for FIBATTN_BF16 the rotated keys and
 * the values are stored as fp16 rows (bf16 values of magnitude below 65504 convert exactly), with
 * the cos/sin table of every position and one range flag per block of 32 positions of 4 (batch,
 * head) rows (nonzero where a key or value row there lies outside what fp16 holds well: an
 * element of 2^15 or more, or a nonzero row maximum below 2^-10). The backward's FIBATTN_STAGE_PREP writes the same arrays
 * at the same places of its (larger) workspace where fibattn_bwd_reuses_fwd_prep says so.
 * k, v: device [B, Hkv, L, D] of `dtype`. Errors as fibattn_fwd.
 */
fibattn_status_t fibattn_fwd_prep(const void* k, const void* v, int32_t B, int32_t L, int32_t Hkv,
                                  int32_t D, int32_t dtype, double rope_theta, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Second stage of fibattn_fwd: the attention itself. Reads what fibattn_fwd_prep left in
 * `workspace` (same shapes, dtype and rope_theta), so it must follow it on the same stream with the
 * workspace untouched in between. q, k, v are the caller's tensors as fibattn_fwd takes them: for
 * FIBATTN_F32, v is read directly (the rotated keys come from the workspace); for FIBATTN_BF16, the
 * staged fp16 keys and values are read, and the caller's k and v only by tiles whose rows the prep
 * found outside fp16's range (see fibattn_fwd), which are computed in float32 from them.
 */
fibattn_status_t fibattn_fwd_attend(const void* q, const void* k, const void* v, double alpha, int32_t W,
                                    const int32_t* offsets, int32_t K, int32_t B, int32_t L,
                                    int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                                    double rope_theta, void* o, float* lse,
                                    const void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid allocation): fibattn_fwd with its workspace in a
 * device array the library holds instead of one the caller passes. The array is
 * fibattn_fwd_noalloc_max_bytes() bytes (32 MiB); each GPU the library runs on holds its own copy
 * until the process ends. Arguments, outputs and errors as fibattn_fwd; WORKSPACE (nothing queued)
 * when the call needs more than the array holds, i.e. fibattn_fwd_workspace_bytes(B, L, Hkv, D,
 * dtype) > fibattn_fwd_noalloc_max_bytes(). The call allocates and frees no device memory.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents (nothing in it
 * needs to start at zero: the prep writes every row the attention reads): calls that overlap on one
 * GPU (other streams, other threads) race, and the caller must order them. Call it with the
 * stream's device current.
 */
fibattn_status_t fibattn_fwd_noalloc(const void* q, const void* k, const void* v, double alpha, int32_t W,
                                     const int32_t* offsets, int32_t K, int32_t B, int32_t L, int32_t Hq,
                                     int32_t Hkv, int32_t D, int32_t dtype, double rope_theta, void* o,
                                     float* lse, void* stream);

/* Bytes of the allocation-free forward's device array (per GPU). */
size_t fibattn_fwd_noalloc_max_bytes(void);

/*
 * Single-token decode (inference with a cache): for each sequence b, its new query at position
 * positions[b] attends to the window and offset slots of that position (§2 "Attended set"; integer
 * offsets read one row, §2 "Implementation note"). The output is the forward pass's output row at
 * that position for the sequence held in the cache.
 * q: device [B, Hq, D] of `dtype`, the new queries (unrotated). k_cache, v_cache: device
 * [B, Hkv, Lmax, D] of `dtype`, keys unrotated (as fibattn_fwd takes them); rows 0..positions[b]
 * of sequence b are read, the new token's own key and value included (write them before the call).
 * positions: device int32 [B]. o: device [B, Hq, D] of `dtype` (written); lse: device float32
 * [B, Hq] (natural log, written) or NULL. No workspace. Arithmetic is float32 for both storage
 * types (keys rotated at their own positions as they are read).
 * A position outside [0, Lmax) is not read from: that sequence's outputs are NaN.
 * Errors: as fibattn_fwd, with Lmax in place of L.
 */
fibattn_status_t fibattn_decode(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* positions, double alpha, int32_t W,
                                const int32_t* offsets, int32_t K, int32_t B, int32_t Lmax,
                                int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                                double rope_theta, void* o, float* lse, void* stream);

/* Bytes of device workspace fibattn_bwd needs. */
size_t fibattn_bwd_workspace_bytes(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D,
                                   int32_t W, int32_t K, int32_t dtype);

/*
 * Backward pass: gradients of sum(do * o) for the forward above (§2 "Attended set": the
 * interpolation keeps a gradient to alpha; §2 "Per-layer scalar": alpha = 0.5 + sigmoid(theta)).
 * Inputs: q, k, v, dout = do, all device, same shapes and storage type as the forward.
 * o and lse (the forward's outputs) are accepted for the usual attention backward signature but
 * are not read and may be NULL: the backward recomputes every score and the log-sum-exp in
 * float32, and forms the row term delta = do . o as sum_s p_s (do . val_s), which keeps the
 * rounding of the forward's outputs (and the forward's fp16 products for bf16 storage) out of
 * the gradients.
 * Outputs (device, overwritten): dq [B, Hq, L, D], dk, dv [B, Hkv, L, D] of `dtype`;
 * dalpha float32[1] or NULL; dtheta float32[1] or NULL, set to dalpha * dalpha_dtheta (pass the
 * factor from fibattn_alpha_from_theta for the learned schedule).
 * d(alpha) takes the slope of each interpolated read in alpha; integral offsets (INT, DUP)
 * contribute nothing, so when dalpha or dtheta is requested and some rung is integral the call
 * returns UNSUPPORTED.
 * workspace: device, >= fibattn_bwd_workspace_bytes(...) bytes.
 * Errors: as fibattn_fwd, plus UNSUPPORTED as above.
 */
fibattn_status_t fibattn_bwd(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, double alpha, int32_t W,
                             const int32_t* offsets, int32_t K, int32_t B, int32_t L, int32_t Hq,
                             int32_t Hkv, int32_t D, int32_t dtype, double rope_theta,
                             double dalpha_dtheta, void* dq, void* dk, void* dv, float* dalpha,
                             float* dtheta, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Stages of the backward pass, for fibattn_bwd_stages (bit mask). */
typedef enum {
    FIBATTN_STAGE_PREP = 1,   /* keys rotated at their positions (and fp16 values) into the workspace;
                                 the same arrays as fibattn_fwd_prep where
                                 fibattn_bwd_reuses_fwd_prep returns 1 */
    FIBATTN_STAGE_QUERY = 2,  /* dq, plus what the key stage reads from the workspace */
    FIBATTN_STAGE_KEY = 4,    /* dk, dv, and dalpha / dtheta when requested */
    FIBATTN_STAGE_ALL = 7
} fibattn_bwd_stage_t;

/*
 * fibattn_bwd split into its stages, so that each kernel can be timed (or overlapped) on its own.
 * stages: a nonzero mask of fibattn_bwd_stage_t bits; the selected stages are queued in the order
 * PREP, QUERY, KEY. A stage reads what the earlier stages left in `workspace`: a call with a subset
 * of the bits must follow the calls that ran the earlier stages, on the same stream, with the same
 * arguments and the workspace untouched in between. dq is written by the QUERY stage, dk, dv,
 * dalpha and dtheta by the KEY stage; pointers a selected stage does not write are not read.
 * FIBATTN_STAGE_ALL is fibattn_bwd (which forwards here). Arguments and errors as fibattn_bwd,
 * plus INVALID for a mask outside [1, 7]; every argument is checked whatever the mask.
 * A training step can leave out PREP where fibattn_bwd_reuses_fwd_prep returns 1 and the
 * backward's workspace is the one the forward (fibattn_fwd or fibattn_fwd_prep) ran with, on the
 * same k, v, shapes, dtype and rope_theta, untouched since: that workspace then already holds what
 * PREP would write.
 */
/*
 * 1 when the backward's FIBATTN_STAGE_PREP writes exactly what fibattn_fwd_prep writes for the same
 * k, v, shapes, dtype and rope_theta (the forward's arrays are a prefix of the backward's
 * workspace), so that a training step may prep once per layer; 0 otherwise (bfloat16 shapes that
 * the backward serves with its general kernels, which rotate float32 keys of their own) and for
 * arguments fibattn_bwd would reject. Host-only: it queues nothing and reads no device memory.
 */
int32_t fibattn_bwd_reuses_fwd_prep(double alpha, int32_t W, const int32_t* offsets, int32_t K,
                                    int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t dtype);

fibattn_status_t fibattn_bwd_stages(int32_t stages, const void* q, const void* k, const void* v,
                                    const void* dout, double alpha, int32_t W,
                                    const int32_t* offsets, int32_t K, int32_t B, int32_t L,
                                    int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                                    double rope_theta, double dalpha_dtheta, void* dq, void* dk,
                                    void* dv, float* dalpha, float* dtheta, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Phase trace of the bfloat16 forward attention kernel, for measurement only (no passage of the
 * pages: it times the kernel that does §2 "Attended set" for bf16 storage). The library built with
 * FIBATTN_PHASE_TRACE (libfibattn_trace.so) records, per workgroup of the kernel's last launch,
 * eight 64-bit words: six stamps of the GPU's 100 MHz real-time counter (start; key near block
 * landed; key pass done; value near block landed; value pass done; outputs stored), then
 * tile | steps << 16 | near steps << 24 | kept rungs reached << 32, and the CU. Records of
 * workgroups 65536 and up are not kept. fibattn_phase_trace_read copies the first n_wg records
 * (0 <= n_wg <= 65536) to out (host, 8 n_wg words), a synchronous copy on the null stream: call it
 * after the traced launch has finished. INVALID for a null out or n_wg out of range, HIP when the
 * copy fails. Every other build returns UNSUPPORTED and touches nothing. */
fibattn_status_t fibattn_phase_trace_read(uint64_t* out, int32_t n_wg);

#ifdef __cplusplus
}
#endif

#endif /* FIBATTN_H */
