/*
 * mlstm.h -- C ABI of the MI355X (gfx950) stabilized parallel mLSTM forward pass.
 *
 * The operation is the stabilized parallel forward pass of the mLSTM cell of
 * "xLSTM: Extended Long Short-Term Memory", Appendix A.3: the parallel form
 * ("Parallel mLSTM Forward Pass", Eqs. 71-77) in the stabilized version that
 * opens "Parallel mLSTM Backward Pass" (Eqs. 79-86), with the log forget gate
 * matrix of Eq. 101.  For one head with queries, keys, values Q, K, V (T x d)
 * and gate pre-activations f~, i~ (length T):
 *
 *   fbar_k   = log sigmoid(f~_k)                                   (Eq. 101)
 *   D~_ij    = sum_{k=j+1..i} fbar_k + i~_j  for j <= i, -inf above (Eqs. 79, 101, 72)
 *   m_i      = max_j D~_ij                                         (Eq. 80)
 *   D'_ij    = exp(D~_ij - m_i)                                    (Eq. 81)
 *   C~'_ij   = (q_i . k_j / sqrt(d)) D'_ij                          (Eq. 82)
 *   b_i      = sum_j C~'_ij                                        (Eq. 83)
 *   n_i      = max(|b_i|, exp(-m_i))                               (Eq. 84)
 *   h~_i     = sum_j C~'_ij v_j / n_i                              (Eqs. 85, 86)
 *
 * Heads are independent (the xLSTM cell has no memory mixing across heads),
 * so every call processes B x NH heads at once.
 *
 * Layouts (all row-major, contiguous, no strides):
 *   q, k, v, h_out  [B][NH][T][d]   element type given by `dtype`
 *   igate, fgate    [B][NH][T]      float32 (i~ and f~ pre-activations)
 *   m_out, n_out    [B][NH][T]      float32
 * k is passed UNSCALED: the library applies the 1/sqrt(d) of Eq. 82.
 *
 * Ownership: every pointer is device memory owned by the caller, on the
 * device that is current when the call is made.  The library never frees or
 * retains a caller pointer beyond the work it enqueues.  Outputs are fully
 * overwritten.  No output may overlap an input or another output (checked
 * from the pointers and sizes: MLSTM_ERR_ALIAS, nothing launched); inputs
 * may overlap each other.  The recurrent step alone may update C in place.
 *
 * Ordering: calls are asynchronous on the given HIP stream (NULL = the null
 * stream); results are valid once that stream has synchronized.  No host
 * synchronization happens inside the library.
 *
 * Errors: every argument check runs before any device work; on error nothing
 * is launched, no output is touched, and a negative status is returned.
 * Faults inside a kernel surface at the caller's next synchronization, as for
 * any stream API.  No C++ exception crosses this interface.
 *
 * Numerics: gates, m and n are float32.  For MLSTM_BF16 the two contractions
 * run on bf16 matrix cores with float32 accumulation; the row sums b are taken
 * from the float32 C~' before it is rounded to bf16; h_out is rounded to
 * nearest even.  Inputs must be finite; NaN/Inf propagate and are not checked.
 * Results are bitwise reproducible run to run (fixed reduction order, no
 * atomics).
 */
#ifndef MLSTM_H
#define MLSTM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of q, k, v, h_out */
enum { MLSTM_FP32 = 0, MLSTM_BF16 = 1 };

/* tile-kernel selector for mlstm_causal_tiles */
enum {
  MLSTM_KERNEL_AUTO = 0,   /* bf16 -> matrix-core kernel; fp32 -> float32 matrix-core kernel
                              (d a multiple of 32 up to 256, or 320, 384, 512), else vector kernel */
  MLSTM_KERNEL_MFMA = 1,   /* bf16 only: bf16 MFMA tiles (the production path) */
  MLSTM_KERNEL_VECTOR = 2, /* any dtype: float32 vector-ALU tiles, no bf16 rounding of C~' */
  MLSTM_KERNEL_MFMA_ALL_TILES = 3, /* as MLSTM_KERNEL_MFMA, but visiting every causal tile */
  MLSTM_KERNEL_MFMA_SINGLE = 4,    /* bf16 only, d <= 512: the one-wave-per-SIMD MFMA kernel */
  MLSTM_KERNEL_MFMA_WIDE = 5       /* bf16 only: the wide-head MFMA kernel, for any d */
};
/*
 * The bf16 MFMA path has three tile kernels, and a fourth on the one-launch
 * path.  For d <= 384 it runs 8 waves
 * per workgroup, two per SIMD: the two waves that share a SIMD share 32 query
 * rows, each forms C~' for its own 32 of every 64 keys and accumulates half
 * of the output columns, so one wave's copies and exponentials overlap the
 * other's matrix-core work.  On the one-launch path with d a multiple of 64
 * up to 192 it runs 4 waves, one per SIMD, each with 32 query rows and all
 * columns, and software-pipelines the key loop (the Q K^T product of one key
 * tile beside the C~' V product of the previous one, K and V staged through
 * registers); its sums are those of the one-wave kernel below.  For 384 < d <= 512 (and with
 * MLSTM_KERNEL_MFMA_SINGLE) it runs 4 waves, one per SIMD, each with 32 query
 * rows and all columns.  For d > 512 (and with MLSTM_KERNEL_MFMA_WIDE) four
 * waves share 32 query rows, each holding a quarter of the head dimension:
 * they add their partial Q K^T products through LDS, and each accumulates a
 * quarter of the output columns.  All give the same results up to float32
 * summation order.  Float32 inputs (MLSTM_KERNEL_AUTO) run on the float32
 * matrix instruction v_mfma_f32_32x32x2_f32: 4 waves, one per SIMD, each with
 * 32 query rows and their Q^T operands in registers, C~' kept in float32 and
 * fed from the first product's registers to the second; above d = 256 two
 * (at d = 512 four) workgroups per 128 query rows split the output columns.  Other
 * float32 head dimensions, and MLSTM_KERNEL_VECTOR, run the float32 vector
 * kernel.
 */
/*
 * Decay-aware tile skipping (MLSTM_KERNEL_AUTO and _MFMA on bf16).  From the
 * gate scan's terms the tile kernel bounds log2(D'_ij / sqrt(d)) over each
 * 32 x 32 block of Eqs. 79-81; where the bound is below -200 every entry's
 * float32 exponential is exactly 0, so the block adds nothing to b (Eq. 83)
 * or to C~'V and is not visited.  Outputs equal those of
 * MLSTM_KERNEL_MFMA_ALL_TILES (up to the sign of exact zeros).  Long
 * sequences with strong forgetting skip most of the causal triangle; the
 * counted work (2 T^2 d per head) is unchanged.
 */

/* status codes */
enum {
  MLSTM_OK = 0,
  MLSTM_ERR_NULL = -1,        /* a required pointer is NULL */
  MLSTM_ERR_SHAPE = -2,       /* B, NH, T or d < 1, or a size overflows */
  MLSTM_ERR_DTYPE = -3,       /* dtype not MLSTM_FP32 / MLSTM_BF16 */
  MLSTM_ERR_HEAD_DIM = -4,    /* d not a multiple of 16 in [16, 1024], or beyond a kernel's limit */
  MLSTM_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
  MLSTM_ERR_HIP = -6,         /* a HIP allocation or launch failed */
  MLSTM_ERR_WORKSPACE = -7,   /* caller workspace smaller than mlstm_workspace_bytes */
  MLSTM_ERR_KERNEL = -8,      /* unknown kernel selector, or an MFMA selector for fp32 */
  MLSTM_ERR_ALIAS = -9,       /* an output overlaps an input or another output */
  MLSTM_ERR_ACTIVATION = -10, /* unknown forget-gate activation */
  MLSTM_ERR_SCRATCH = -11     /* beyond the allocation-free entry point's fixed workspace */
};

/*
 * Forget-gate activation (the `forget_activation` argument of
 * mlstm_gate_scan, mlstm_parallel_fwd_train, mlstm_parallel_bwd and
 * mlstm_recurrent_step).  The mLSTM forward equations (Eq. 71) allow the
 * forget gate to be either sigma(f~) or exp(f~); every formula of the
 * parallel and recurrent forms uses it only through its logarithm
 * fbar = log f, which is log sigma(f~) or f~ itself.  With MLSTM_FORGET_EXP
 * the caller keeps f~ <= 0 if it wants f <= 1; nothing here requires it.
 * mlstm_parallel_fwd, _stream and _gated use MLSTM_FORGET_SIGMOID.
 */
enum { MLSTM_FORGET_SIGMOID = 0, MLSTM_FORGET_EXP = 1 };

/*
 * mlstm_parallel_fwd -- the whole forward pass (Eqs. 79-86) for B x NH heads.
 *   q, k, v   in   [B][NH][T][d], dtype
 *   igate     in   [B][NH][T] float32, i~ (input gate pre-activations, Eq. 72)
 *   fgate     in   [B][NH][T] float32, f~ (forget gate pre-activations, Eq. 71;
 *                  sigmoid forget activation; f~ at t = 0 never affects a result)
 *   h_out     out  [B][NH][T][d], dtype: h~ (Eq. 86), before any output gate
 *   m_out     out  [B][NH][T] float32: the row maximum m (Eq. 80)
 *   n_out     out  [B][NH][T] float32: the normalizer n (Eq. 84)
 *   B, NH, T  >= 1;  d a multiple of 16 in [16, 1024]
 *   dtype     MLSTM_FP32 or MLSTM_BF16
 * Runs on the null stream.  For bf16 with d <= 512 and T <= 2048, T a
 * multiple of 4, the pass is one kernel launch that needs no workspace: each
 * workgroup scans its head's gates itself (the gate-scan arithmetic in the
 * same order, so every output is bitwise that of the two stages with the same
 * tile arithmetic: the one-wave kernel where the pipelined kernel runs, the
 * kernel MLSTM_KERNEL_AUTO picks otherwise).  So is the pass for float32
 * inputs with T <= 2048: the float32 tile kernel (matrix-core where it takes
 * d, vector otherwise) scans its head's gates itself, bitwise as its two
 * stages would.  Otherwise the gate scan and the tile kernel run as two
 * launches on a library-allocated, stream-ordered workspace.
 * Returns MLSTM_OK or a negative status.
 */
int mlstm_parallel_fwd(const void* q, const void* k, const void* v,
                       const float* igate, const float* fgate,
                       void* h_out, float* m_out, float* n_out,
                       int64_t B, int64_t NH, int64_t T, int64_t d, int dtype);

/* As mlstm_parallel_fwd, enqueued on `stream` (a hipStream_t; NULL = null stream). */
int mlstm_parallel_fwd_stream(const void* q, const void* k, const void* v,
                              const float* igate, const float* fgate,
                              void* h_out, float* m_out, float* n_out,
                              int64_t B, int64_t NH, int64_t T, int64_t d, int dtype,
                              void* stream);

/*
 * mlstm_parallel_fwd_noalloc -- mlstm_parallel_fwd_stream for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It calls no allocating routine.
 * Its workspace is a fixed array of MLSTM_NOALLOC_SCRATCH_BYTES in the
 * library's device code, one per GPU, held until the process ends; a call
 * needs mlstm_workspace_bytes(B, NH, T) of it (about 20.5 bytes per position
 * of B * NH * T, T padded to a multiple of 128: up to ~800 K positions) and
 * returns MLSTM_ERR_SCRATCH, before any device work, for a problem that needs
 * more.  Where mlstm_parallel_fwd runs as a single launch (bf16, d <= 512,
 * T <= 2048, T a multiple of 4; float32, T <= 2048) no workspace is used
 * and any size is accepted.  All calls on one GPU share that GPU's array:
 * calls that overlap in time on one GPU (different streams, host threads)
 * race and must be serialized by the caller.  Nothing needs to be cleared between calls: each
 * call writes every workspace byte it reads.  Arguments, results and other
 * errors as for mlstm_parallel_fwd_stream; the first call on a device also
 * looks up the array's address on that device (MLSTM_ERR_HIP if that fails).
 */
enum { MLSTM_NOALLOC_SCRATCH_BYTES = 16 << 20 };
int mlstm_parallel_fwd_noalloc(const void* q, const void* k, const void* v,
                               const float* igate, const float* fgate,
                               void* h_out, float* m_out, float* n_out,
                               int64_t B, int64_t NH, int64_t T, int64_t d, int dtype,
                               void* stream);

/*
 * mlstm_parallel_fwd_gated -- the forward pass followed by the output gate of
 * "Parallel mLSTM Forward Pass" (Eq. 78): H = sigma(O~) (.) H~, elementwise,
 * with the logistic sigmoid.  The gate is applied to the float32 h~ inside
 * the tile kernel's epilogue, before the result is rounded to `dtype`.
 *   ogate       in   [B][NH][T][d], dtype: O~ (output gate pre-activations); required
 *   h_out       out  [B][NH][T][d], dtype: H (Eq. 78)
 *   htilde_out  out  [B][NH][T][d], dtype: H~ (Eq. 86), bitwise what
 *                    mlstm_parallel_fwd writes to its h_out; may be NULL (not stored)
 *   all other arguments as for mlstm_parallel_fwd_stream.
 * ogate and htilde_out must be 16-byte aligned and must not alias any other
 * argument.  Errors as for mlstm_parallel_fwd (MLSTM_ERR_NULL for ogate NULL).
 */
int mlstm_parallel_fwd_gated(const void* q, const void* k, const void* v,
                             const float* igate, const float* fgate, const void* ogate,
                             void* h_out, void* htilde_out, float* m_out, float* n_out,
                             int64_t B, int64_t NH, int64_t T, int64_t d, int dtype,
                             void* stream);

/*
 * The same pass split into its two stages with a caller-owned workspace, for
 * callers that time or schedule the stages separately.
 *
 * mlstm_workspace_bytes: bytes of device workspace the two stages need for
 * B x NH heads of length T (0 if the sizes are invalid).
 */
size_t mlstm_workspace_bytes(int64_t B, int64_t NH, int64_t T);

/*
 * mlstm_gate_scan -- stage 1: the gate-only part of Eqs. 79-81 and 101.
 * Computes fbar = log f (log sigmoid(f~), or f~ for MLSTM_FORGET_EXP), its
 * prefix sums, and the row maximum
 *   m_i = max_{j<=i} (sum_{k=j+1..i} fbar_k + i~_j)                 (Eq. 80)
 * through the equivalent recurrence m_i = max(m_{i-1} + fbar_i, i~_i),
 * m_0 = i~_0, before any Q K^T work.  Writes m_out and the per-row and
 * per-column exponent terms and block anchors the tile stage reads into
 * `workspace` (device memory, >= mlstm_workspace_bytes(B, NH, T) bytes,
 * 256-byte aligned).  `d` is needed for the 1/sqrt(d) folded into the
 * exponent terms.
 */
int mlstm_gate_scan(const float* igate, const float* fgate, float* m_out,
                    void* workspace, size_t workspace_bytes,
                    int64_t B, int64_t NH, int64_t T, int64_t d,
                    int forget_activation, void* stream);

/*
 * mlstm_causal_tiles -- stage 2: Eqs. 81-86 over causal tiles.  Reads q, k,
 * v, m (from stage 1) and the workspace stage 1 wrote on the same stream, and
 * writes h_out and n_out.  `kernel` is an MLSTM_KERNEL_* selector.
 */
int mlstm_causal_tiles(const void* q, const void* k, const void* v, const float* m,
                       const void* workspace, size_t workspace_bytes,
                       void* h_out, float* n_out,
                       int64_t B, int64_t NH, int64_t T, int64_t d, int dtype,
                       int kernel, void* stream);

/*
 * mlstm_parallel_fwd_train -- mlstm_parallel_fwd_stream that also stores the
 * row sums b = C~' 1 (Eq. 83), which the backward pass needs (Eq. 90).
 *   b_out              out  [B][NH][T] float32 (required, 16-byte aligned)
 *   forget_activation  MLSTM_FORGET_SIGMOID or MLSTM_FORGET_EXP
 * Other arguments, layouts and errors as for mlstm_parallel_fwd_stream.
 */
int mlstm_parallel_fwd_train(const void* q, const void* k, const void* v,
                             const float* igate, const float* fgate,
                             void* h_out, float* m_out, float* n_out, float* b_out,
                             int64_t B, int64_t NH, int64_t T, int64_t d, int dtype,
                             int forget_activation, void* stream);

/*
 * mlstm_parallel_bwd -- gradients of the stabilized parallel forward pass
 * ("Parallel mLSTM Backward Pass", Eqs. 87-105) with respect to q, k, v and
 * the gate pre-activations, given dh = dL/dH~.
 *   q, k, v, igate, fgate   in: the forward inputs
 *   h, m, n, b              in: the forward outputs of mlstm_parallel_fwd_train
 *                           (h~ before any output gate, [B][NH][T][d] dtype;
 *                           m, n, b [B][NH][T] float32)
 *   dh                      in  [B][NH][T][d], dtype
 *   dq, dk, dv              out [B][NH][T][d], dtype (float32 accumulation)
 *   digate, dfgate          out [B][NH][T] float32
 * m is held constant (its contributions cancel, as the pages note).  Eq. 90
 * is applied with the derivative of |b|, sign(b): the printed sign(n) is 1
 * for every row, since n > 0.  d(log sigma(x))/dx = sigma(-x) (Eq. 104);
 * with forget_activation MLSTM_FORGET_EXP, d(log f)/df~ = 1.  The forward
 * outputs must come from the same forget_activation.
 * dL/dn uses sum_j C~'_ij v_j = n_i h~_i, so for bf16 it carries the
 * rounding of the stored h~.  For bf16 with d <= 512 the contractions run
 * on the matrix cores (bf16 operands, float32 accumulation; the operand
 * E (.) dC~' of the dQ and dK products and C~'/n of the dV product are
 * rounded to bf16, the row and column sums of dD~ behind the gate gradients
 * are not); for float32 with d a multiple of 32 up to 384 they run on the
 * float32 matrix instruction (float32 operands and sums throughout; the
 * environment variable MLSTM_BWD_F32=vector, read at each call, selects the
 * vector passes instead); for the other float32 head dims, and for bf16
 * above d = 512, everything is float32 on the vector ALUs (above d = 512 in
 * head-dimension chunks, a correctness path far slower than the matrix
 * cores).  Results are bitwise reproducible.  The library allocates a stream-ordered workspace: per-row
 * terms and, for bf16 on the matrix cores, the bf16 operands of the dV and
 * dQ products, which the key pass stores so that the dV and dQ passes need
 * not recompute S and G: 8 KiB per head, 128-key block and 32-query tile of
 * the causal triangle for dV, 2 KiB per head and pair of 32-row tiles for dQ
 * (278 MB for 32 heads of 2048).  Above 2 GiB (or the byte count in the
 * environment variable MLSTM_BWD_STORE_MAX, read at each call) those passes
 * recompute them instead: dV is then bitwise the same, dQ, dK and the gate
 * gradients equal up to float32 rounding order.
 * Pointers 16-byte aligned; no output may alias an input.  Any d of the
 * forward pass (a multiple of 16 up to 1024).  Errors as for
 * mlstm_parallel_fwd.
 */
int mlstm_parallel_bwd(const void* q, const void* k, const void* v,
                       const float* igate, const float* fgate,
                       const void* h, const float* m, const float* n, const float* b,
                       const void* dh, void* dq, void* dk, void* dv,
                       float* digate, float* dfgate,
                       int64_t B, int64_t NH, int64_t T, int64_t d, int dtype,
                       int forget_activation, void* stream);

/*
 * mlstm_recurrent_step -- one step of the recurrent mLSTM (the generation
 * form that the parallel pass reformulates; its equations are those the
 * recurrent backward pass of appendix A.3 differentiates, Eqs. 59-70), with
 * the states stabilized by the running maximum of the log gates, the same
 * recurrence as the parallel form's row maximum (Eq. 80):
 *   m_t  = max(fbar_t + m_{t-1}, i~_t),  fbar_t = log f_t (log sigmoid(f~_t),
 *          or f~_t with forget_activation MLSTM_FORGET_EXP)
 *   f'_t = exp(fbar_t + m_{t-1} - m_t),  i'_t = exp(i~_t - m_t)
 *   C_t  = f'_t C_{t-1} + i'_t v_t (k_t / sqrt(d))^T
 *   n_t  = f'_t n_{t-1} + i'_t k_t / sqrt(d)
 *   h~_t = C_t q_t / max(|n_t . q_t|, exp(-m_t))
 * These states are the unstabilized ones times exp(-m_t); h~_t, m_t and the
 * denominator equal row t of mlstm_parallel_fwd's h~, m and n.
 *   q, k, v      in   [B][NH][d], dtype: this step's query, key, value
 *   igate, fgate in   [B][NH] float32: i~_t, f~_t
 *   C_in, n_in, m_in   in  [B][NH][d][d], [B][NH][d], [B][NH] float32: the
 *                state after step t-1 (C rows index the value dimension);
 *                a fresh state is C = 0, n = 0, m = -inf
 *   C_out, n_out, m_out out: the state after step t.  C_out may be C_in
 *                (updated in place); n_out and m_out must not overlap n_in and
 *                m_in (MLSTM_ERR_ALIAS)
 *   h_out        out  [B][NH][d], dtype: h~_t (before any output gate)
 *   den_out      out  [B][NH] float32: max(|n_t . q_t|, exp(-m_t)); may be NULL
 *   d            a multiple of 16 in [16, 1024]
 * Vectors and C need 16-byte alignment, scalars 4-byte.  Asynchronous on
 * `stream`; no workspace.  Bound by memory bandwidth: the state is read and
 * written once per step.
 */
int mlstm_recurrent_step(const void* q, const void* k, const void* v,
                         const float* igate, const float* fgate,
                         const float* C_in, const float* n_in, const float* m_in,
                         float* C_out, float* n_out, float* m_out,
                         void* h_out, float* den_out,
                         int64_t B, int64_t NH, int64_t d, int dtype,
                         int forget_activation, void* stream);

/* Human-readable text of a status code (static storage). */
const char* mlstm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLSTM_H */
