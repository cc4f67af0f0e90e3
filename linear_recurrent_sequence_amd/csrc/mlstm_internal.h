// Internal declarations shared by the HIP translation units of libmlstm.
//
// Workspace written by the gate scan and read by the tile kernels, for H
// heads of length T, padded to Tp = ceil(T / 128) * 128 positions:
//
//   rowt   [H][Tp]     float64  R_i = (cs_i - m_i - ln(d)/2) * log2(e)      (0 on padding)
//   colt   [H][Tp]     float64  C_j = (i~_j - cs_j) * log2(e)               (-inf on padding)
//   colx   [H][Tp]     float32  e_j = 2^fl32(C_j - keyb_{j/32})             (0 on padding)
//   rowb   [H][Tp/32]  float64  max of R_i over each 32-row block
//   keyb   [H][Tp/32]  float64  max of C_j over each 32-key tile (-inf if all padding)
//   segs   [H][nchunk][2] float64  the scan element (max-plus map a, b; a is the
//                                sum of fbar) of each 2048-position chunk
//                                (long sequences)
//
// where fbar = log sigmoid(f~) (or f~ for an exponential forget gate) and cs
// is its inclusive prefix sum, so that, for j <= i (Eqs. 79-82 and 101 of the
// xLSTM appendix),
//
//   log2( D'_ij / sqrt(d) ) = R_i + C_j.
//
// Every term is float64, and a kernel forms each exponent in float64 and
// rounds it to float32 once, right before the exp2: the rounding error of an
// exponent is then 2^-24 of its own magnitude, whatever the sizes of R_i and
// C_j (both grow with the prefix sums).  The float64 prefix sums resolve
// differences cs_i - cs_j to about 2^-53 |cs| per position between j and i.
//
// Factored exponent: below the diagonal (every key of a 32-key tile J before
// every query of a 32-row block), 2^(R_i + C_j) equals 2^(R_i + keyb_J) * e_j,
// with both exponents formed in float64 and rounded once; neither factor can
// overflow: the first is at most 1 (D' <= 1 and keyb_J is attained by a key of
// the tile), the second lies in (0, 1].  Each rounding is bounded by its own
// exponent, and the two exponents have the sign and sum of R_i + C_j.
//
// Tile bound: every exponent a tile kernel forms for the 32 x 32 block of a
// 32-row block W and a 32-key tile J is fl32 of a float64 value at most
// rowb_W + keyb_J (float64 addition and rounding are monotone).  Where that
// sum is below kSkipLog2 every exponential of the tile is exactly 0 in
// float32, every C~' entry is 0, and the tile contributes nothing: the tile
// kernels skip it without changing any result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlstm {

constexpr int kRowPad = 128;     // T is padded to a multiple of this
constexpr int kBoundTile = 32;   // rows / keys per entry of rowb and keyb
constexpr double kSkipLog2 = -200.0;
constexpr int kScanChunk = 2048;        // positions per workgroup pass of the gate scan
constexpr int kScanTwoPassChunks = 4;   // from this many chunks on, the scan runs in two passes

struct Workspace {
  double* rowt;
  double* colt;
  float* colx;
  double* rowb;
  double* keyb;
  double* segs;
  int64_t Tp;
};

inline int64_t padded_len(int64_t T) { return (T + kRowPad - 1) / kRowPad * kRowPad; }

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// chunks of the gate scan over a sequence of T positions
inline int64_t scan_chunks(int64_t T) { return (padded_len(T) + kScanChunk - 1) / kScanChunk; }

inline size_t workspace_bytes(int64_t H, int64_t T) {
  const int64_t Tp = padded_len(T);
  return 2 * align256(size_t(H) * size_t(Tp) * sizeof(double)) +
         align256(size_t(H) * size_t(Tp) * sizeof(float)) +
         2 * align256(size_t(H) * size_t(Tp / kBoundTile) * sizeof(double)) +
         align256(size_t(H) * size_t(scan_chunks(T)) * 2 * sizeof(double));
}

inline Workspace carve(void* base, int64_t H, int64_t T) {
  Workspace w;
  w.Tp = padded_len(T);
  char* p = static_cast<char*>(base);
  w.rowt = reinterpret_cast<double*>(p);
  p += align256(size_t(H) * size_t(w.Tp) * sizeof(double));
  w.colt = reinterpret_cast<double*>(p);
  p += align256(size_t(H) * size_t(w.Tp) * sizeof(double));
  w.colx = reinterpret_cast<float*>(p);
  p += align256(size_t(H) * size_t(w.Tp) * sizeof(float));
  w.rowb = reinterpret_cast<double*>(p);
  p += align256(size_t(H) * size_t(w.Tp / kBoundTile) * sizeof(double));
  w.keyb = reinterpret_cast<double*>(p);
  p += align256(size_t(H) * size_t(w.Tp / kBoundTile) * sizeof(double));
  w.segs = reinterpret_cast<double*>(p);
  return w;
}

// Optional epilogue of the tile kernels: the output gate H = sigma(O~) (.) H~
// (Eq. 78), applied to the float32 h~ before it is rounded and stored.
// ogate = NULL: h_out receives h~.  htilde != NULL: h~ is stored there too.
// Both are [H][T][d] in the element type of q.
// b != NULL: the row sums b (Eq. 83), float32 [H][T], are stored too (the
// backward pass needs their sign).
struct Epilogue {
  const void* ogate = nullptr;
  void* htilde = nullptr;
  float* b = nullptr;
};

// Stage 1: gate scan (one workgroup per head).  exp_forget: the forget gate
// is exp(f~) (log f = f~) instead of sigmoid(f~).
hipError_t launch_gate_scan(const float* igate, const float* fgate, float* m_out,
                            const Workspace& ws, int64_t H, int64_t T, int64_t d,
                            bool exp_forget, hipStream_t stream);

// Stage 2, bf16 matrix-core tiles; `skip` enables the decay-aware skipping
// of tiles whose bound is below kSkipLog2 (results are identical either way).
// Returns hipErrorInvalidValue for an unsupported head dimension (none for
// d % 16 == 0, 16 <= d <= 512).
hipError_t launch_tiles_mfma(const void* q, const void* k, const void* v, const float* m,
                             const Workspace& ws, void* h_out, float* n_out,
                             const Epilogue& ep, bool skip, int64_t H, int64_t T, int64_t d,
                             hipStream_t stream);

// Both stages in one launch of that kernel for 384 < d <= 512 (T <= 2048, T
// divisible by 4): it scans its head's gates in its prologue (as the gate
// scan does, bitwise) and keeps the terms it reads in LDS, with no workspace.
bool tiles_mfma_fused_supports(int64_t T, int64_t d);
hipError_t launch_tiles_mfma_fused(const void* q, const void* k, const void* v,
                                   const float* igate, const float* fgate, void* h_out,
                                   float* m_out, float* n_out, const Epilogue& ep,
                                   bool exp_forget, int64_t H, int64_t T, int64_t d,
                                   hipStream_t stream);

// Stage 2, bf16 matrix-core tiles with two waves per SIMD (d <= 384), the
// same results up to float32 rounding order.
bool tiles_pairs_supports(int64_t d);
hipError_t launch_tiles_pairs(const void* q, const void* k, const void* v, const float* m,
                              const Workspace& ws, void* h_out, float* n_out,
                              const Epilogue& ep, bool skip, int64_t H, int64_t T, int64_t d,
                              hipStream_t stream);

// Both stages in one launch (d <= 384, T <= 2048, T divisible by 4): the
// same kernel, which scans its head's gates in its prologue and keeps the
// terms in LDS, with no workspace; m, n, h (and the epilogue's outputs)
// bitwise those of the two stages.  Decay-aware skipping is on.
bool tiles_pairs_fused_supports(int64_t T, int64_t d);
hipError_t launch_tiles_pairs_fused(const void* q, const void* k, const void* v,
                                    const float* igate, const float* fgate, void* h_out,
                                    float* m_out, float* n_out, const Epilogue& ep,
                                    bool exp_forget, int64_t H, int64_t T, int64_t d,
                                    hipStream_t stream);

// Both stages in one launch with a software-pipelined key loop (bf16, d a
// multiple of 64 up to 384, T <= 2048, T divisible by 4): four waves, one per
// SIMD, each with 32 query rows and all columns; K and V staged through
// registers into double-buffered LDS tiles.
bool tiles_pipe_supports(int64_t T, int64_t d);
// whether the one-launch forward pass takes this kernel (d <= 192)
bool tiles_pipe_preferred(int64_t T, int64_t d);
hipError_t launch_tiles_pipe(const void* q, const void* k, const void* v, const float* igate,
                             const float* fgate, void* h_out, float* m_out, float* n_out,
                             const Epilogue& ep, bool exp_forget, int64_t H, int64_t T,
                             int64_t d, hipStream_t stream);

// Stage 2, bf16 matrix-core tiles for wide heads (d <= 1024): four waves
// share 32 query rows and split the head dimension in quarters.
bool tiles_wide_supports(int64_t d);
hipError_t launch_tiles_wide(const void* q, const void* k, const void* v, const float* m,
                             const Workspace& ws, void* h_out, float* n_out,
                             const Epilogue& ep, bool skip, int64_t H, int64_t T, int64_t d,
                             hipStream_t stream);

// Stage 2, float32 matrix-core tiles (v_mfma_f32_32x32x2_f32) for float32
// inputs, d a multiple of 32 up to 256, or 320, 384, 512; `skip` as for the
// bf16 kernels.
bool tiles_f32_supports(int64_t d);
hipError_t launch_tiles_f32(const void* q, const void* k, const void* v, const float* m,
                            const Workspace& ws, void* h_out, float* n_out, const Epilogue& ep,
                            bool skip, int64_t H, int64_t T, int64_t d, hipStream_t stream);

// Stage 2, float32 vector-ALU tiles; is_bf16 selects the element type.
hipError_t launch_tiles_vector(const void* q, const void* k, const void* v, const float* m,
                               const Workspace& ws, void* h_out, float* n_out,
                               const Epilogue& ep, int64_t H, int64_t T, int64_t d,
                               bool is_bf16, hipStream_t stream);

// Both stages in one launch on the float32 matrix-core kernel (T <= 2048, a
// d it takes): the kernel scans its head's gates in its prologue.
bool tiles_f32_fused_supports(int64_t T, int64_t d);
hipError_t launch_tiles_f32_fused(const void* q, const void* k, const void* v, const float* igate,
                                  const float* fgate, void* h_out, float* m_out, float* n_out,
                                  const Epilogue& ep, bool exp_forget, int64_t H, int64_t T,
                                  int64_t d, hipStream_t stream);

// Both stages in one launch on the vector tiles (T <= 2048, any d of the
// vector kernel): the kernel scans its head's gates in its prologue.
bool tiles_vector_fused_supports(int64_t T, int64_t d);
hipError_t launch_tiles_vector_fused(const void* q, const void* k, const void* v,
                                     const float* igate, const float* fgate, void* h_out,
                                     float* m_out, float* n_out, const Epilogue& ep,
                                     bool exp_forget, int64_t H, int64_t T, int64_t d,
                                     bool is_bf16, hipStream_t stream);

// Backward pass (Eqs. 87-105), d <= kBackwardMaxHeadDim: bf16 inputs with
// d <= 512 on the matrix cores, everything else on float32 vector tiles (whole
// 16-row tiles in LDS up to d = 512, head-dimension chunks of 256 above).  `ws` holds
// the gate scan's terms for the same inputs.  backward_store_bytes gives the
// size of the stored operand of the dV product (0: the values pass recomputes
// it); it reads the environment, so a caller evaluates it once and passes the
// same value to backward_scratch_bytes and launch_backward.  `scratch` holds
// backward_scratch_bytes(H, T, store_bytes) bytes (256-byte aligned): per-row
// temporaries, then the stored operand.
constexpr int kBackwardMaxHeadDim = 1024;
size_t backward_store_bytes(int64_t H, int64_t T, int64_t d, bool is_bf16);
size_t backward_scratch_bytes(int64_t H, int64_t T, size_t store_bytes);
hipError_t launch_backward(const void* q, const void* k, const void* v, const float* fgate,
                           const void* h, const float* m, const float* n, const float* b,
                           const void* dh, const Workspace& ws, void* scratch,
                           size_t store_bytes, void* dq, void* dk, void* dv, float* digate,
                           float* dfgate, int64_t H, int64_t T, int64_t d, bool is_bf16,
                           bool exp_forget, hipStream_t stream);

// The row and column passes of the backward on the matrix cores (bf16,
// d <= 512): dQ and the row sums r of dD~ (the rows pass also stores the
// per-row scalars 1/n and db into inv_n, db), dK and the column sums c, dV.
// With vstore != NULL (backward_mfma_store_bytes(H, T) bytes) the keys pass
// also stores bf16(C~'/n), the operand of the dV product, and the values
// pass reads it instead of recomputing S; dV is bitwise the same either way.
bool backward_mfma_supports(int64_t d);
size_t backward_mfma_store_bytes(int64_t H, int64_t T);
hipError_t launch_backward_mfma_tiles(const void* q, const void* k, const void* v,
                                      const void* dh, const void* h, const float* m,
                                      const float* n, const float* b, float* inv_n, float* db,
                                      const Workspace& ws, void* dq, void* dk, void* dv,
                                      float* rsum, float* csum, void* vstore, int64_t H,
                                      int64_t T, int64_t d, hipStream_t stream);

// The row and column passes of the backward on the float32 matrix
// instruction (float32 inputs, d a multiple of 32 up to 384): dQ and the row
// sums r of dD~, dK and the column sums c, dV, from the per-row scalars 1/n
// and db.
bool backward_f32_supports(int64_t d);
hipError_t launch_backward_f32_tiles(const float* q, const float* k, const float* v,
                                     const float* dh, const float* inv_n, const float* db,
                                     const Workspace& ws, float* dq, float* dk, float* dv,
                                     float* rsum, float* csum, int64_t H, int64_t T, int64_t d,
                                     hipStream_t stream);

// Recurrent step (generation), stabilized states in float32: C [H][d][d],
// n [H][d], m [H].  C_out may equal C_in; n_out / m_out must not overlap
// n_in / m_in.  den_out [H] is optional.  hipErrorInvalidValue for an
// unsupported d (a multiple of 16 in [16, 1024] is supported).
hipError_t launch_recurrent_step(const void* q, const void* k, const void* v, const float* igate,
                                 const float* fgate, const float* C_in, const float* n_in,
                                 const float* m_in, float* C_out, float* n_out, float* m_out,
                                 void* h_out, float* den_out, int64_t H, int64_t d, bool is_bf16,
                                 bool exp_forget, hipStream_t stream);

}  // namespace mlstm
