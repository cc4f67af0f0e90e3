// Stage 1 of the stabilized parallel mLSTM forward pass: the gate scan.
//
// Everything in Eqs. 79-81 of the xLSTM appendix that depends only on the
// gates is computed here, before any Q K^T work:
//
//   fbar_k = log sigmoid(f~_k)   (f~_k for an exponential forget gate) (Eq. 101)
//   m_i    = max_{j<=i} (sum_{k=j+1..i} fbar_k + i~_j)          (Eqs. 79, 80)
//
// The row maximum is evaluated through the recurrence obtained by splitting
// j = i (where log F_ii = 0, so D~_ii = i~_i) from j < i (where
// D~_ij = fbar_i + D~_{i-1,j}):  m_i = max(m_{i-1} + fbar_i, i~_i), m_0 = i~_0.
// Each step is the map x -> max(x + a, b); composing two such maps gives
// another, (a1, b1) then (a2, b2) = (a1 + a2, max(b1 + a2, b2)), so the
// recurrence is an associative scan and runs in parallel.  This avoids the
// cancellation of the closed form cs_i + max_j (i~_j - cs_j), whose two
// terms each grow with the sequence length.  The shift a of a composed map is
// the sum of fbar over its positions, so the same scan also yields the prefix
// sums of fbar.
//
// A workgroup of 512 threads scans a chunk of 2048 positions; each thread
// owns 4 consecutive positions (an eighth of a 32-position tile),
// loaded and stored as 16-byte vectors where the row alignment allows.  Short
// sequences take one workgroup per head that walks its chunks in order.  Long
// ones are scanned in two passes, so that every chunk has a workgroup of its
// own: the first reduces each chunk to its element (sum, map), the second
// gives each chunk the composition of all earlier chunks' elements (folded in
// order across the workgroup's threads) as its carry and scans it.  Sums and
// the max-plus maps are carried in float64.  log sigmoid(x) is the exact
// min(x, 0) minus log1p(exp(-|x|)), a value in (0, ln 2] whose float32
// evaluation is off by about 1e-7 at most: the sum is taken in float64, so
// the error of fbar does not grow with |x|.
#include "mlstm_internal.h"
#include "scan_common.h"

namespace mlstm {
namespace {

using namespace scan;

// First pass of the two-pass scan: the element of chunk c of head h
// (workgroup h * nchunk + c), stored as (a, b).
__global__ __launch_bounds__(kScanThreads) void scan_totals_kernel(
    const float* __restrict__ igate, const float* __restrict__ fgate, double* __restrict__ segs,
    int64_t T, int64_t nchunk, int exp_forget) {
  const int64_t head = int64_t(blockIdx.x) / nchunk;
  const int64_t c = int64_t(blockIdx.x) % nchunk;
  const int64_t p0 = c * kScanChunk + int64_t(threadIdx.x) * kScanPer;
  double fb[kScanPer];
  float iv[kScanPer];
  load_gates(fgate + head * T, igate + head * T, p0, T, (T & 3) == 0, exp_forget, fb, iv);
  Elem total;
  block_scan(thread_elem(fb, iv), total);
  if (threadIdx.x == 0) {
    double* s = segs + (head * nchunk + c) * 2;
    s[0] = total.a;
    s[1] = total.b;
  }
}

// Scans chunks [c0, c0 + count) of one head: workgroup x covers head
// x / groups and c0 = (x % groups) * count.  With segs != NULL the carry into
// chunk c0 is the composition of the stored elements of chunks 0 .. c0 - 1
// (each thread folds a contiguous run of them in order, then the runs are
// composed in thread order).  kLoop = false handles count == 1 only: without
// the chunk loop the kernel needs 63 registers instead of 108, so twice as
// many workgroups fit on a CU.
template <bool kLoop>
__global__ __launch_bounds__(kScanThreads) void gate_scan_kernel(
    const float* __restrict__ igate, const float* __restrict__ fgate, float* __restrict__ m_out,
    double* __restrict__ rowt, double* __restrict__ colt, float* __restrict__ colx,
    double* __restrict__ rowb, double* __restrict__ keyb, const double* __restrict__ segs,
    int64_t T, int64_t Tp, int64_t nchunk, int64_t groups, int64_t count, double half_ln_d,
    int exp_forget) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t head = int64_t(blockIdx.x) / groups;
  const int64_t c0 = (int64_t(blockIdx.x) % groups) * count;
  const float* f = fgate + head * T;
  const float* ig = igate + head * T;
  float* mo = m_out + head * T;
  double* rt = rowt + head * Tp;
  double* ct = colt + head * Tp;
  float* cx = colx + head * Tp;
  double* rb = rowb + head * (Tp / kBoundTile);
  double* kb = keyb + head * (Tp / kBoundTile);
  // the rows of the [H][T] arrays start 16-byte aligned when T % 4 == 0
  // (their base pointers are 16-byte aligned)
  const bool vec_rows = (T & 3) == 0;

  Elem carry = identity();  // everything before the current chunk
  if (segs != nullptr && c0 > 0) {
    const int64_t per = (c0 + kScanThreads - 1) / kScanThreads;
    Elem run = identity();
    for (int64_t j = int64_t(tid) * per; j < c0 && j < int64_t(tid + 1) * per; ++j) {
      const double* s = segs + (head * nchunk + j) * 2;
      run = combine(run, Elem{s[0], s[1]});
    }
    block_scan(run, carry);
  }

  // the gates of the next chunk are loaded before the current one is scanned
  const int64_t c_end = c0 + count < (Tp + kScanChunk - 1) / kScanChunk
                            ? c0 + count
                            : (Tp + kScanChunk - 1) / kScanChunk;
  float fn[kScanPer], in[kScanPer];
  if (c0 < c_end) load_raw(f, ig, c0 * kScanChunk + int64_t(tid) * kScanPer, T, vec_rows, fn, in);
  for (int64_t chunk = c0; chunk < (kLoop ? c_end : c0 + 1); ++chunk) {
    const int64_t p0 = chunk * kScanChunk + int64_t(tid) * kScanPer;
    float fr[kScanPer], iv[kScanPer];
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
      fr[e] = fn[e];
      iv[e] = in[e];
    }
    if (kLoop && chunk + 1 < c_end) load_raw(f, ig, p0 + kScanChunk, T, vec_rows, fn, in);
    double fb[kScanPer];
    to_log_forget(p0, T, exp_forget, fr, fb);
    Elem total;
    const Elem before = block_scan(thread_elem(fb, iv), total);

    Terms t;
    position_terms(carry, before, fb, iv, p0, T, half_ln_d, t);
    if (p0 < Tp) {  // Tp is a multiple of 128: the 4 positions are all below it
      *reinterpret_cast<double2*>(rt + p0) = make_double2(t.r[0], t.r[1]);
      *reinterpret_cast<double2*>(rt + p0 + 2) = make_double2(t.r[2], t.r[3]);
      *reinterpret_cast<double2*>(ct + p0) = make_double2(t.c[0], t.c[1]);
      *reinterpret_cast<double2*>(ct + p0 + 2) = make_double2(t.c[2], t.c[3]);
      *reinterpret_cast<float4*>(cx + p0) = make_float4(t.e[0], t.e[1], t.e[2], t.e[3]);
      if ((p0 & (kBoundTile - 1)) == 0) {
        rb[p0 / kBoundTile] = t.rmax;
        kb[p0 / kBoundTile] = t.cmax;
      }
    }
    if (vec_rows && p0 + kScanPer <= T) {
      *reinterpret_cast<float4*>(mo + p0) = make_float4(t.m[0], t.m[1], t.m[2], t.m[3]);
    } else {
#pragma unroll
      for (int e = 0; e < kScanPer; ++e)
        if (p0 + e < T) mo[p0 + e] = t.m[e];
    }
    carry = combine(carry, total);
  }
}

}  // namespace

hipError_t launch_gate_scan(const float* igate, const float* fgate, float* m_out,
                            const Workspace& ws, int64_t H, int64_t T, int64_t d,
                            bool exp_forget, hipStream_t stream) {
  const int64_t nchunk = scan_chunks(T);
  const double half_ln_d = 0.5 * log(double(d));
  if (nchunk < kScanTwoPassChunks) {  // one workgroup per head, chunks in order
    if (nchunk == 1)
      hipLaunchKernelGGL(gate_scan_kernel<false>, dim3(unsigned(H)), dim3(kScanThreads), 0, stream,
                         igate, fgate, m_out, ws.rowt, ws.colt, ws.colx, ws.rowb, ws.keyb,
                         static_cast<const double*>(nullptr), T, ws.Tp, nchunk, int64_t(1),
                         int64_t(1), half_ln_d, int(exp_forget));
    else
      hipLaunchKernelGGL(gate_scan_kernel<true>, dim3(unsigned(H)), dim3(kScanThreads), 0, stream,
                         igate, fgate, m_out, ws.rowt, ws.colt, ws.colx, ws.rowb, ws.keyb,
                         static_cast<const double*>(nullptr), T, ws.Tp, nchunk, int64_t(1),
                         nchunk, half_ln_d, int(exp_forget));
    return hipGetLastError();
  }
  const dim3 grid(unsigned(H * nchunk));
  hipLaunchKernelGGL(scan_totals_kernel, grid, dim3(kScanThreads), 0, stream, igate, fgate,
                     ws.segs, T, nchunk, int(exp_forget));
  hipLaunchKernelGGL(gate_scan_kernel<false>, grid, dim3(kScanThreads), 0, stream, igate, fgate, m_out,
                     ws.rowt, ws.colt, ws.colx, ws.rowb, ws.keyb,
                     static_cast<const double*>(ws.segs), T, ws.Tp, nchunk, nchunk, int64_t(1),
                     half_ln_d, int(exp_forget));
  return hipGetLastError();
}

}  // namespace mlstm
