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

namespace mlstm {
namespace {

constexpr int kScanThreads = 512;
constexpr int kScanPer = 4;  // positions per thread per chunk
constexpr int kScanWaves = kScanThreads / 64;
static_assert(kScanThreads * kScanPer == kScanChunk, "chunk of the gate scan");

struct MaxPlus {  // the map x -> max(x + a, b)
  double a, b;
};

__device__ inline MaxPlus compose(MaxPlus first, MaxPlus second) {
  return {first.a + second.a, fmax(first.b + second.a, second.b)};
}

__device__ inline double apply(MaxPlus f, double x) { return fmax(x + f.a, f.b); }

// a scan element: the map of a run of positions; its shift a is the sum of
// fbar over the run
typedef MaxPlus Elem;

__device__ inline Elem identity() { return {0.0, -INFINITY}; }

__device__ inline Elem combine(Elem first, Elem second) { return compose(first, second); }

// log sigmoid(x) = min(x, 0) - log1p(exp(-|x|)): never forms exp(+|x|).  The
// first term is exact; the second, in (0, ln 2], is evaluated in float32 and
// subtracted in float64.
__device__ inline double log_sigmoid(float x) {
  return double(fminf(x, 0.0f)) - double(log1pf(expf(-fabsf(x))));
}

// A float64 value from another lane by a DPP pattern (two 32-bit moves);
// lanes without a source in the pattern, and rows outside ROW_MASK, get `old`.
template <int CTRL, int ROW_MASK>
__device__ inline double dpp64(double x, double old) {
  const uint64_t xb = __builtin_bit_cast(uint64_t, x), ob = __builtin_bit_cast(uint64_t, old);
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(int(uint32_t(ob)), int(uint32_t(xb)),
                                                            CTRL, ROW_MASK, 0xF, false));
  const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(int(uint32_t(ob >> 32)),
                                                            int(uint32_t(xb >> 32)), CTRL, ROW_MASK,
                                                            0xF, false));
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}
// the element of an earlier lane by the pattern, the identity where there is none
template <int CTRL, int ROW_MASK>
__device__ inline Elem dpp_elem(Elem x) {
  const Elem id = identity();
  return {dpp64<CTRL, ROW_MASK>(x.a, id.a), dpp64<CTRL, ROW_MASK>(x.b, id.b)};
}
// DPP controls (gfx9): shift right within rows of 16 lanes, broadcast lane 15
// of a row to the next row, lane 31 to rows 2 and 3, shift the wave right by 1
constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

// Ordered scan of one element per thread over the workgroup (thread order):
// returns the composition of the elements of all earlier threads and stores
// that of all threads in `total`.  Within a wave: an inclusive scan by row
// shifts of 1, 2, 4, 8 lanes, then the row totals by the two row broadcasts
// (DPP moves, no LDS); across the waves, in order through LDS.
__device__ Elem block_scan(Elem x, Elem& total) {
  __shared__ double s_a[kScanWaves];
  __shared__ double s_b[kScanWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  Elem incl = x;  // inclusive scan across the wave
  incl = combine(dpp_elem<kRowShr + 1, 0xF>(incl), incl);
  incl = combine(dpp_elem<kRowShr + 2, 0xF>(incl), incl);
  incl = combine(dpp_elem<kRowShr + 4, 0xF>(incl), incl);
  incl = combine(dpp_elem<kRowShr + 8, 0xF>(incl), incl);
  incl = combine(dpp_elem<kRowBcast15, 0xA>(incl), incl);
  incl = combine(dpp_elem<kRowBcast31, 0xC>(incl), incl);
  if (lane == 63) {
    s_a[wave] = incl.a;
    s_b[wave] = incl.b;
  }
  __syncthreads();
  Elem before = identity();  // the waves before this one
  total = identity();
  for (int w = 0; w < kScanWaves; ++w) {
    const Elem e = {s_a[w], s_b[w]};
    if (w < wave) before = combine(before, e);
    total = combine(total, e);
  }
  // lane-exclusive = inclusive of the previous lane (the identity on lane 0)
  const Elem lexcl = dpp_elem<kWaveShr1, 0xF>(incl);
  __syncthreads();  // the shared totals may be rewritten by the next call
  return combine(before, lexcl);
}

// f~ and i~ of positions p0 .. p0 + 3 as stored (padding: f~ = 0, i~ = -inf)
__device__ inline void load_raw(const float* f, const float* ig, int64_t p0, int64_t T,
                                bool vec_rows, float fb[kScanPer], float iv[kScanPer]) {
  if (vec_rows && p0 + kScanPer <= T) {
    const float4 f4 = *reinterpret_cast<const float4*>(f + p0);
    const float4 i4 = *reinterpret_cast<const float4*>(ig + p0);
    fb[0] = f4.x; fb[1] = f4.y; fb[2] = f4.z; fb[3] = f4.w;
    iv[0] = i4.x; iv[1] = i4.y; iv[2] = i4.z; iv[3] = i4.w;
  } else {
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
      const int64_t p = p0 + e;
      fb[e] = p < T ? f[p] : 0.0f;
      iv[e] = p < T ? ig[p] : -INFINITY;
    }
  }
}

// log f_t of the same positions (padding: no forgetting, no input; it never
// reaches a real row)
__device__ inline void to_log_forget(int64_t p0, int64_t T, int exp_forget,
                                     const float fr[kScanPer], double fb[kScanPer]) {
#pragma unroll
  for (int e = 0; e < kScanPer; ++e)
    fb[e] = p0 + e < T ? (exp_forget ? double(fr[e]) : log_sigmoid(fr[e])) : 0.0;
}

__device__ inline void load_gates(const float* f, const float* ig, int64_t p0, int64_t T,
                                  bool vec_rows, int exp_forget, double fb[kScanPer],
                                  float iv[kScanPer]) {
  float fr[kScanPer];
  load_raw(f, ig, p0, T, vec_rows, fr, iv);
  to_log_forget(p0, T, exp_forget, fr, fb);
}

// the element of one thread's positions
__device__ inline Elem thread_elem(const double fb[kScanPer], const float iv[kScanPer]) {
  Elem t = identity();
#pragma unroll
  for (int e = 0; e < kScanPer; ++e)
    t = combine(t, Elem{fb[e], double(iv[e])});
  return t;
}

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
  const double kLog2e = 1.4426950408889634074;
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

    double cs = carry.a + before.a;                     // sum of fbar before p0
    double m = apply(before, apply(carry, -INFINITY));  // m at p0 - 1
    double rmax = -INFINITY, cmax = -INFINITY;  // of the values stored below
    float mv[kScanPer];
    double rv[kScanPer], cv[kScanPer];
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
      const int64_t p = p0 + e;
      cs += fb[e];
      m = fmax(m + fb[e], double(iv[e]));
      if (p < T) {
        mv[e] = float(m);
        rv[e] = (cs - m - half_ln_d) * kLog2e;
        cv[e] = (double(iv[e]) - cs) * kLog2e;
        rmax = fmax(rmax, rv[e]);
        cmax = fmax(cmax, cv[e]);
      } else {  // padding up to Tp
        mv[e] = 0.0f;
        rv[e] = 0.0;
        cv[e] = -INFINITY;
        rmax = fmax(rmax, 0.0);
      }
    }
    // tile bounds: the 8 threads of a 32-position tile are 8 consecutive lanes
    rmax = fmax(rmax, __shfl_xor(rmax, 1, 64));
    rmax = fmax(rmax, __shfl_xor(rmax, 2, 64));
    rmax = fmax(rmax, __shfl_xor(rmax, 4, 64));
    cmax = fmax(cmax, __shfl_xor(cmax, 1, 64));
    cmax = fmax(cmax, __shfl_xor(cmax, 2, 64));
    cmax = fmax(cmax, __shfl_xor(cmax, 4, 64));
    // the key factor of the factored exponent, relative to its tile's maximum:
    // the difference is formed in float64 and rounded once
    float xv[kScanPer];
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) xv[e] = p0 + e < T ? exp2f(float(cv[e] - cmax)) : 0.0f;
    if (p0 < Tp) {  // Tp is a multiple of 128: the 4 positions are all below it
      *reinterpret_cast<double2*>(rt + p0) = make_double2(rv[0], rv[1]);
      *reinterpret_cast<double2*>(rt + p0 + 2) = make_double2(rv[2], rv[3]);
      *reinterpret_cast<double2*>(ct + p0) = make_double2(cv[0], cv[1]);
      *reinterpret_cast<double2*>(ct + p0 + 2) = make_double2(cv[2], cv[3]);
      *reinterpret_cast<float4*>(cx + p0) = make_float4(xv[0], xv[1], xv[2], xv[3]);
      if ((p0 & (kBoundTile - 1)) == 0) {
        rb[p0 / kBoundTile] = rmax;
        kb[p0 / kBoundTile] = cmax;
      }
    }
    if (vec_rows && p0 + kScanPer <= T) {
      *reinterpret_cast<float4*>(mo + p0) = make_float4(mv[0], mv[1], mv[2], mv[3]);
    } else {
#pragma unroll
      for (int e = 0; e < kScanPer; ++e)
        if (p0 + e < T) mo[p0 + e] = mv[e];
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
