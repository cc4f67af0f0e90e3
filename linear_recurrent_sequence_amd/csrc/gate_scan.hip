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
// terms each grow with the sequence length.
//
// One workgroup of 512 threads per head walks the sequence in chunks of
// 2048 positions; each thread owns 4 consecutive positions (one sixteenth of
// a 64-position anchor block), loaded and stored as 16-byte vectors where the
// row alignment allows.  Sums and the max-plus maps are carried in float64;
// log sigmoid is evaluated in float32 (its relative error stays local: only
// sums over the few positions where D' is not negligible matter).
#include "mlstm_internal.h"

namespace mlstm {
namespace {

constexpr int kScanThreads = 512;
constexpr int kScanPer = 4;  // positions per thread per chunk
constexpr int kScanWaves = kScanThreads / 64;

struct MaxPlus {  // the map x -> max(x + a, b)
  double a, b;
};

__device__ inline MaxPlus compose(MaxPlus first, MaxPlus second) {
  return {first.a + second.a, fmax(first.b + second.a, second.b)};
}

__device__ inline double apply(MaxPlus f, double x) { return fmax(x + f.a, f.b); }

// log sigmoid(x) = min(x, 0) - log1p(exp(-|x|)): never forms exp(+|x|).
__device__ inline float log_sigmoid(float x) {
  return fminf(x, 0.0f) - log1pf(expf(-fabsf(x)));
}

__global__ __launch_bounds__(kScanThreads) void gate_scan_kernel(
    const float* __restrict__ igate, const float* __restrict__ fgate, float* __restrict__ m_out,
    double* __restrict__ anchor, float* __restrict__ rowt, float* __restrict__ colt,
    float* __restrict__ colx, float* __restrict__ rowb, float* __restrict__ keyb, int64_t T,
    int64_t Tp, int64_t nblk,
    double half_ln_d, int exp_forget) {
  const double kLog2e = 1.4426950408889634074;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t head = blockIdx.x;
  const float* f = fgate + head * T;
  const float* ig = igate + head * T;
  float* mo = m_out + head * T;
  double* anc = anchor + head * nblk;
  float* rt = rowt + head * Tp;
  float* ct = colt + head * Tp;
  float* cx = colx + head * Tp;
  float* rb = rowb + head * (Tp / kBoundTile);
  float* kb = keyb + head * (Tp / kBoundTile);
  // the rows of the [H][T] arrays start 16-byte aligned when T % 4 == 0
  // (their base pointers are 16-byte aligned)
  const bool vec_rows = (T & 3) == 0;

  __shared__ double s_sum[kScanWaves];
  __shared__ double s_a[kScanWaves];
  __shared__ double s_b[kScanWaves];

  double carry_cs = 0.0;        // sum of fbar over all earlier chunks
  double carry_m = -INFINITY;   // m at the last position of the previous chunk

  for (int64_t base = 0; base < Tp; base += int64_t(kScanThreads) * kScanPer) {
    const int64_t p0 = base + int64_t(tid) * kScanPer;
    float fb[kScanPer];
    float iv[kScanPer];
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
    double tsum = 0.0;
    MaxPlus tmap = {0.0, -INFINITY};
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
      // log f_t; padding has no forgetting and no input and never reaches a real row
      fb[e] = p0 + e < T ? (exp_forget ? fb[e] : log_sigmoid(fb[e])) : 0.0f;
      tsum += double(fb[e]);
      tmap = compose(tmap, MaxPlus{double(fb[e]), double(iv[e])});
    }

    // inclusive scan across the wave
    double isum = tsum;
    MaxPlus imap = tmap;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double os = __shfl_up(isum, off, 64);
      const double oa = __shfl_up(imap.a, off, 64);
      const double ob = __shfl_up(imap.b, off, 64);
      if (lane >= off) {
        isum = os + isum;
        imap = compose(MaxPlus{oa, ob}, imap);
      }
    }
    if (lane == 63) {
      s_sum[wave] = isum;
      s_a[wave] = imap.a;
      s_b[wave] = imap.b;
    }
    __syncthreads();
    // exclusive prefix of the wave totals (each thread recomputes it; 16 terms)
    double wsum = 0.0;
    MaxPlus wmap = {0.0, -INFINITY};
    for (int w = 0; w < wave; ++w) {
      wsum += s_sum[w];
      wmap = compose(wmap, MaxPlus{s_a[w], s_b[w]});
    }
    double tot_sum = 0.0;
    MaxPlus tot_map = {0.0, -INFINITY};
    for (int w = 0; w < kScanWaves; ++w) {
      tot_sum += s_sum[w];
      tot_map = compose(tot_map, MaxPlus{s_a[w], s_b[w]});
    }
    // lane-exclusive = inclusive of the previous lane
    double lsum = __shfl_up(isum, 1, 64);
    MaxPlus lmap = {__shfl_up(imap.a, 1, 64), __shfl_up(imap.b, 1, 64)};
    if (lane == 0) {
      lsum = 0.0;
      lmap = {0.0, -INFINITY};
    }

    double cs = carry_cs + wsum + lsum;                 // sum of fbar before p0
    double m = apply(lmap, apply(wmap, carry_m));       // m at p0 - 1
    // anchor of this thread's 64-block: the prefix sum before the block start,
    // held by the first of the 16 threads that share the block
    const double blk_anchor = __shfl(cs, lane & ~15, 64);
    if (p0 < Tp && (p0 & (kAnchorBlock - 1)) == 0) anc[p0 / kAnchorBlock] = blk_anchor * kLog2e;
    float rmax = -INFINITY, cmax = -INFINITY;  // of the values stored below
    float mv[kScanPer], rv[kScanPer], cv[kScanPer];
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
      const int64_t p = p0 + e;
      cs += double(fb[e]);
      m = fmax(m + double(fb[e]), double(iv[e]));
      const double loc = cs - blk_anchor;
      if (p < T) {
        mv[e] = float(m);
        rv[e] = float((loc - m - half_ln_d) * kLog2e);
        cv[e] = float((double(iv[e]) - loc) * kLog2e);
        rmax = fmaxf(rmax, rv[e]);
        cmax = fmaxf(cmax, cv[e]);
      } else {  // padding up to Tp
        mv[e] = 0.0f;
        rv[e] = 0.0f;
        cv[e] = -INFINITY;
        rmax = fmaxf(rmax, 0.0f);
      }
    }
    // tile bounds: the 8 threads of a 32-position tile are 8 consecutive lanes
    rmax = fmaxf(rmax, __shfl_xor(rmax, 1, 64));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 2, 64));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 4, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 1, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 2, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 4, 64));
    // the key factor of the factored exponent, relative to its tile's maximum
    float xv[kScanPer];
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) xv[e] = p0 + e < T ? exp2f(cv[e] - cmax) : 0.0f;
    if (p0 < Tp) {  // Tp is a multiple of 128: the 4 positions are all below it
      *reinterpret_cast<float4*>(rt + p0) = make_float4(rv[0], rv[1], rv[2], rv[3]);
      *reinterpret_cast<float4*>(ct + p0) = make_float4(cv[0], cv[1], cv[2], cv[3]);
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
    carry_cs += tot_sum;
    carry_m = apply(tot_map, carry_m);
    __syncthreads();  // s_* are rewritten by the next chunk
  }
}

}  // namespace

hipError_t launch_gate_scan(const float* igate, const float* fgate, float* m_out,
                            const Workspace& ws, int64_t H, int64_t T, int64_t d,
                            bool exp_forget, hipStream_t stream) {
  hipLaunchKernelGGL(gate_scan_kernel, dim3(unsigned(H)), dim3(kScanThreads), 0, stream, igate,
                     fgate, m_out, ws.anchor, ws.rowt, ws.colt, ws.colx, ws.rowb, ws.keyb, T, ws.Tp,
                     ws.nblk,
                     0.5 * log(double(d)), int(exp_forget));
  return hipGetLastError();
}

}  // namespace mlstm
