// The gate scan's building blocks, shared by the gate-scan kernels and the
// tile kernel that scans its own head's gates in its prologue, so that both
// evaluate the same arithmetic in the same order:
//
//   fbar_k = log sigmoid(f~_k)   (f~_k for an exponential forget gate) (Eq. 101)
//   m_i    = max_{j<=i} (sum_{k=j+1..i} fbar_k + i~_j)          (Eqs. 79, 80)
//
// m is evaluated through the recurrence m_i = max(m_{i-1} + fbar_i, i~_i),
// m_0 = i~_0, obtained by splitting j = i (where log F_ii = 0, so
// D~_ii = i~_i) from j < i (where D~_ij = fbar_i + D~_{i-1,j}).  Each step is
// the map x -> max(x + a, b); composing two such maps gives another,
// (a1, b1) then (a2, b2) = (a1 + a2, max(b1 + a2, b2)), so the recurrence is an
// associative scan.  The shift a of a composed map is the sum of fbar over its
// positions, so the same scan also yields the prefix sums cs of fbar.  A
// workgroup of 512 threads scans 2048 positions, 4 consecutive ones per
// thread; sums and maps are carried in float64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlstm {
namespace scan {

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

// log1p(u) for u in [0, 1], in float32: with s = u / (2 + u), in [0, 1/3],
// log1p(u) = log((1 + s) / (1 - s)) = 2 atanh(s) = 2 (s + s^3/3 + s^5/5 + ...);
// the series is cut after s^17 (the next term is below 2^-32 of the sum).
// The quotient is refined by one Newton step of the reciprocal and one
// residual correction.  Measured against a float64 reference over 6 M
// arguments (x on a grid over [-40, 40] and drawn from the gate laws of the
// named workloads): at most 2.8 units in the last place, mean error within
// 2e-10 of zero (the library's log1pf: at most 1.7 units) for a quarter of its
// instructions.
__device__ inline float log1p_unit(float u) {
  const float den = 2.0f + u;
  float r = __builtin_amdgcn_rcpf(den);
  r = fmaf(fmaf(-den, r, 1.0f), r, r);
  float s = u * r;
  s = fmaf(fmaf(-s, den, u), r, s);
  const float z = s * s;
  float p = 1.0f / 17.0f;
  p = fmaf(p, z, 1.0f / 15.0f);
  p = fmaf(p, z, 1.0f / 13.0f);
  p = fmaf(p, z, 1.0f / 11.0f);
  p = fmaf(p, z, 1.0f / 9.0f);
  p = fmaf(p, z, 1.0f / 7.0f);
  p = fmaf(p, z, 1.0f / 5.0f);
  p = fmaf(p, z, 1.0f / 3.0f);
  return fmaf(2.0f * s, z * p, 2.0f * s);
}

// log sigmoid(x) = min(x, 0) - log1p(exp(-|x|)): never forms exp(+|x|).  The
// first term is exact; the second, in (0, ln 2], is evaluated in float32 and
// subtracted in float64.
__device__ inline double log_sigmoid(float x) {
  return double(fminf(x, 0.0f)) - double(log1p_unit(expf(-fabsf(x))));
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

// Inclusive scan of one element per lane across a wave: row shifts of 1, 2,
// 4, 8 lanes, then the row totals by the two row broadcasts (DPP moves, no
// LDS).
__device__ inline Elem wave_inclusive(Elem x) {
  Elem incl = x;
  incl = combine(dpp_elem<kRowShr + 1, 0xF>(incl), incl);
  incl = combine(dpp_elem<kRowShr + 2, 0xF>(incl), incl);
  incl = combine(dpp_elem<kRowShr + 4, 0xF>(incl), incl);
  incl = combine(dpp_elem<kRowShr + 8, 0xF>(incl), incl);
  incl = combine(dpp_elem<kRowBcast15, 0xA>(incl), incl);
  incl = combine(dpp_elem<kRowBcast31, 0xC>(incl), incl);
  return incl;
}

// Ordered scan of one element per thread over the workgroup (thread order):
// returns the composition of the elements of all earlier threads and stores
// that of all threads in `total`.  Within a wave by wave_inclusive; across
// the waves, in order through LDS.
__device__ inline Elem block_scan(Elem x, Elem& total) {
  __shared__ double s_a[kScanWaves];
  __shared__ double s_b[kScanWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const Elem incl = wave_inclusive(x);
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

// block_scan over kScanThreads elements run by a workgroup of half as many
// threads: thread t holds the elements x0 and x1 of threads t and
// t + kScanThreads / 2 of the full block and receives what block_scan gives
// those two threads (before0, before1) and the total, bit for bit: the same
// combinations in the same order.
__device__ inline void block_scan_halves(Elem x0, Elem x1, Elem& before0, Elem& before1,
                                         Elem& total) {
  __shared__ double s_a[kScanWaves];
  __shared__ double s_b[kScanWaves];
  constexpr int kHalf = kScanWaves / 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;  // 0 .. kHalf - 1
  const Elem incl0 = wave_inclusive(x0);
  const Elem incl1 = wave_inclusive(x1);
  if (lane == 63) {
    s_a[wave] = incl0.a;
    s_b[wave] = incl0.b;
    s_a[wave + kHalf] = incl1.a;
    s_b[wave + kHalf] = incl1.b;
  }
  __syncthreads();
  Elem b0 = identity(), b1 = identity();
  total = identity();
  for (int w = 0; w < kScanWaves; ++w) {
    const Elem e = {s_a[w], s_b[w]};
    if (w < wave) b0 = combine(b0, e);
    if (w < wave + kHalf) b1 = combine(b1, e);
    total = combine(total, e);
  }
  const Elem lexcl0 = dpp_elem<kWaveShr1, 0xF>(incl0);
  const Elem lexcl1 = dpp_elem<kWaveShr1, 0xF>(incl1);
  __syncthreads();
  before0 = combine(b0, lexcl0);
  before1 = combine(b1, lexcl1);
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

// The per-position terms of a thread's 4 positions p0 .. p0 + 3, from the
// composition of everything before its chunk (`carry`) and of the chunk's
// positions before them (`before`): m (Eq. 80, rounded to
// float32), R_i = (cs_i - m_i - ln(d)/2) log2(e), C_j = (i~_j - cs_j) log2(e)
// (float64), e_j = 2^fl32(C_j - keyb) with keyb the maximum of C over the
// position's 32-position tile, and the tile maxima rmax (of R) and cmax (of
// C).  Positions past T are padding: m = 0, R = 0, C = -inf, e = 0.  Every
// lane of the wave must call it (the tile maxima are reduced across 8 lanes).
struct Terms {
  float m[kScanPer];
  double r[kScanPer];
  double c[kScanPer];
  float e[kScanPer];
  double rmax, cmax;
};

__device__ inline void position_terms(Elem carry, Elem before, const double fb[kScanPer],
                                      const float iv[kScanPer], int64_t p0, int64_t T,
                                      double half_ln_d, Terms& out) {
  const double kLog2e = 1.4426950408889634074;
  double cs = carry.a + before.a;                     // sum of fbar before p0
  double m = apply(before, apply(carry, -INFINITY));  // m at p0 - 1
  double rmax = -INFINITY, cmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < kScanPer; ++e) {
    const int64_t p = p0 + e;
    cs += fb[e];
    m = fmax(m + fb[e], double(iv[e]));
    if (p < T) {
      out.m[e] = float(m);
      out.r[e] = (cs - m - half_ln_d) * kLog2e;
      out.c[e] = (double(iv[e]) - cs) * kLog2e;
      rmax = fmax(rmax, out.r[e]);
      cmax = fmax(cmax, out.c[e]);
    } else {  // padding
      out.m[e] = 0.0f;
      out.r[e] = 0.0;
      out.c[e] = -INFINITY;
      rmax = fmax(rmax, 0.0);
    }
  }
  // tile maxima: the 8 threads of a 32-position tile are 8 consecutive lanes
  rmax = fmax(rmax, __shfl_xor(rmax, 1, 64));
  rmax = fmax(rmax, __shfl_xor(rmax, 2, 64));
  rmax = fmax(rmax, __shfl_xor(rmax, 4, 64));
  cmax = fmax(cmax, __shfl_xor(cmax, 1, 64));
  cmax = fmax(cmax, __shfl_xor(cmax, 2, 64));
  cmax = fmax(cmax, __shfl_xor(cmax, 4, 64));
  // the key factor of the factored exponent, relative to its tile's maximum:
  // the difference is formed in float64 and rounded once
#pragma unroll
  for (int e = 0; e < kScanPer; ++e) out.e[e] = p0 + e < T ? exp2f(float(out.c[e] - cmax)) : 0.0f;
  out.rmax = rmax;
  out.cmax = cmax;
}

}  // namespace scan
}  // namespace mlstm
