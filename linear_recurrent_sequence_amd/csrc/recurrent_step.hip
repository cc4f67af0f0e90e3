// One step of the recurrent mLSTM for generation, with stabilized states.
//
// The recurrent form (xLSTM appendix A.3; its forward equations are those the
// recurrent backward pass differentiates, Eqs. 59-70) keeps, per head, a
// d x d matrix memory C and a normalizer vector n.  Their stabilized versions
// are the unstabilized states scaled by exp(-m_t), where m_t is the running
// maximum of the log gates -- the same recurrence that gives the parallel
// form's row maximum (Eq. 80):
//
//   fbar_t = log sigmoid(f~_t)  (or f~_t for an exponential forget gate, Eq. 101)
//   m_t    = max(fbar_t + m_{t-1}, i~_t),   m_0 = -inf
//   f'_t   = exp(fbar_t + m_{t-1} - m_t),   i'_t = exp(i~_t - m_t)
//   C_t    = f'_t C_{t-1} + i'_t v_t k'_t^T,  k'_t = k_t / sqrt(d)
//   n_t    = f'_t n_{t-1} + i'_t k'_t
//   h~_t   = C_t q_t / max(|n_t . q_t|, exp(-m_t))           (Eqs. 84-86 for row t)
//
// The step reads and writes the whole state, d^2 + d + 1 floats per head, so
// it is bound by memory bandwidth.  One workgroup owns 16 rows of one head's
// C (rows are indexed by the value dimension, so h~_i = C_i . q); each wave
// owns 4 rows and each lane strided pairs of columns (4 pairs for d <= 512,
// 8 up to 1024).  A wave loads all of
// its rows before it stores any, so C may be updated in place.  Every
// workgroup forms n_t . q_t itself (d terms); the first workgroup of a head
// writes n_t and m_t.  Reductions are fixed-order butterflies: results are
// bitwise reproducible.
#include "mlstm_internal.h"

#include <hip/hip_bf16.h>

namespace mlstm {
namespace {

constexpr int kStepThreads = 256;
constexpr int kStepWaves = kStepThreads / 64;
constexpr int kRowsPerWave = 4;
constexpr int kStepRows = kStepWaves * kRowsPerWave;  // rows of C per workgroup

__device__ inline float load_elem(const float* p) { return *p; }
__device__ inline float load_elem(const __hip_bfloat16* p) { return __bfloat162float(*p); }
__device__ inline float2 load_pair(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ inline float2 load_pair(const __hip_bfloat16* p) {
  const __hip_bfloat162 x = *reinterpret_cast<const __hip_bfloat162*>(p);
  return make_float2(__low2float(x), __high2float(x));
}
__device__ inline void store_elem(float* p, float x) { *p = x; }
__device__ inline void store_elem(__hip_bfloat16* p, float x) { *p = __float2bfloat16(x); }

// log sigmoid(x) = min(x, 0) - log1p(exp(-|x|)): never forms exp(+|x|).
__device__ inline float log_sigmoid(float x) { return fminf(x, 0.0f) - log1pf(expf(-fabsf(x))); }

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <typename Tin, int kPairsPerLane>  // d <= 128 * kPairsPerLane
__global__ __launch_bounds__(kStepThreads) void recurrent_step_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ igate, const float* __restrict__ fgate, const float* C_in,
    const float* __restrict__ n_in, const float* __restrict__ m_in, float* C_out,
    float* __restrict__ n_out, float* __restrict__ m_out, Tin* __restrict__ h_out,
    float* __restrict__ den_out, int d, int blocks_per_head, int exp_forget) {
  const int64_t head = blockIdx.x / blocks_per_head;
  const int rb = blockIdx.x % blocks_per_head;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int npairs = d / 2;

  // gates and stabilizer
  const float fbar = exp_forget ? fgate[head] : log_sigmoid(fgate[head]);  // log f_t
  const float ig = igate[head];
  const float m_old = m_in[head];
  const float m_new = fmaxf(fbar + m_old, ig);
  const float f_p = m_old == -INFINITY ? 0.0f : expf(fbar + m_old - m_new);
  const float i_p = expf(ig - m_new);
  const float kscale = rsqrtf(float(d));

  // this lane's columns: pairs p = lane + 64 u
  const int64_t vec = head * int64_t(d);
  float2 qv[kPairsPerLane], kv[kPairsPerLane], nv[kPairsPerLane];
  float b = 0.0f;
#pragma unroll
  for (int u = 0; u < kPairsPerLane; ++u) {
    const int p = lane + 64 * u;
    qv[u] = kv[u] = nv[u] = make_float2(0.0f, 0.0f);
    if (p < npairs) {
      qv[u] = load_pair(q + vec + 2 * p);
      const float2 kk = load_pair(k + vec + 2 * p);
      kv[u] = make_float2(kk.x * kscale, kk.y * kscale);
      const float2 no = load_pair(n_in + vec + 2 * p);
      nv[u] = make_float2(f_p * no.x + i_p * kv[u].x, f_p * no.y + i_p * kv[u].y);
      b += nv[u].x * qv[u].x + nv[u].y * qv[u].y;
    }
  }
  b = wave_sum(b);  // n_t . q_t
  const float den = fmaxf(fabsf(b), expf(-m_new));
  const float inv = 1.0f / den;
  if (rb == 0 && w == 0) {
#pragma unroll
    for (int u = 0; u < kPairsPerLane; ++u) {
      const int p = lane + 64 * u;
      if (p < npairs) *reinterpret_cast<float2*>(n_out + vec + 2 * p) = nv[u];
    }
    if (lane == 0) {
      m_out[head] = m_new;
      if (den_out) den_out[head] = den;
    }
  }

  // this wave's rows: load them all, then update, store, and reduce
  const int row0 = rb * kStepRows + w * kRowsPerWave;
  float2 cr[kRowsPerWave][kPairsPerLane];
  float vi[kRowsPerWave];
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int i = row0 + rr;
    vi[rr] = 0.0f;
#pragma unroll
    for (int u = 0; u < kPairsPerLane; ++u) cr[rr][u] = make_float2(0.0f, 0.0f);
    if (i < d) {
      vi[rr] = load_elem(v + vec + i);
      const float* crow = C_in + (vec + i) * d;
#pragma unroll
      for (int u = 0; u < kPairsPerLane; ++u) {
        const int p = lane + 64 * u;
        if (p < npairs) cr[rr][u] = *reinterpret_cast<const float2*>(crow + 2 * p);
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int i = row0 + rr;
    if (i >= d) break;  // uniform across the wave
    const float a = i_p * vi[rr];
    float* orow = C_out + (vec + i) * d;
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < kPairsPerLane; ++u) {
      const int p = lane + 64 * u;
      if (p < npairs) {
        const float2 c = make_float2(f_p * cr[rr][u].x + a * kv[u].x,
                                     f_p * cr[rr][u].y + a * kv[u].y);
        *reinterpret_cast<float2*>(orow + 2 * p) = c;
        acc += c.x * qv[u].x + c.y * qv[u].y;
      }
    }
    acc = wave_sum(acc);  // C_t q_t, row i
    if (lane == 0) store_elem(h_out + vec + i, acc * inv);
  }
}

template <typename Tin, int P>
void launch_r(const void* q, const void* k, const void* v, const float* igate, const float* fgate,
              const float* C_in, const float* n_in, const float* m_in, float* C_out,
              float* n_out, float* m_out, void* h_out, float* den_out, int64_t H, int64_t d,
              bool exp_forget, hipStream_t stream) {
  const int blocks_per_head = int((d + kStepRows - 1) / kStepRows);
  hipLaunchKernelGGL((recurrent_step_kernel<Tin, P>), dim3(unsigned(H * blocks_per_head)),
                     dim3(kStepThreads), 0, stream, static_cast<const Tin*>(q),
                     static_cast<const Tin*>(k), static_cast<const Tin*>(v), igate, fgate, C_in,
                     n_in, m_in, C_out, n_out, m_out, static_cast<Tin*>(h_out), den_out, int(d),
                     blocks_per_head, int(exp_forget));
}

}  // namespace

hipError_t launch_recurrent_step(const void* q, const void* k, const void* v, const float* igate,
                                 const float* fgate, const float* C_in, const float* n_in,
                                 const float* m_in, float* C_out, float* n_out, float* m_out,
                                 void* h_out, float* den_out, int64_t H, int64_t d, bool is_bf16,
                                 bool exp_forget, hipStream_t stream) {
  if (d % 16 != 0 || d < 16 || d > 1024) return hipErrorInvalidValue;
  using B16 = __hip_bfloat16;
  if (is_bf16) {
    if (d <= 512)
      launch_r<B16, 4>(q, k, v, igate, fgate, C_in, n_in, m_in, C_out, n_out, m_out, h_out,
                       den_out, H, d, exp_forget, stream);
    else
      launch_r<B16, 8>(q, k, v, igate, fgate, C_in, n_in, m_in, C_out, n_out, m_out, h_out,
                       den_out, H, d, exp_forget, stream);
  } else {
    if (d <= 512)
      launch_r<float, 4>(q, k, v, igate, fgate, C_in, n_in, m_in, C_out, n_out, m_out, h_out,
                         den_out, H, d, exp_forget, stream);
    else
      launch_r<float, 8>(q, k, v, igate, fgate, C_in, n_in, m_in, C_out, n_out, m_out, h_out,
                         den_out, H, d, exp_forget, stream);
  }
  return hipGetLastError();
}

}  // namespace mlstm
