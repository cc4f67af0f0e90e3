// Backward pass of the stabilized parallel mLSTM (xLSTM appendix A.3,
// "Parallel mLSTM Backward Pass", Eqs. 87-105), float32 vector-ALU tiles.
//
// With E_ij = D'_ij / sqrt(d) (the same exponent terms the forward tile
// kernels use), s_ij = q_i . k_j and g_ij = dh_i . v_j, the equations
// reduce per causal entry (j <= i) to
//
//   C~'_ij = s_ij E_ij                                            (Eq. 82)
//   dC~'_ij = g_ij / n_i + db_i                                   (Eqs. 87, 91-93)
//   dn_i   = -(dh_i . h~_i) / n_i                                 (Eqs. 88-89: sum_j C~'_ij v_j = n_i h~_i)
//   db_i   = sign(b_i) [|b_i| > exp(-m_i)] dn_i                   (Eq. 90, with the derivative of |b|)
//   dQ_i   = sum_j E_ij dC~'_ij k_j                               (Eq. 98)
//   dK_j   = sum_i E_ij dC~'_ij q_i                               (Eq. 99)
//   dV_j   = sum_i (C~'_ij / n_i) dh_i                            (Eq. 100)
//   dD~_ij = C~'_ij dC~'_ij                                       (Eqs. 94-95)
//   di~_j  = sum_i dD~_ij                                         (Eqs. 97, 105)
//   dfbar_k = sum_{j<k<=i} dD~_ij = sum_{i>=k} (r_i - c_i)        (Eqs. 96, 102)
//   df~_k  = sigma(-f~_k) dfbar_k  (dfbar_k for an exponential gate) (Eqs. 103, 104)
//
// with r_i = sum_j dD~_ij and c_j = di~_j: splitting the sum over i >= k of
// the row sums r_i into the entries with j < k (Eq. 102) and those with
// j >= k (the column sums c_j, j >= k) turns the double sum into a reverse
// cumulative sum.  m is held constant (its contributions cancel).
//
// Four kernels: per-row scalars (1/n and db), a row pass (dQ and r, one
// workgroup per 16 query rows), a column pass (dK, dV and c, one workgroup
// per 16 keys), and a per-head reverse scan for the gate gradients.  Every
// reduction has a fixed order: results are bitwise reproducible.  For bf16
// inputs the row and column passes run on the matrix cores instead
// (backward_mfma.hip, whose rows pass also forms the per-row scalars); the
// gate-gradient scan is shared.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "mlstm_internal.h"

#include <hip/hip_bf16.h>

namespace mlstm {
namespace {

constexpr int kBT = 16;    // rows and keys per tile
constexpr int kBMaxD = 512;  // the row and column passes hold whole rows in LDS up to here
constexpr int kBPad = kBMaxD + 1;
// above kBMaxD (up to kBackwardMaxHeadDim) the wide passes take the head
// dimension in LDS chunks of kWC columns
constexpr int kWC = 256;
constexpr int kWChunks = kBackwardMaxHeadDim / kWC;
constexpr int kWPer = kWC / kBT;  // accumulator columns per thread and chunk

__device__ inline float load_elem(const float* p) { return *p; }
__device__ inline float load_elem(const __hip_bfloat16* p) { return __bfloat162float(*p); }
__device__ inline void store_elem(float* p, float x) { *p = x; }
__device__ inline void store_elem(__hip_bfloat16* p, float x) { *p = __float2bfloat16(x); }

// E_ij = D'_ij / sqrt(d) = 2^(R_i + C_j) from the gate-scan terms, the
// exponent summed in float64 and rounded once (0 above the diagonal or past
// the sequence end)
__device__ inline float gate_factor(double r_i, double c_j, bool valid) {
  return valid ? exp2f(float(r_i + c_j)) : 0.0f;
}

// 1/n_i and db_i, one wave per row
template <typename Tin>
__global__ __launch_bounds__(256) void bwd_rows_prep_kernel(
    const Tin* __restrict__ h, const Tin* __restrict__ dh, const float* __restrict__ m,
    const float* __restrict__ n, const float* __restrict__ b, float* __restrict__ inv_n,
    float* __restrict__ db, int64_t rows, int d) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  // the row's scalars are loaded with its vectors, so that their latencies overlap
  const float nn = n[row], bb = b[row], mm = m[row];
  float acc = 0.0f;
  if constexpr (std::is_same<Tin, float>::value) {  // 16 bytes per lane (d % 16 == 0)
    for (int c = 4 * lane; c < d; c += 256) {
      const float4 x = *reinterpret_cast<const float4*>(dh + row * d + c);
      const float4 y = *reinterpret_cast<const float4*>(h + row * d + c);
      acc += x.x * y.x;
      acc += x.y * y.y;
      acc += x.z * y.z;
      acc += x.w * y.w;
    }
  } else {
    for (int c = lane; c < d; c += 64) acc += load_elem(dh + row * d + c) * load_elem(h + row * d + c);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) {
    const float dn = -acc / nn;
    const bool above_floor = fabsf(bb) > expf(-mm);
    inv_n[row] = 1.0f / nn;
    db[row] = above_floor ? (bb > 0.0f ? dn : (bb < 0.0f ? -dn : 0.0f)) : 0.0f;
  }
}

// Row pass: dQ for 16 query rows and r_i = sum_j dD~_ij.  Thread (rl, cl) of
// the 16 x 16 grid forms entry (i = q0 + rl, j = k0 + cl) of each key tile,
// then accumulates columns cl, cl + 16, ... of dQ row rl.
template <typename Tin>
__global__ __launch_bounds__(256) void bwd_rows_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ dh, const float* __restrict__ inv_n, const float* __restrict__ db,
    const double* __restrict__ rowt, const double* __restrict__ colt, Tin* __restrict__ dq,
    float* __restrict__ rsum, int64_t T, int d, int64_t Tp, int64_t row_tiles) {
  __shared__ float Qs[kBT][kBPad];
  __shared__ float Gs[kBT][kBPad];  // dh rows
  __shared__ float Ks[kBT][kBPad];
  __shared__ float Vs[kBT][kBPad];
  __shared__ float Ps[kBT][kBT + 1];  // E dC~'

  const int tid = threadIdx.x;
  const int rl = tid / kBT, cl = tid % kBT;
  const int64_t head = blockIdx.x / row_tiles;
  const int64_t q0 = (blockIdx.x % row_tiles) * kBT;
  const int64_t qi = q0 + rl;
  const int64_t hoff = head * T * int64_t(d);
  for (int idx = tid; idx < kBT * d; idx += 256) {
    const int r = idx / d, c = idx % d;
    const bool in = q0 + r < T;
    Qs[r][c] = in ? load_elem(q + hoff + (q0 + r) * d + c) : 0.0f;
    Gs[r][c] = in ? load_elem(dh + hoff + (q0 + r) * d + c) : 0.0f;
  }
  const bool row_in = qi < T;
  const double r_i = rowt[head * Tp + qi];
  const float in_i = row_in ? inv_n[head * T + qi] : 0.0f;
  const float db_i = row_in ? db[head * T + qi] : 0.0f;

  float acc[kBMaxD / kBT];
#pragma unroll
  for (int u = 0; u < kBMaxD / kBT; ++u) acc[u] = 0.0f;
  float rs = 0.0f;

  const int64_t last_key = (q0 + kBT - 1 < T ? q0 + kBT - 1 : T - 1);
  for (int64_t k0 = 0; k0 <= last_key; k0 += kBT) {
    __syncthreads();
    for (int idx = tid; idx < kBT * d; idx += 256) {
      const int r = idx / d, c = idx % d;
      const bool in = k0 + r < T;
      Ks[r][c] = in ? load_elem(k + hoff + (k0 + r) * d + c) : 0.0f;
      Vs[r][c] = in ? load_elem(v + hoff + (k0 + r) * d + c) : 0.0f;
    }
    __syncthreads();
    const int64_t kj = k0 + cl;
    float s = 0.0f, gg = 0.0f;
    for (int c = 0; c < d; ++c) {
      s = fmaf(Qs[rl][c], Ks[cl][c], s);
      gg = fmaf(Gs[rl][c], Vs[cl][c], gg);
    }
    const bool valid = row_in && kj <= qi && kj < T;
    const float e = gate_factor(r_i, colt[head * Tp + kj], valid);
    const float dct = gg * in_i + db_i;  // dC~' (Eqs. 91-93)
    rs += (s * e) * dct;                 // dD~ = C~' dC~' (Eq. 95)
    Ps[rl][cl] = e * dct;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kBMaxD / kBT; ++u) {
      const int c = cl + kBT * u;
      if (c < d) {
        float a = 0.0f;
#pragma unroll
        for (int t = 0; t < kBT; ++t) a = fmaf(Ps[rl][t], Ks[t][c], a);
        acc[u] += a;
      }
    }
  }
  // the 16 threads of a row are 16 consecutive lanes
#pragma unroll
  for (int off = kBT / 2; off > 0; off >>= 1) rs += __shfl_xor(rs, off, 64);
  if (row_in) {
    if (cl == 0) rsum[head * T + qi] = rs;
#pragma unroll
    for (int u = 0; u < kBMaxD / kBT; ++u) {
      const int c = cl + kBT * u;
      if (c < d) store_elem(dq + hoff + qi * d + c, acc[u]);  // Eq. 98
    }
  }
}

// Column pass: dK and dV for 16 keys and c_j = sum_i dD~_ij.  Thread
// (kl, cl) forms entry (i = q0 + cl, j = k0 + kl) of each query tile, then
// accumulates columns cl, cl + 16, ... of dK and dV row kl.
template <typename Tin>
__global__ __launch_bounds__(256) void bwd_cols_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ dh, const float* __restrict__ inv_n, const float* __restrict__ db,
    const double* __restrict__ rowt, const double* __restrict__ colt, Tin* __restrict__ dk,
    Tin* __restrict__ dv, float* __restrict__ csum, int64_t T, int d, int64_t Tp,
    int64_t key_tiles) {
  __shared__ float Ks[kBT][kBPad];
  __shared__ float Vs[kBT][kBPad];
  __shared__ float Qs[kBT][kBPad];
  __shared__ float Gs[kBT][kBPad];
  __shared__ float Ps[kBT][kBT + 1];  // E dC~' (key-major)
  __shared__ float Ns[kBT][kBT + 1];  // C~' / n (key-major)

  const int tid = threadIdx.x;
  const int kl = tid / kBT, cl = tid % kBT;
  const int64_t head = blockIdx.x / key_tiles;
  const int64_t k0 = (blockIdx.x % key_tiles) * kBT;
  const int64_t kj = k0 + kl;
  const int64_t hoff = head * T * int64_t(d);
  for (int idx = tid; idx < kBT * d; idx += 256) {
    const int r = idx / d, c = idx % d;
    const bool in = k0 + r < T;
    Ks[r][c] = in ? load_elem(k + hoff + (k0 + r) * d + c) : 0.0f;
    Vs[r][c] = in ? load_elem(v + hoff + (k0 + r) * d + c) : 0.0f;
  }
  const bool key_in = kj < T;
  const double c_j = colt[head * Tp + kj];  // kj < Tp

  float acck[kBMaxD / kBT], accv[kBMaxD / kBT];
#pragma unroll
  for (int u = 0; u < kBMaxD / kBT; ++u) acck[u] = accv[u] = 0.0f;
  float cs = 0.0f;

  for (int64_t q0 = k0; q0 < T; q0 += kBT) {
    __syncthreads();
    for (int idx = tid; idx < kBT * d; idx += 256) {
      const int r = idx / d, c = idx % d;
      const bool in = q0 + r < T;
      Qs[r][c] = in ? load_elem(q + hoff + (q0 + r) * d + c) : 0.0f;
      Gs[r][c] = in ? load_elem(dh + hoff + (q0 + r) * d + c) : 0.0f;
    }
    __syncthreads();
    const int64_t qi = q0 + cl;
    const bool row_in = qi < T;
    float s = 0.0f, gg = 0.0f;
    for (int c = 0; c < d; ++c) {
      s = fmaf(Qs[cl][c], Ks[kl][c], s);
      gg = fmaf(Gs[cl][c], Vs[kl][c], gg);
    }
    const bool valid = key_in && row_in && kj <= qi;
    const double r_i = rowt[head * Tp + (row_in ? qi : 0)];
    const float e = gate_factor(r_i, c_j, valid);
    const float in_i = row_in ? inv_n[head * T + qi] : 0.0f;
    const float db_i = row_in ? db[head * T + qi] : 0.0f;
    const float dct = gg * in_i + db_i;
    const float ct = s * e;
    cs += ct * dct;
    Ps[kl][cl] = e * dct;
    Ns[kl][cl] = ct * in_i;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kBMaxD / kBT; ++u) {
      const int c = cl + kBT * u;
      if (c < d) {
        float a = 0.0f, bsum = 0.0f;
#pragma unroll
        for (int t = 0; t < kBT; ++t) {
          a = fmaf(Ps[kl][t], Qs[t][c], a);
          bsum = fmaf(Ns[kl][t], Gs[t][c], bsum);
        }
        acck[u] += a;
        accv[u] += bsum;
      }
    }
  }
#pragma unroll
  for (int off = kBT / 2; off > 0; off >>= 1) cs += __shfl_xor(cs, off, 64);
  if (key_in) {
    if (cl == 0) csum[head * T + kj] = cs;
#pragma unroll
    for (int u = 0; u < kBMaxD / kBT; ++u) {
      const int c = cl + kBT * u;
      if (c < d) {
        store_elem(dk + hoff + kj * d + c, acck[u]);  // Eq. 99
        store_elem(dv + hoff + kj * d + c, accv[u]);  // Eq. 100
      }
    }
  }
}

// The row pass for kBMaxD < d <= kBackwardMaxHeadDim: the same entries and
// sums in the same order, with the head dimension in LDS chunks of kWC
// columns.  The dot products s_ij and g_ij run over the chunks in turn (each
// chunk of the tile's Q, dH, K and V rows staged once per key tile); the dQ
// columns of each chunk accumulate from that chunk of K, staged again.
template <typename Tin>
__global__ __launch_bounds__(256) void bwd_rows_wide_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ dh, const float* __restrict__ inv_n, const float* __restrict__ db,
    const double* __restrict__ rowt, const double* __restrict__ colt, Tin* __restrict__ dq,
    float* __restrict__ rsum, int64_t T, int d, int64_t Tp, int64_t row_tiles) {
  __shared__ float Qs[kBT][kWC + 1];
  __shared__ float Gs[kBT][kWC + 1];  // dh rows
  __shared__ float Ks[kBT][kWC + 1];
  __shared__ float Vs[kBT][kWC + 1];
  __shared__ float Ps[kBT][kBT + 1];  // E dC~'

  const int tid = threadIdx.x;
  const int rl = tid / kBT, cl = tid % kBT;
  const int64_t head = blockIdx.x / row_tiles;
  const int64_t q0 = (blockIdx.x % row_tiles) * kBT;
  const int64_t qi = q0 + rl;
  const int64_t hoff = head * T * int64_t(d);
  const bool row_in = qi < T;
  const double r_i = rowt[head * Tp + qi];  // qi < Tp
  const float in_i = row_in ? inv_n[head * T + qi] : 0.0f;
  const float db_i = row_in ? db[head * T + qi] : 0.0f;

  float acc[kWChunks * kWPer];
#pragma unroll
  for (int u = 0; u < kWChunks * kWPer; ++u) acc[u] = 0.0f;
  float rs = 0.0f;

  const int64_t last_key = (q0 + kBT - 1 < T ? q0 + kBT - 1 : T - 1);
  for (int64_t k0 = 0; k0 <= last_key; k0 += kBT) {
    float s = 0.0f, gg = 0.0f;
#pragma unroll
    for (int ch = 0; ch < kWChunks; ++ch) {
      const int c0 = ch * kWC;
      if (c0 < d) {
        const int wc = d - c0 < kWC ? d - c0 : kWC;
        __syncthreads();
        for (int idx = tid; idx < kBT * wc; idx += 256) {
          const int r = idx / wc, c = idx % wc;
          const bool qin = q0 + r < T, kin = k0 + r < T;
          Qs[r][c] = qin ? load_elem(q + hoff + (q0 + r) * d + c0 + c) : 0.0f;
          Gs[r][c] = qin ? load_elem(dh + hoff + (q0 + r) * d + c0 + c) : 0.0f;
          Ks[r][c] = kin ? load_elem(k + hoff + (k0 + r) * d + c0 + c) : 0.0f;
          Vs[r][c] = kin ? load_elem(v + hoff + (k0 + r) * d + c0 + c) : 0.0f;
        }
        __syncthreads();
        for (int c = 0; c < wc; ++c) {
          s = fmaf(Qs[rl][c], Ks[cl][c], s);
          gg = fmaf(Gs[rl][c], Vs[cl][c], gg);
        }
      }
    }
    const int64_t kj = k0 + cl;
    const bool valid = row_in && kj <= qi && kj < T;
    const float e = gate_factor(r_i, colt[head * Tp + kj], valid);
    const float dct = gg * in_i + db_i;  // dC~' (Eqs. 91-93)
    rs += (s * e) * dct;                 // dD~ = C~' dC~' (Eq. 95)
    Ps[rl][cl] = e * dct;
#pragma unroll
    for (int ch = 0; ch < kWChunks; ++ch) {
      const int c0 = ch * kWC;
      if (c0 < d) {
        const int wc = d - c0 < kWC ? d - c0 : kWC;
        __syncthreads();  // P is complete; every read of the previous chunk is done
        for (int idx = tid; idx < kBT * wc; idx += 256) {
          const int r = idx / wc, c = idx % wc;
          Ks[r][c] = k0 + r < T ? load_elem(k + hoff + (k0 + r) * d + c0 + c) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kWPer; ++u) {
          const int c = cl + kBT * u;
          if (c < wc) {
            float a = 0.0f;
#pragma unroll
            for (int t = 0; t < kBT; ++t) a = fmaf(Ps[rl][t], Ks[t][c], a);
            acc[ch * kWPer + u] += a;
          }
        }
      }
    }
  }
#pragma unroll
  for (int off = kBT / 2; off > 0; off >>= 1) rs += __shfl_xor(rs, off, 64);
  if (row_in) {
    if (cl == 0) rsum[head * T + qi] = rs;
#pragma unroll
    for (int ch = 0; ch < kWChunks; ++ch) {
#pragma unroll
      for (int u = 0; u < kWPer; ++u) {
        const int c = ch * kWC + cl + kBT * u;
        if (c < d) store_elem(dq + hoff + qi * d + c, acc[ch * kWPer + u]);  // Eq. 98
      }
    }
  }
}

// The column pass for kBMaxD < d <= kBackwardMaxHeadDim, in head-dimension
// chunks as the wide row pass.
template <typename Tin>
__global__ __launch_bounds__(256) void bwd_cols_wide_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ dh, const float* __restrict__ inv_n, const float* __restrict__ db,
    const double* __restrict__ rowt, const double* __restrict__ colt, Tin* __restrict__ dk,
    Tin* __restrict__ dv, float* __restrict__ csum, int64_t T, int d, int64_t Tp,
    int64_t key_tiles) {
  __shared__ float Ks[kBT][kWC + 1];
  __shared__ float Vs[kBT][kWC + 1];
  __shared__ float Qs[kBT][kWC + 1];
  __shared__ float Gs[kBT][kWC + 1];
  __shared__ float Ps[kBT][kBT + 1];  // E dC~' (key-major)
  __shared__ float Ns[kBT][kBT + 1];  // C~' / n (key-major)

  const int tid = threadIdx.x;
  const int kl = tid / kBT, cl = tid % kBT;
  const int64_t head = blockIdx.x / key_tiles;
  const int64_t k0 = (blockIdx.x % key_tiles) * kBT;
  const int64_t kj = k0 + kl;
  const int64_t hoff = head * T * int64_t(d);
  const bool key_in = kj < T;
  const double c_j = colt[head * Tp + kj];  // kj < Tp

  float acck[kWChunks * kWPer], accv[kWChunks * kWPer];
#pragma unroll
  for (int u = 0; u < kWChunks * kWPer; ++u) acck[u] = accv[u] = 0.0f;
  float cs = 0.0f;

  for (int64_t q0 = k0; q0 < T; q0 += kBT) {
    float s = 0.0f, gg = 0.0f;
#pragma unroll
    for (int ch = 0; ch < kWChunks; ++ch) {
      const int c0 = ch * kWC;
      if (c0 < d) {
        const int wc = d - c0 < kWC ? d - c0 : kWC;
        __syncthreads();
        for (int idx = tid; idx < kBT * wc; idx += 256) {
          const int r = idx / wc, c = idx % wc;
          const bool kin = k0 + r < T, qin = q0 + r < T;
          Ks[r][c] = kin ? load_elem(k + hoff + (k0 + r) * d + c0 + c) : 0.0f;
          Vs[r][c] = kin ? load_elem(v + hoff + (k0 + r) * d + c0 + c) : 0.0f;
          Qs[r][c] = qin ? load_elem(q + hoff + (q0 + r) * d + c0 + c) : 0.0f;
          Gs[r][c] = qin ? load_elem(dh + hoff + (q0 + r) * d + c0 + c) : 0.0f;
        }
        __syncthreads();
        for (int c = 0; c < wc; ++c) {
          s = fmaf(Qs[cl][c], Ks[kl][c], s);
          gg = fmaf(Gs[cl][c], Vs[kl][c], gg);
        }
      }
    }
    const int64_t qi = q0 + cl;
    const bool row_in = qi < T;
    const bool valid = key_in && row_in && kj <= qi;
    const double r_i = rowt[head * Tp + (row_in ? qi : 0)];
    const float e = gate_factor(r_i, c_j, valid);
    const float in_i = row_in ? inv_n[head * T + qi] : 0.0f;
    const float db_i = row_in ? db[head * T + qi] : 0.0f;
    const float dct = gg * in_i + db_i;
    const float ct = s * e;
    cs += ct * dct;
    Ps[kl][cl] = e * dct;
    Ns[kl][cl] = ct * in_i;
#pragma unroll
    for (int ch = 0; ch < kWChunks; ++ch) {
      const int c0 = ch * kWC;
      if (c0 < d) {
        const int wc = d - c0 < kWC ? d - c0 : kWC;
        __syncthreads();  // P and N are complete; every read of the previous chunk is done
        for (int idx = tid; idx < kBT * wc; idx += 256) {
          const int r = idx / wc, c = idx % wc;
          const bool qin = q0 + r < T;
          Qs[r][c] = qin ? load_elem(q + hoff + (q0 + r) * d + c0 + c) : 0.0f;
          Gs[r][c] = qin ? load_elem(dh + hoff + (q0 + r) * d + c0 + c) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kWPer; ++u) {
          const int c = cl + kBT * u;
          if (c < wc) {
            float a = 0.0f, bsum = 0.0f;
#pragma unroll
            for (int t = 0; t < kBT; ++t) {
              a = fmaf(Ps[kl][t], Qs[t][c], a);
              bsum = fmaf(Ns[kl][t], Gs[t][c], bsum);
            }
            acck[ch * kWPer + u] += a;
            accv[ch * kWPer + u] += bsum;
          }
        }
      }
    }
  }
#pragma unroll
  for (int off = kBT / 2; off > 0; off >>= 1) cs += __shfl_xor(cs, off, 64);
  if (key_in) {
    if (cl == 0) csum[head * T + kj] = cs;
#pragma unroll
    for (int ch = 0; ch < kWChunks; ++ch) {
#pragma unroll
      for (int u = 0; u < kWPer; ++u) {
        const int c = ch * kWC + cl + kBT * u;
        if (c < d) {
          store_elem(dk + hoff + kj * d + c, acck[ch * kWPer + u]);  // Eq. 99
          store_elem(dv + hoff + kj * d + c, accv[ch * kWPer + u]);  // Eq. 100
        }
      }
    }
  }
}

// Gate gradients for one head per workgroup: di~ = c (Eq. 105) and
// df~_k = sigma(-f~_k) sum_{i>=k} (r_i - c_i) (Eqs. 102-104), the suffix
// sums accumulated in float64 from the end of the sequence, one chunk of
// 256 x 8 positions at a time.
constexpr int kGThreads = 256;
constexpr int kGPer = 8;
__global__ __launch_bounds__(kGThreads) void bwd_gates_kernel(
    const float* __restrict__ fgate, const float* __restrict__ rsum,
    const float* __restrict__ csum, float* __restrict__ digate, float* __restrict__ dfgate,
    int64_t T, int exp_forget) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t head = blockIdx.x;
  const float* r = rsum + head * T;
  const float* c = csum + head * T;
  __shared__ double s_tot[kGThreads / 64];
  double carry = 0.0;  // sum over every later chunk
  const int64_t chunk = int64_t(kGThreads) * kGPer;
  for (int64_t end = T; end > 0; end -= chunk) {
    // thread tid owns positions end - 1 - (tid * kGPer + e), e = 0..7 (walking backwards)
    double x[kGPer];
    double tsum = 0.0;
#pragma unroll
    for (int e = 0; e < kGPer; ++e) {
      const int64_t p = end - 1 - (int64_t(tid) * kGPer + e);
      x[e] = p >= 0 ? double(r[p]) - double(c[p]) : 0.0;
      tsum += x[e];
    }
    // inclusive scan of the thread totals in the backward order
    double incl = tsum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) s_tot[wave] = incl;
    __syncthreads();
    double before = carry;
    for (int w = 0; w < wave; ++w) before += s_tot[w];
    double chunk_tot = 0.0;
    for (int w = 0; w < kGThreads / 64; ++w) chunk_tot += s_tot[w];
    double run = before + incl - tsum;  // sum over positions after this thread's first
#pragma unroll
    for (int e = 0; e < kGPer; ++e) {
      const int64_t p = end - 1 - (int64_t(tid) * kGPer + e);
      run += x[e];
      if (p >= 0) {
        const float f = fgate[head * T + p];
        // d(log f)/d f~: sigma(-f~) (Eq. 104), or 1 for the exponential gate
        const double dlogf = exp_forget ? 1.0 : 1.0 / (1.0 + exp(double(f)));
        // f_0 never enters F (Eq. 101): its sum is empty, exactly 0, where the
        // suffix form would leave the rounding of sum r - sum c
        dfgate[head * T + p] = p == 0 ? 0.0f : float(dlogf * run);
        digate[head * T + p] = c[p];
      }
    }
    carry += chunk_tot;
    __syncthreads();  // s_tot is rewritten by the next chunk
  }
}

template <typename Tin>
hipError_t launch_typed(const Tin* q, const Tin* k, const Tin* v, const float* fgate,
                        const Tin* h, const float* m, const float* n, const float* b,
                        const Tin* dh, const Workspace& ws, float* inv_n, float* db, float* rsum,
                        float* csum, void* vstore, Tin* dq, Tin* dk, Tin* dv, float* digate,
                        float* dfgate, int64_t H, int64_t T, int64_t d, bool exp_forget, bool mfma,
                        bool f32_tiles, hipStream_t stream) {
  if (mfma) {  // the rows pass forms the per-row scalars itself
    const hipError_t e = launch_backward_mfma_tiles(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq,
                                                    dk, dv, rsum, csum, vstore, H, T, d, stream);
    if (e != hipSuccess) return e;
  } else {
    const int64_t rows = H * T;
    hipLaunchKernelGGL(bwd_rows_prep_kernel<Tin>, dim3(unsigned((rows + 3) / 4)), dim3(256), 0,
                       stream, h, dh, m, n, b, inv_n, db, rows, int(d));
    const int64_t tiles = (T + kBT - 1) / kBT;
    if (f32_tiles) {  // float32 inputs only
      if constexpr (std::is_same<Tin, float>::value) {
        const hipError_t e = launch_backward_f32_tiles(q, k, v, dh, inv_n, db, ws, dq, dk, dv,
                                                       rsum, csum, H, T, d, stream);
        if (e != hipSuccess) return e;
      }
    } else if (d <= kBMaxD) {
      hipLaunchKernelGGL(bwd_rows_kernel<Tin>, dim3(unsigned(tiles * H)), dim3(256), 0, stream,
                         q, k, v, dh, inv_n, db, ws.rowt, ws.colt, dq, rsum, T, int(d), ws.Tp,
                         tiles);
      hipLaunchKernelGGL(bwd_cols_kernel<Tin>, dim3(unsigned(tiles * H)), dim3(256), 0, stream,
                         q, k, v, dh, inv_n, db, ws.rowt, ws.colt, dk, dv, csum, T, int(d),
                         ws.Tp, tiles);
    } else {
      hipLaunchKernelGGL(bwd_rows_wide_kernel<Tin>, dim3(unsigned(tiles * H)), dim3(256), 0,
                         stream, q, k, v, dh, inv_n, db, ws.rowt, ws.colt, dq, rsum, T, int(d),
                         ws.Tp, tiles);
      hipLaunchKernelGGL(bwd_cols_wide_kernel<Tin>, dim3(unsigned(tiles * H)), dim3(256), 0,
                         stream, q, k, v, dh, inv_n, db, ws.rowt, ws.colt, dk, dv, csum, T,
                         int(d), ws.Tp, tiles);
    }
  }
  hipLaunchKernelGGL(bwd_gates_kernel, dim3(unsigned(H)), dim3(kGThreads), 0, stream, fgate,
                     rsum, csum, digate, dfgate, T, int(exp_forget));
  return hipGetLastError();
}

}  // namespace

// The stored dV operand is used up to this size (the environment variable
// MLSTM_BWD_STORE_MAX, in bytes, overrides it); above it the values pass
// recomputes S (bitwise the same results, more time, no quadratic memory).
// The entry point calls this once per call and hands the result to both the
// scratch sizing and the launch, so the two can never disagree.
constexpr size_t kBackwardStoreMax = size_t(2) << 30;

size_t backward_store_bytes(int64_t H, int64_t T, int64_t d, bool is_bf16) {
  if (!is_bf16 || !backward_mfma_supports(d)) return 0;
  size_t cap = kBackwardStoreMax;
  if (const char* e = std::getenv("MLSTM_BWD_STORE_MAX")) cap = size_t(std::strtoull(e, nullptr, 10));
  const size_t b = backward_mfma_store_bytes(H, T);
  return b <= cap ? b : 0;
}

size_t backward_scratch_bytes(int64_t H, int64_t T, size_t store_bytes) {
  return 4 * align256(size_t(H) * size_t(T) * sizeof(float)) + align256(store_bytes);
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const float* fgate,
                           const void* h, const float* m, const float* n, const float* b,
                           const void* dh, const Workspace& ws, void* scratch,
                           size_t store_bytes, void* dq, void* dk, void* dv, float* digate,
                           float* dfgate, int64_t H, int64_t T, int64_t d, bool is_bf16,
                           bool exp_forget, hipStream_t stream) {
  if (d % 16 != 0 || d < 16 || d > kBackwardMaxHeadDim) return hipErrorInvalidValue;
  // the stored operand is all or nothing: a partial size would be overrun
  if (store_bytes != 0 &&
      (!is_bf16 || !backward_mfma_supports(d) || store_bytes != backward_mfma_store_bytes(H, T)))
    return hipErrorInvalidValue;
  char* p = static_cast<char*>(scratch);
  const size_t one = align256(size_t(H) * size_t(T) * sizeof(float));
  float* inv_n = reinterpret_cast<float*>(p);
  float* db = reinterpret_cast<float*>(p + one);
  float* rsum = reinterpret_cast<float*>(p + 2 * one);
  float* csum = reinterpret_cast<float*>(p + 3 * one);
  void* vstore = store_bytes ? p + 4 * one : nullptr;
  if (is_bf16) {
    using B16 = __hip_bfloat16;
    return launch_typed<B16>(static_cast<const B16*>(q), static_cast<const B16*>(k),
                             static_cast<const B16*>(v), fgate, static_cast<const B16*>(h), m, n,
                             b, static_cast<const B16*>(dh), ws, inv_n, db, rsum, csum, vstore,
                             static_cast<B16*>(dq), static_cast<B16*>(dk), static_cast<B16*>(dv),
                             digate, dfgate, H, T, d, exp_forget, backward_mfma_supports(d),
                             false, stream);
  }
  // float32 inputs: the matrix-core passes where they apply, unless the
  // environment variable MLSTM_BWD_F32=vector asks for the vector passes
  const char* sel = std::getenv("MLSTM_BWD_F32");
  const bool f32_tiles =
      backward_f32_supports(d) && !(sel != nullptr && std::strcmp(sel, "vector") == 0);
  return launch_typed<float>(static_cast<const float*>(q), static_cast<const float*>(k),
                             static_cast<const float*>(v), fgate, static_cast<const float*>(h), m,
                             n, b, static_cast<const float*>(dh), ws, inv_n, db, rsum, csum,
                             nullptr, static_cast<float*>(dq), static_cast<float*>(dk),
                             static_cast<float*>(dv), digate, dfgate, H, T, d, exp_forget, false,
                             f32_tiles, stream);
}

}  // namespace mlstm
