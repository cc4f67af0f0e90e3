// Stage 2, float32 vector-ALU variant: Eqs. 81-86 of the xLSTM appendix
// ("Parallel mLSTM Backward Pass" opens with the stabilized forward pass) over
// causal 16 x 16 tiles.
//
// This is the path for float32 inputs and a second, independent GPU
// evaluation for bf16 inputs: both contractions run on the vector ALUs in
// float32 and C~' is never rounded to bf16.  One workgroup of 256 threads owns
// 16 query rows of one head; thread (r, c) of the 16 x 16 grid forms one
// entry of S = Q K^T and of C~' per key tile, and then accumulates output
// columns c, c + 16, ... of row r.  For head dims above 512 the K and V
// tiles take turns in one LDS buffer (Q, K and V tiles of 16 x 1024 float32
// would not fit together).
//
// On sequences of at most 2048 positions the kernel can also scan its head's
// gates itself (the whole pass in one launch, no workspace): its 256 threads
// run the gate-scan kernel's 512-thread block scan over positions
// [0, q0 + 16), two scan threads each (the same combinations in the same
// order, so R_i, C_j and m are bitwise those of the two-launch path), and keep
// C_j of those positions and R_i, m of the workgroup's rows in LDS.
#include "mlstm_internal.h"
#include "scan_common.h"
#include "tile_common.h"

#include <hip/hip_bf16.h>

namespace mlstm {
namespace {

using tilecommon::FusedGates;

constexpr int kVT = 16;  // query rows per workgroup and keys per tile
constexpr int kVFusedMaxT = scan::kScanThreads * scan::kScanPer;  // one block scan: 2048

__device__ inline float load_elem(const float* p) { return *p; }
__device__ inline float load_elem(const __hip_bfloat16* p) { return __bfloat162float(*p); }
__device__ inline void store_elem(float* p, float x) { *p = x; }
__device__ inline void store_elem(__hip_bfloat16* p, float x) { *p = __float2bfloat16(x); }

template <typename Tin, int MAXD, bool FUSED>
__global__ __launch_bounds__(256) void tiles_vector_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ m_in, const double* __restrict__ rowt,
    const double* __restrict__ colt, Tin* __restrict__ h_out, float* __restrict__ n_out,
    const Tin* __restrict__ ogate, Tin* __restrict__ htilde, float* __restrict__ b_out,
    int64_t T, int d, int64_t Tp, int64_t row_tiles, FusedGates fg) {
  constexpr bool kShared = MAXD > 512;  // K and V tiles share one buffer
  __shared__ float Qs[kVT][MAXD + 1];
  __shared__ float Ks[kVT][MAXD + 1];
  __shared__ float Vbuf[kShared ? 1 : kVT][kShared ? 1 : MAXD];
  __shared__ float Ps[kVT][kVT + 1];
  // fused gate scan: C_j of positions [0, q0 + 16), R_i and m of the rows
  __shared__ double Cs[FUSED ? kVFusedMaxT : 1];
  __shared__ double Rs[FUSED ? kVT : 1];
  __shared__ float Ms[FUSED ? kVT : 1];
  auto Vs = [&](int r, int c) -> float& { return kShared ? Ks[r][c] : Vbuf[r][c]; };

  const int tid = threadIdx.x;
  const int rl = tid / kVT;  // local query row
  const int cl = tid % kVT;  // local key (S phase) / column group (PV phase)
  const int64_t head = blockIdx.x / row_tiles;
  const int64_t q0 = (blockIdx.x % row_tiles) * kVT;
  const int64_t qi = q0 + rl;
  const int64_t hoff = head * T * int64_t(d);

  for (int idx = tid; idx < kVT * d; idx += 256) {
    const int r = idx / d, c = idx % d;
    Qs[r][c] = (q0 + r < T) ? load_elem(q + hoff + (q0 + r) * d + c) : 0.0f;
  }
  double r_i;  // R_i
  if constexpr (FUSED) {
    using namespace scan;
    // positions at or past t_eff are padding (no forgetting, no input): they
    // follow every position this workgroup reads, so they change none of them
    const int64_t t_eff = T < q0 + kVT ? T : q0 + kVT;
    const float* fgh = fg.fgate + head * T;
    const float* igh = fg.igate + head * T;
    const bool vec_rows = (T & 3) == 0;  // rows of the [H][T] gates 16-byte aligned
    const int w = tid >> 6;
    double fb[2][kScanPer];
    float iv[2][kScanPer];
    bool active[2];
    scan::Elem mine[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t p0 = int64_t(kScanPer) * (tid + (kScanThreads / 2) * u);
      // a scan wave whose positions all lie at or past t_eff holds padding only
      active[u] = int64_t(kScanPer) * 64 * (w + 4 * u) < t_eff;  // uniform across the wave
#pragma unroll
      for (int e = 0; e < kScanPer; ++e) {
        fb[u][e] = 0.0;
        iv[u][e] = -INFINITY;
      }
      if (active[u]) load_gates(fgh, igh, p0, t_eff, vec_rows, fg.exp_forget, fb[u], iv[u]);
      mine[u] = thread_elem(fb[u], iv[u]);
    }
    scan::Elem before[2], total;
    block_scan_halves(mine[0], mine[1], before[0], before[1], total);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!active[u]) continue;
      const int64_t p0 = int64_t(kScanPer) * (tid + (kScanThreads / 2) * u);
      Terms tm;
      position_terms(identity(), before[u], fb[u], iv[u], p0, t_eff, fg.half_ln_d, tm);
#pragma unroll
      for (int e = 0; e < kScanPer; ++e) {
        const int64_t p = p0 + e;
        if (p < t_eff) {
          Cs[p] = tm.c[e];
          if (p >= q0) {
            Rs[p - q0] = tm.r[e];
            Ms[p - q0] = tm.m[e];
            fg.m_out[head * T + p] = tm.m[e];
          }
        }
      }
    }
    __syncthreads();
    r_i = qi < T ? Rs[rl] : 0.0;
  } else {
    r_i = rowt[head * Tp + qi];  // qi < Tp: Tp is T rounded up to 128
  }

  float acc[MAXD / kVT];
#pragma unroll
  for (int u = 0; u < MAXD / kVT; ++u) acc[u] = 0.0f;
  float bsum = 0.0f;

  const int64_t last_key = (q0 + kVT - 1 < T ? q0 + kVT - 1 : T - 1);
  for (int64_t k0 = 0; k0 <= last_key; k0 += kVT) {
    __syncthreads();  // previous tile fully consumed
    for (int idx = tid; idx < kVT * d; idx += 256) {
      const int r = idx / d, c = idx % d;
      const bool in = k0 + r < T;
      Ks[r][c] = in ? load_elem(k + hoff + (k0 + r) * d + c) : 0.0f;
      if (!kShared) Vs(r, c) = in ? load_elem(v + hoff + (k0 + r) * d + c) : 0.0f;
    }
    __syncthreads();
    const int64_t kj = k0 + cl;
    float s = 0.0f;
    for (int c = 0; c < d; ++c) s = fmaf(Qs[rl][c], Ks[cl][c], s);
    // log2(D'_ij / sqrt(d)) = R_i + C_j, rounded once   (Eqs. 79, 81, 82)
    // (with the fused scan, C_j of keys past the workgroup's last row is not
    // formed: such entries are masked below whatever the exponent)
    const float ex = float(r_i + (FUSED ? Cs[kj < kVFusedMaxT ? kj : 0] : colt[head * Tp + kj]));
    const bool valid = (kj <= qi) && (kj < T) && (qi < T);
    const float cv = valid ? s * exp2f(ex) : 0.0f;  // C~'_ij (Eq. 82)
    bsum += cv;                                     // b_i (Eq. 83), float32
    Ps[rl][cl] = cv;
    __syncthreads();
    if (kShared) {  // every S entry is formed: the V tile replaces the K tile
      for (int idx = tid; idx < kVT * d; idx += 256) {
        const int r = idx / d, c = idx % d;
        Vs(r, c) = k0 + r < T ? load_elem(v + hoff + (k0 + r) * d + c) : 0.0f;
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < MAXD / kVT; ++u) {
      const int c = cl + kVT * u;
      if (c < d) {
        float a = 0.0f;
#pragma unroll
        for (int t = 0; t < kVT; ++t) a = fmaf(Ps[rl][t], Vs(t, c), a);
        acc[u] += a;
      }
    }
  }
  // the 16 threads of a row are 16 consecutive lanes of one wave
#pragma unroll
  for (int off = kVT / 2; off > 0; off >>= 1) bsum += __shfl_xor(bsum, off, 64);
  if (qi < T) {
    const float m_i = FUSED ? Ms[rl] : m_in[head * T + qi];
    const float nn = fmaxf(fabsf(bsum), expf(-m_i));  // Eq. 84
    if (cl == 0) n_out[head * T + qi] = nn;
    if (cl == 0 && b_out) b_out[head * T + qi] = bsum;
#pragma unroll
    for (int u = 0; u < MAXD / kVT; ++u) {
      const int c = cl + kVT * u;
      if (c < d) {
        const int64_t at = hoff + qi * d + c;
        float hv = acc[u] / nn;  // Eqs. 85, 86
        if (htilde) store_elem(htilde + at, hv);
        if (ogate) hv *= 1.0f / (1.0f + __expf(-load_elem(ogate + at)));  // Eq. 78
        store_elem(h_out + at, hv);
      }
    }
  }
}

template <typename Tin, int MAXD, bool FUSED>
void launch_v(const void* q, const void* k, const void* v, const float* m, const Workspace& ws,
              void* h_out, float* n_out, const Epilogue& ep, int64_t H, int64_t T, int64_t d,
              const FusedGates& fg, hipStream_t stream) {
  const int64_t row_tiles = (T + kVT - 1) / kVT;
  hipLaunchKernelGGL((tiles_vector_kernel<Tin, MAXD, FUSED>), dim3(unsigned(row_tiles * H)),
                     dim3(256), 0, stream, static_cast<const Tin*>(q), static_cast<const Tin*>(k),
                     static_cast<const Tin*>(v), m, ws.rowt, ws.colt,
                     static_cast<Tin*>(h_out), n_out, static_cast<const Tin*>(ep.ogate),
                     static_cast<Tin*>(ep.htilde), ep.b, T, int(d), ws.Tp, row_tiles, fg);
}

// the instantiation for head dim d (LDS tiles and accumulators sized to it)
template <typename Tin, bool FUSED>
void launch_d(const void* q, const void* k, const void* v, const float* m, const Workspace& ws,
              void* h_out, float* n_out, const Epilogue& ep, int64_t H, int64_t T, int64_t d,
              const FusedGates& fg, hipStream_t stream) {
  if (d <= 64) launch_v<Tin, 64, FUSED>(q, k, v, m, ws, h_out, n_out, ep, H, T, d, fg, stream);
  else if (d <= 512) launch_v<Tin, 512, FUSED>(q, k, v, m, ws, h_out, n_out, ep, H, T, d, fg, stream);
  else launch_v<Tin, 1024, FUSED>(q, k, v, m, ws, h_out, n_out, ep, H, T, d, fg, stream);
}

}  // namespace

hipError_t launch_tiles_vector(const void* q, const void* k, const void* v, const float* m,
                               const Workspace& ws, void* h_out, float* n_out,
                               const Epilogue& ep, int64_t H, int64_t T, int64_t d,
                               bool is_bf16, hipStream_t stream) {
  if (d % 16 != 0 || d < 16 || d > 1024) return hipErrorInvalidValue;
  const FusedGates none{};
  if (is_bf16) launch_d<__hip_bfloat16, false>(q, k, v, m, ws, h_out, n_out, ep, H, T, d, none, stream);
  else launch_d<float, false>(q, k, v, m, ws, h_out, n_out, ep, H, T, d, none, stream);
  return hipGetLastError();
}

bool tiles_vector_fused_supports(int64_t T, int64_t d) {
  return d % 16 == 0 && d >= 16 && d <= 1024 && T >= 1 && T <= kVFusedMaxT;
}

hipError_t launch_tiles_vector_fused(const void* q, const void* k, const void* v,
                                     const float* igate, const float* fgate, void* h_out,
                                     float* m_out, float* n_out, const Epilogue& ep,
                                     bool exp_forget, int64_t H, int64_t T, int64_t d,
                                     bool is_bf16, hipStream_t stream) {
  if (!tiles_vector_fused_supports(T, d)) return hipErrorInvalidValue;
  FusedGates fg;
  fg.igate = igate;
  fg.fgate = fgate;
  fg.m_out = m_out;
  fg.half_ln_d = 0.5 * log(double(d));  // as the gate-scan kernel forms it
  fg.exp_forget = int(exp_forget);
  const Workspace none{};
  if (is_bf16) launch_d<__hip_bfloat16, true>(q, k, v, nullptr, none, h_out, n_out, ep, H, T, d, fg, stream);
  else launch_d<float, true>(q, k, v, nullptr, none, h_out, n_out, ep, H, T, d, fg, stream);
  return hipGetLastError();
}

}  // namespace mlstm
