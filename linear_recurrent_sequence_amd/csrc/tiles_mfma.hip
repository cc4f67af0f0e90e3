// Stage 2, bf16 matrix-core variant: Eqs. 81-86 of the xLSTM appendix over
// causal tiles, with both contractions on gfx950 MFMA
// (v_mfma_f32_32x32x16_bf16, float32 accumulation).
//
// Work decomposition.  A workgroup of 4 waves owns 128 query rows of one head
// (32 rows per wave, the N = 32 side of every MFMA) and walks the key axis in
// tiles of 32 keys up to its diagonal; tiles above the diagonal are never
// visited (D' = 0 there, Eq. 71).  Because the stabilizer m depends only on
// the gates and is known from the scan, there is no running maximum and no
// rescaling of the accumulator: the exponent of every entry is final when it
// is formed, and the only row-wide quantity, the normalizer n (Eq. 84), is
// applied once at the end.
//
// Transposed products keep every intermediate in registers:
//   S^T (32 keys x 32 queries)  = K_J  Q^T          A = K from LDS, B = Q^T held in VGPRs
//   C~'^T = S^T (.) D'^T, row sums b from the float32 C~' (Eq. 83)
//   O^T (d x 32 queries)       += V_J^T C~'^T       A = V^T from LDS, B = bf16(C~'^T)
// In the 32x32 accumulator layout a lane holds one query column and 16 key
// rows, which is exactly the B-operand layout of the second product once the
// 16 keys are listed in the order the lane holds them; V^T is stored in LDS
// with its key axis permuted the same way (bits 2 and 3 of the key index
// swapped), so the contraction pairs each V row with its own C~' entry.
//
// Exponents: log2(D'_ij / sqrt(d)) = (A_{i/64} - A_{j/64}) + r_i + c_j with the
// terms of the gate scan; the anchor difference is formed in float64 once per
// (wave, tile).
//
// Pipelining: K, V^T and c of tile J+1 are fetched into registers while tile J
// is computed from the other half of a double-buffered LDS area, then stored;
// one barrier per tile.
#include "mlstm_internal.h"

namespace mlstm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;

constexpr int kBM = 128;   // query rows per workgroup
constexpr int kBN = 32;    // keys per tile
constexpr int kThreads = 256;
constexpr int kPf = 3;     // LDS fragment prefetch distance (MFMA steps)

template <int DP>
struct Cfg {
  static_assert(DP % 32 == 0 && DP >= 32 && DP <= 512, "padded head dim");
  static constexpr int KS = DP * 2 + 16;           // K tile row stride, bytes
  static constexpr int VS = kBN * 2 + 16;          // V^T tile row stride, bytes
  static constexpr int K_BYTES = kBN * KS;
  static constexpr int V_BYTES = DP * VS;
  static constexpr int C_BYTES = kBN * 4;
  static constexpr int BUF = (K_BYTES + V_BYTES + C_BYTES + 15) / 16 * 16;
  static constexpr int K_CHUNKS = kBN * DP / 8;    // 16-byte chunks of a K tile
  static constexpr int K_PER = (K_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int V_UNITS = (kBN / 2) * (DP / 8);  // (key pair, 8 columns)
  static constexpr int V_PER = (V_UNITS + kThreads - 1) / kThreads;
};

// key position inside a 32-key tile as stored in V^T: swap bits 2 and 3
__device__ __host__ constexpr int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Heaviest row tiles first (a row tile I costs ~I + 1 key tiles), and when the
// head count allows, every row tile of a head on the same XCD (workgroups are
// dealt to the 8 XCDs round-robin), so a head's K and V stay in one L2.
__device__ inline void map_tile(int64_t wg, int64_t row_tiles, int64_t H, int64_t& I,
                                int64_t& head) {
  if ((H & 7) == 0) {
    const int64_t x = wg & 7, s = wg >> 3, hpx = H >> 3;
    head = x + 8 * (s % hpx);
    I = row_tiles - 1 - s / hpx;
  } else {
    I = row_tiles - 1 - wg / H;
    head = wg % H;
  }
}

__device__ inline bf16x8 load16(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

template <int DP>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void tiles_mfma_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ m_in, const double* __restrict__ anchor,
    const float* __restrict__ rowt, const float* __restrict__ colt, u16* __restrict__ h_out,
    float* __restrict__ n_out, int64_t T, int d, int64_t Tp, int64_t nblk, int64_t row_tiles,
    int64_t H) {
  using C = Cfg<DP>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 5;    // half-wave: selects 8 of the 16 reduction indices
  const int l32 = lane & 31;  // query column of this lane
  int64_t I, head;
  map_tile(blockIdx.x, row_tiles, H, I, head);
  const int64_t hoff = head * T * int64_t(d);
  const int64_t q0 = I * kBM;
  const int64_t qw = q0 + 32 * w;  // first query row of this wave
  const int64_t qi = qw + l32;     // query row of this lane

  // Q^T fragments: B operand of S^T = K Q^T, reduction index = head dim
  // (branch-free: out-of-range rows and padded columns read a valid address
  // and are replaced by zeros)
  bf16x8 qf[DP / 16];
  {
    const int64_t qrow = qi < T ? qi : T - 1;
#pragma unroll
    for (int s = 0; s < DP / 16; ++s) {
      const int col = 16 * s + 8 * g;
      const bool ok = qi < T && col < d;
      const uint4 raw = *reinterpret_cast<const uint4*>(q + hoff + qrow * d + (ok ? col : 0));
      const uint4 z = make_uint4(0, 0, 0, 0);
      const uint4 val = ok ? raw : z;
      qf[s] = *reinterpret_cast<const bf16x8*>(&val);
    }
  }
  const float r_i = rowt[head * Tp + qi];
  const double a_i = anchor[head * nblk + qw / kAnchorBlock];

  f32x16 acc[DP / 32];
#pragma unroll
  for (int b = 0; b < DP / 32; ++b) acc[b] = f32x16{};
  float bsum = 0.0f;

  const int64_t n_key_tiles = (T + kBN - 1) / kBN;
  const int64_t last_tile = (4 * I + 3 < n_key_tiles - 1) ? 4 * I + 3 : n_key_tiles - 1;
  const int64_t wave_last = (4 * I + w < n_key_tiles - 1) ? 4 * I + w : n_key_tiles - 1;

  // ---- tile fetch (global -> registers) and store (registers -> LDS) ----
  uint4 kreg[C::K_PER];
  uint4 vreg[C::V_PER][2];
  float4 creg;
  auto fetch_k = [&](int64_t J) {
    const int64_t k0 = J * kBN;
#pragma unroll
    for (int it = 0; it < C::K_PER; ++it) {
      const int u = tid + kThreads * it;
      const int key = u / (DP / 8), dc = u % (DP / 8);
      const bool ok = u < C::K_CHUNKS && k0 + key < T && 8 * dc < d;
      const uint4 raw =
          *reinterpret_cast<const uint4*>(k + hoff + (ok ? (k0 + key) * d + 8 * dc : 0));
      kreg[it] = ok ? raw : make_uint4(0, 0, 0, 0);
    }
    if (tid < kBN / 4) creg = *reinterpret_cast<const float4*>(colt + head * Tp + k0 + 4 * tid);
  };
  auto fetch_v = [&](int64_t J) {
    const int64_t k0 = J * kBN;
#pragma unroll
    for (int it = 0; it < C::V_PER; ++it) {
      const int u = tid + kThreads * it;
      const int kp = u % (kBN / 2), dc = u / (kBN / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t key = k0 + 2 * kp + e;
        const bool ok = u < C::V_UNITS && key < T && 8 * dc < d;
        const uint4 raw = *reinterpret_cast<const uint4*>(v + hoff + (ok ? key * d + 8 * dc : 0));
        vreg[it][e] = ok ? raw : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_k = [&](int buf) {
    char* kb = smem + buf * C::BUF;
    char* cb = kb + C::K_BYTES + C::V_BYTES;
#pragma unroll
    for (int it = 0; it < C::K_PER; ++it) {
      const int u = tid + kThreads * it;
      const int key = u / (DP / 8), dc = u % (DP / 8);
      if (u < C::K_CHUNKS) *reinterpret_cast<uint4*>(kb + key * C::KS + 16 * dc) = kreg[it];
    }
    if (tid < kBN / 4) *reinterpret_cast<float4*>(cb + 16 * tid) = creg;
  };
  auto store_v = [&](int buf) {
    char* vb = smem + buf * C::BUF + C::K_BYTES;
#pragma unroll
    for (int it = 0; it < C::V_PER; ++it) {
      const int u = tid + kThreads * it;
      const int kp = u % (kBN / 2), dc = u / (kBN / 2);
      if (u < C::V_UNITS) {
        const u16* r0 = reinterpret_cast<const u16*>(&vreg[it][0]);
        const u16* r1 = reinterpret_cast<const u16*>(&vreg[it][1]);
        const int pos = vt_pos(2 * kp);  // keys 2kp, 2kp+1 stay adjacent
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned pair = unsigned(r0[e]) | (unsigned(r1[e]) << 16);
          *reinterpret_cast<unsigned*>(vb + (8 * dc + e) * C::VS + 2 * pos) = pair;
        }
      }
    }
  };

  fetch_k(0);
  fetch_v(0);
  store_k(0);
  store_v(0);
  __syncthreads();

  for (int64_t J = 0; J <= last_tile; ++J) {
    const int buf = int(J & 1);
    const bool more = J + 1 <= last_tile;
    const bool active = J <= wave_last;
    if (more) fetch_k(J + 1);
    f32x16 st = f32x16{};
    if (active) {
      const char* kb = smem + buf * C::BUF;
      const char* vb = kb + C::K_BYTES;
      const float* cb = reinterpret_cast<const float*>(vb + C::V_BYTES);
      // S^T = K_J Q^T: two partial accumulators keep two MFMA chains in flight;
      // K fragments are read kPf steps ahead (the scheduling barriers stop the
      // compiler from hoisting every LDS read of the unrolled loop)
      f32x16 s0 = f32x16{}, s1 = f32x16{};
      const char* kp = kb + l32 * C::KS + 16 * g;
      constexpr int NS = DP / 16;
      bf16x8 kf[kPf + 1];
#pragma unroll
      for (int t = 0; t < kPf && t < NS; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(kp + 32 * t);
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        if (t + kPf < NS) kf[(t + kPf) % (kPf + 1)] = *reinterpret_cast<const bf16x8*>(kp + 32 * (t + kPf));
        if (t & 1)
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % (kPf + 1)], qf[t], s1, 0, 0, 0);
        else
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % (kPf + 1)], qf[t], s0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      st = s0 + s1;
    }
    if (more) {
      store_k(buf ^ 1);
      fetch_v(J + 1);
    }
    if (active) {
      const char* kb = smem + buf * C::BUF;
      const char* vb = kb + C::K_BYTES;
      const float* cb = reinterpret_cast<const float*>(vb + C::V_BYTES);
      // lane (g, l32), register r holds S^T[key 8(r/4) + 4g + r%4][query l32]
      const float base = float(a_i - anchor[head * nblk + (J * kBN) / kAnchorBlock]) + r_i;
      const bool diag = (J * kBN == qw);
      float cv[16];
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float4 c4 = *reinterpret_cast<const float4*>(cb + 8 * rq + 4 * g);
        const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 8 * rq + 4 * g + e;
          float ex = base + cc[e];
          if (diag && key > l32) ex = -INFINITY;  // above the diagonal (Eq. 71)
          const float c = st[4 * rq + e] * __builtin_amdgcn_exp2f(ex);  // C~' (Eq. 82)
          bsum += c;                                                 // b (Eq. 83)
          cv[4 * rq + e] = c;
        }
      }
      bf16x8 p0, p1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p0[e] = (__bf16)cv[e];
        p1[e] = (__bf16)cv[8 + e];
      }
      // O^T += V_J^T C~'^T, V^T fragments read kPf steps ahead
      const char* vp = vb + l32 * C::VS + 16 * g;
      constexpr int NV = DP / 16;  // (column block, key half) steps
      bf16x8 vf[kPf + 1];
#pragma unroll
      for (int t = 0; t < kPf && t < NV; ++t)
        vf[t] = *reinterpret_cast<const bf16x8*>(vp + 32 * (t >> 1) * C::VS + 32 * (t & 1));
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const int tn = t + kPf;
        if (tn < NV)
          vf[tn % (kPf + 1)] =
              *reinterpret_cast<const bf16x8*>(vp + 32 * (tn >> 1) * C::VS + 32 * (tn & 1));
        acc[t >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t % (kPf + 1)], (t & 1) ? p1 : p0,
                                                              acc[t >> 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (more) store_v(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: n (Eq. 84), h~ = acc / n (Eqs. 85, 86) ----
  bsum += __shfl_xor(bsum, 32, 64);
  if (qi < T) {
    const float nn = fmaxf(fabsf(bsum), expf(-m_in[head * T + qi]));
    if (g == 0) n_out[head * T + qi] = nn;
    const float inv = 1.0f / nn;
    u16* hrow = h_out + hoff + qi * d;
#pragma unroll
    for (int b = 0; b < DP / 32; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = 32 * b + 8 * rq + 4 * g;
        if (col < d) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[b][4 * rq + e] * inv);
          *reinterpret_cast<bf16x4*>(hrow + col) = o;
        }
      }
    }
  }
}

template <int DP>
hipError_t launch_dp(const void* q, const void* k, const void* v, const float* m,
                     const Workspace& ws, void* h_out, float* n_out, int64_t H, int64_t T,
                     int64_t d, hipStream_t stream) {
  const int64_t row_tiles = (T + kBM - 1) / kBM;
  hipLaunchKernelGGL(tiles_mfma_kernel<DP>, dim3(unsigned(row_tiles * H)), dim3(kThreads), 0,
                     stream, static_cast<const u16*>(q), static_cast<const u16*>(k),
                     static_cast<const u16*>(v), m, ws.anchor, ws.rowt, ws.colt,
                     static_cast<u16*>(h_out), n_out, T, int(d), ws.Tp, ws.nblk, row_tiles, H);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tiles_mfma(const void* q, const void* k, const void* v, const float* m,
                             const Workspace& ws, void* h_out, float* n_out, int64_t H,
                             int64_t T, int64_t d, hipStream_t stream) {
  // head dims are padded up to a multiple of 32 (zero columns add nothing)
  switch ((d + 31) / 32) {
    case 1: return launch_dp<32>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 2: return launch_dp<64>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 3: return launch_dp<96>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 4: return launch_dp<128>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 5: return launch_dp<160>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 6: return launch_dp<192>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 7: return launch_dp<224>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 8: return launch_dp<256>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 9: return launch_dp<288>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 10: return launch_dp<320>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 11: return launch_dp<352>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 12: return launch_dp<384>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 13: return launch_dp<416>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 14: return launch_dp<448>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 15: return launch_dp<480>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    case 16: return launch_dp<512>(q, k, v, m, ws, h_out, n_out, H, T, d, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mlstm
