// Stage 2, bf16 matrix-core variant for wide heads (up to d = 1024): Eqs.
// 81-86 of the xLSTM appendix over causal tiles, both contractions on gfx950
// MFMA (v_mfma_f32_32x32x16_bf16, float32 accumulation).
//
// Why a separate kernel.  A wave of the narrower kernels keeps, for its 32
// query rows, the Q^T fragments over the whole head dimension (the B operand
// of S^T = K Q^T) and all output columns in registers: at d = 1024 that is
// 256 + 512 registers, more than a wave can hold even alone on its SIMD.
// Here four waves ("members") share a 32-row query block and split the head
// dimension in quarters, both as the reduction index of the first product and
// as the output columns of the second.  Member u holds Q^T for head dims
// [u d/4, (u + 1) d/4) and accumulates the output columns of the same range:
//   partial S^T_u = K[:, quarter u] Q^T[quarter u]      (32 keys x 32 queries)
//   S^T = sum over u of S^T_u: a reduce-scatter through LDS in float32.  In
//     the 32x32 accumulator layout a lane holds 16 keys of its query column
//     in four groups of four registers; member u receives group u from the
//     other three and adds the four partials in the fixed order 0, 1, 2, 3
//   member u forms C~'^T = S^T (.) D'^T and the row sums b on its group
//     (Eqs. 81-83) and hands bf16(C~'^T) of the group to the others
//   O^T[quarter u] += V^T[quarter u] C~'^T over the tile's 32 keys
// The matrix-core work equals that of one wave per query block without any
// split, nothing is recomputed, and each exponential is taken once.  Two query
// blocks (64 rows, 8 waves, two per SIMD) form a workgroup, so that one wave's
// copies, exponentials and LDS traffic overlap the other's matrix products.
//
// Data movement.  One 32-key K tile and one V tile live in LDS (130 KiB at
// d = 1024), each refilled while the other is read: the copies of V_J run
// during the partial products of tile J, those of K_{J+1} and its gate terms
// during the output products of J.  Three barriers per tile separate the
// partial products, the reduction with the exponentials, and the output
// products.  Copies, LDS padding, exponent factoring and decay-aware skipping
// are those of the two-wave kernel for d <= 384.
#include "mlstm_internal.h"
#include "tile_common.h"

namespace mlstm {
namespace {

using namespace tilecommon;

constexpr int kXThreads = 512;  // 8 waves: two per SIMD
constexpr int kXWaves = kXThreads / 64;
constexpr int kXM = 64;         // query rows per workgroup: two blocks of 32
constexpr int kXPf = 3;         // LDS fragment prefetch distance (MFMA steps)

// LDS layout (bytes).  K rows stride 2 DP + 16 and V rows 2 DP + 64 make the
// fragment and transpose reads conflict-free (DP / 8 + 1 and DP / 32 + 1 are
// odd for every DP here).  The partial sums of a query block take
// [dest member][3 sources] slots of 1 KiB (16 bytes per lane); its bf16 C~'^T
// takes [key half][group parity] slots of 512 bytes (8 bytes per lane).
template <int DP>
struct XCfg {
  static_assert(DP % 128 == 0 && DP >= 512 && DP <= 1024, "head dim of the wide kernel");
  static constexpr int QD = DP / 4;           // head dims of a member
  static constexpr int CH = DP / 8;           // 16-byte chunks per row
  static constexpr int NCP = (CH + 63) / 64;  // copy instructions per row
  static constexpr int RSK = 2 * DP + 16;     // K row stride
  static constexpr int RSV = 2 * DP + 64;     // V row stride
  static constexpr int NB = QD / 32;          // 32-column output blocks per wave
  static constexpr int NS = QD / 16;          // MFMA steps of a partial S^T
  static constexpr int RPW = kBN / kXWaves;   // rows of a 32-key tile copied per wave
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = kBN * RSK;
  static constexpr int GC = V_OFF + kBN * RSV;  // C_j of the K tile's 32 keys (float64)
  static constexpr int GE = GC + 256;           // e_j (float32)
  static constexpr int GB = GC + 384;           // keyb of the tile (float64)
  static constexpr int X_OFF = GC + 400;        // partial sums, 12 KiB per query block
  static constexpr int P_OFF = X_OFF + 2 * 12 * 1024;  // bf16 C~'^T, 2 KiB per query block
  static constexpr int BYTES = P_OFF + 2 * 2048;
  static_assert(kXM * RSK <= GC, "the staged Q and output blocks fit in the K and V regions");
  static_assert(GC % 256 == 0, "alignment of the gate terms and exchange slots");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int DP>
__global__ __attribute__((amdgpu_flat_work_group_size(kXThreads, kXThreads),
                          amdgpu_waves_per_eu(2, 2))) void tiles_wide_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ m_in, const double* __restrict__ rowt,
    const double* __restrict__ colt, const float* __restrict__ colx, u16* __restrict__ h_out,
    const double* __restrict__ rowb, const double* __restrict__ keyb, float* __restrict__ n_out,
    const u16* __restrict__ ogate, u16* __restrict__ htilde, float* __restrict__ b_out, int T,
    int d, int Tp, int row_tiles, int H, int skip) {
  using C = XCfg<DP>;
  __shared__ __attribute__((aligned(1024))) char lds[C::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pq = w >> 2;      // query block
  const int hh = w & 3;       // member: head-dim quarter, key group of the reduction
  const int g = lane >> 5;    // half-wave: selects 8 of the 16 reduction indices
  const int l32 = lane & 31;  // query column of this lane
  const int j16 = l32 & 15;
  int64_t I64, head64;
  map_tile(blockIdx.x, row_tiles, H, I64, head64);
  const int I = int(I64), head = int(head64);
  const int64_t hoff = int64_t(head) * T * d;
  const int q0 = I * kXM;
  const int qw = q0 + 32 * pq;  // first query row of this block
  const int qi = qw + l32;      // query row of this lane (< Tp: Tp is a multiple of 128)
  const int dch = d / 8;        // real 16-byte chunks per row

  bf16x8 qf[C::NS];  // Q^T over this member's quarter: B operand of the partial S^T
  const double r_i = rowt[int64_t(head) * Tp + qi];  // R_i

  f32x16 acc[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) acc[b] = f32x16{};
  float bsum = 0.0f;

  const int n_key_tiles = (T + kBN - 1) / kBN;
  const int last_tile = (2 * I + 1 < n_key_tiles - 1) ? 2 * I + 1 : n_key_tiles - 1;
  const int block_last = (2 * I + pq < n_key_tiles - 1) ? 2 * I + pq : n_key_tiles - 1;
  const int nb32 = Tp / kBoundTile;

  // ---- copies: one padded row takes NCP instructions of up to 64 lanes x 16
  // bytes; chunks past the real head dimension, and rows past the sequence
  // end (empty buffer range), arrive as zeros.
  unsigned vch[C::NCP];
#pragma unroll
  for (int c = 0; c < C::NCP; ++c)
    vch[c] = 64 * c + lane < dch ? unsigned(16 * (64 * c + lane)) : kOutOfRange;
  auto copy_part = [&](const u16* src, int row, unsigned dst, int c) {
    const i32x4 rs = rsrc_words(src + hoff + int64_t(row) * d, row < T ? 2 * d : 0);
    if (64 * c + lane < C::CH) copy16(rs, vch[c], dst + 1024 * c);
  };
  // copy unit u (0 <= u < RPW * NCP) of this wave's share of a tile:
  // row w + 8 (u / NCP), instruction u % NCP
  auto copy_k = [&](int J, int u) {
    const int r = w + kXWaves * (u / C::NCP);
    copy_part(k, J * kBN + r, lds_addr(lds + C::K_OFF + r * C::RSK), u % C::NCP);
  };
  auto copy_v = [&](int J, int u) {
    const int r = w + kXWaves * (u / C::NCP);
    copy_part(v, J * kBN + r, lds_addr(lds + C::V_OFF + r * C::RSV), u % C::NCP);
  };
  auto copy_gates = [&](int J) {
    const int k0 = J * kBN;
    if (w == 0 && lane < 16)
      copy16(rsrc_words(colt + int64_t(head) * Tp + k0, kBN * 8), unsigned(16 * lane),
             lds_addr(lds + C::GC));
    if (w == 1 && lane < 8)
      copy16(rsrc_words(colx + int64_t(head) * Tp + k0, kBN * 4), unsigned(16 * lane),
             lds_addr(lds + C::GE));
    if (w == 2 && lane < 2)
      copy4(rsrc_words(keyb + int64_t(head) * nb32 + J, 8), unsigned(4 * lane),
            lds_addr(lds + C::GB));
  };
  constexpr int kUnits = C::RPW * C::NCP;

  // ---- the workgroup's Q block (64 rows, contiguous in memory) is staged in
  // the K and V regions, overlapping the first-tile search
#pragma unroll
  for (int i = 0; i < kXM / kXWaves; ++i) {
    const int r = w + kXWaves * i;
#pragma unroll
    for (int c = 0; c < C::NCP; ++c) copy_part(q, q0 + r, lds_addr(lds + C::K_OFF + r * C::RSK), c);
  }

  // ---- decay-aware start of the key loop: the first 32-key tile either
  // block needs (the bound of mlstm_internal.h); inside the loop each block
  // skips the products of tiles its rows do not need.
  const double rb_w = rowb[int64_t(head) * nb32 + qw / kBoundTile];  // uniform across the wave
  auto tile_needed = [&](double rb, double kb) { return rb + kb >= kSkipLog2; };
  int first_tile = 0;
  if (skip) {
    __shared__ int s_first[kXWaves];
    double rb_rows[2];
    int last_b[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int qu = q0 + 32 * u;
      rb_rows[u] = rowb[int64_t(head) * nb32 + qu / kBoundTile];
      last_b[u] = (2 * I + u < n_key_tiles - 1) ? 2 * I + u : n_key_tiles - 1;
    }
    int mine = last_tile;
    for (int J = tid; J < last_tile; J += kXThreads) {
      const double kb = keyb[int64_t(head) * nb32 + J];
      bool need = false;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        need = need || (J <= last_b[u] && tile_needed(rb_rows[u], kb));
      if (need) {
        mine = J;
        break;  // J grows with each iteration: the first hit is this thread's least
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const int o = __shfl_xor(mine, off, 64);
      mine = o < mine ? o : mine;
    }
    if (lane == 0) s_first[w] = mine;
    __syncthreads();
    first_tile = s_first[0];
#pragma unroll
    for (int u = 1; u < kXWaves; ++u) first_tile = s_first[u] < first_tile ? s_first[u] : first_tile;
    first_tile = __builtin_amdgcn_readfirstlane(first_tile);
  }

  // per-lane LDS offsets of the fragment reads.
  // K: row l32, bytes 2 QD hh + 32 t + 16 g for MFMA step t.
  const int krow = C::K_OFF + l32 * C::RSK + 16 * g + 2 * C::QD * hh;
  // V^T gather (ds_read_b64_tr_b16): rows 16 c + 4 g + j16 / 4 (+ 8) of the
  // tile for key half c, bytes 2 QD hh + 64 b + 32 (l32 / 16) + 8 (j16 % 4)
  // for this member's 32-column block b.
  const int vrow = C::V_OFF + (4 * g + (j16 >> 2)) * C::RSV + 32 * (l32 >> 4) + 8 * (j16 & 3) +
                   2 * C::QD * hh;
  char* const xblk = lds + C::X_OFF + 12 * 1024 * pq;
  char* const pblk = lds + C::P_OFF + 2048 * pq;

  // ---- prologue: Q^T fragments from the staged block; then K and the gate
  // terms of the first tile
  {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int qrow = C::K_OFF + (32 * pq + l32) * C::RSK + 16 * g + 2 * C::QD * hh;
#pragma unroll
    for (int t = 0; t < C::NS; ++t) qf[t] = *reinterpret_cast<const bf16x8*>(lds + qrow + 32 * t);
    __syncthreads();  // the region is refilled below
  }
  {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) copy_k(first_tile, u);
    copy_gates(first_tile);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // the wave's copy units are spread over the n matrix instructions of a phase
  auto copies_at = [&](int t, int n, auto&& copy) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u)
      if ((u * n) / kUnits == t) copy(u);
  };

  for (int J = first_tile; J <= last_tile; ++J) {
    // ===== phase 1: K_J and its gate terms are resident; copies bring V_J =====
    const double kb = *reinterpret_cast<const double*>(lds + C::GB);
    const bool need = __builtin_amdgcn_readfirstlane(
                          int(J <= block_last && (!skip || tile_needed(rb_w, kb)))) != 0;
    f32x16 st = f32x16{};
    if (need) {
      bf16x8 kf[kXPf + 1];
      auto kaddr = [&](int t) { return lds + krow + 32 * t; };
#pragma unroll
      for (int t = 0; t < kXPf && t < C::NS; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(kaddr(t));
#pragma unroll
      for (int t = 0; t < C::NS; ++t) {
        if (t + kXPf < C::NS)
          kf[(t + kXPf) % (kXPf + 1)] = *reinterpret_cast<const bf16x8*>(kaddr(t + kXPf));
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % (kXPf + 1)], qf[t], st, 0, 0, 0);
        copies_at(t, C::NS, [&](int u) { copy_v(J, u); });
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane (g, l32), register r holds the partial S^T[key 8(r/4) + 4g + r%4][query l32];
      // group dest (registers 4 dest .. 4 dest + 3) goes to member dest
#pragma unroll
      for (int dest = 0; dest < 4; ++dest) {
        if (dest != hh) {
          const int slot = hh < dest ? hh : hh - 1;
          const float4 val = {st[4 * dest], st[4 * dest + 1], st[4 * dest + 2], st[4 * dest + 3]};
          *reinterpret_cast<float4*>(xblk + 3072 * dest + 1024 * slot + 16 * lane) = val;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kUnits; ++u) copy_v(J, u);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ===== phase 2: S^T on this member's key group; C~' = S (.) D' (Eq. 82),
    // b += C~' (Eq. 83); bf16(C~'^T) to the exchange slots =====
    if (need) {
      float4 pr[3];
#pragma unroll
      for (int s = 0; s < 3; ++s)
        pr[s] = *reinterpret_cast<const float4*>(xblk + 3072 * hh + 1024 * s + 16 * lane);
      const float4 own = hh == 0   ? float4{st[0], st[1], st[2], st[3]}
                         : hh == 1 ? float4{st[4], st[5], st[6], st[7]}
                         : hh == 2 ? float4{st[8], st[9], st[10], st[11]}
                                   : float4{st[12], st[13], st[14], st[15]};
      // partials of members 0, 1, 2, 3 in that order
      float4 tot = hh == 0 ? own : pr[0];
      tot += hh == 1 ? own : hh < 1 ? pr[0] : pr[1];
      tot += hh == 2 ? own : hh < 2 ? pr[1] : pr[2];
      tot += hh == 3 ? own : pr[2];
      float p[4] = {tot.x, tot.y, tot.z, tot.w};
      if (J * kBN == qw) {  // diagonal tile: causal mask (Eq. 71)
        const double* gc = reinterpret_cast<const double*>(lds + C::GC) + 8 * hh + 4 * g;
        const double2 c01 = *reinterpret_cast<const double2*>(gc);
        const double2 c23 = *reinterpret_cast<const double2*>(gc + 2);
        const double cc[4] = {c01.x, c01.y, c23.x, c23.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 8 * hh + 4 * g + e;
          const float ex = key > l32 ? -INFINITY : float(r_i + cc[e]);
          p[e] *= __builtin_amdgcn_exp2f(ex);
          bsum += p[e];
        }
      } else {
        const float ei = __builtin_amdgcn_exp2f(float(r_i + kb));
        const float4 e4 = *reinterpret_cast<const float4*>(lds + C::GE + 4 * (8 * hh + 4 * g));
        const float ee[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] *= ei * ee[e];
          bsum += p[e];
        }
      }
      bf16x4 pg;
#pragma unroll
      for (int e = 0; e < 4; ++e) pg[e] = (__bf16)p[e];
      *reinterpret_cast<bf16x4*>(pblk + 1024 * (hh >> 1) + 512 * (hh & 1) + 8 * lane) = pg;
    }
    __syncthreads();

    // ===== phase 3: V_J is resident; copies bring K_{J+1} and its gate terms =====
    const bool more = J < last_tile;
    // The products run even when the tile does not reach the block's rows
    // (their operands are then zero): a branch around them would make the
    // compiler copy the accumulators.
    {
      const bf16x8 zero8 = bf16x8{};
      bf16x8 pb[2] = {zero8, zero8};
      if (need) {
        // key half c: groups 2c (slots 0..3) and 2c + 1 (slots 4..7), the
        // order in which S^T registers 8c .. 8c + 7 hold the keys
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(pblk + 1024 * c + 8 * lane);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(pblk + 1024 * c + 512 + 8 * lane);
          pb[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
      // O^T[own columns] += V^T C~'^T: step t = (column block b, key half c);
      // the A operand holds V[16 c + 4g + 0..3][col + l32] and
      // V[16 c + 8 + 4g + 0..3][col + l32]
      constexpr int NV = 2 * C::NB;
      auto vaddr = [&](int t) { return lds + vrow + 64 * (t >> 1) + 16 * (t & 1) * C::RSV; };
      i16x4 vlo[kXPf + 1], vhi[kXPf + 1];
#pragma unroll
      for (int t = 0; t < kXPf && t < NV; ++t) {
        vlo[t] = tr_read(vaddr(t));
        vhi[t] = tr_read(vaddr(t) + 8 * C::RSV);
      }
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const int tn = t + kXPf;
        if (tn < NV) {
          vlo[tn % (kXPf + 1)] = tr_read(vaddr(tn));
          vhi[tn % (kXPf + 1)] = tr_read(vaddr(tn) + 8 * C::RSV);
        }
        const i16x8 a16 = __builtin_shufflevector(vlo[t % (kXPf + 1)], vhi[t % (kXPf + 1)], 0, 1,
                                                  2, 3, 4, 5, 6, 7);
        acc[t >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16),
                                                              pb[t & 1], acc[t >> 1], 0, 0, 0);
        if (more) copies_at(t, NV, [&](int u) { copy_k(J + 1, u); });
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (more) copy_gates(J + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: b of the block (members 0..3 in order), n (Eq. 84),
  // h~ = acc / n (Eqs. 85, 86), output gate (Eq. 78) on this member's columns
  bsum += __shfl_xor(bsum, 32, 64);
  const float m_q = qi < T ? m_in[int64_t(head) * T + qi] : 0.0f;
  float* red = reinterpret_cast<float*>(lds + C::X_OFF) + 256 * pq;
  red[64 * hh + lane] = bsum;
  __syncthreads();
  const float btot = ((red[lane] + red[64 + lane]) + red[128 + lane]) + red[192 + lane];
  const float nn = fmaxf(fabsf(btot), expf(-m_q));
  const float inv = 1.0f / nn;
  if (qi < T && g == 0 && hh == 0) {
    n_out[int64_t(head) * T + qi] = nn;
    if (b_out) b_out[int64_t(head) * T + qi] = btot;
  }
  if (ogate == nullptr && htilde == nullptr) {
    // bf16(h~) is staged in LDS (the tile regions are free now) as row
    // 32 pq + l32 of the block; the block's rows, contiguous in memory, are
    // then stored 1 KiB per instruction.  Rows past the sequence end fall
    // outside the buffer range and are not written.
    const int orow = C::K_OFF + (32 * pq + l32) * C::RSK;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = C::QD * hh + 32 * b + 8 * rq + 4 * g;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[b][4 * rq + e] * inv);
        *reinterpret_cast<bf16x4*>(lds + orow + 2 * col) = o;
      }
    }
    __syncthreads();
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const int rows = T - q0 < kXM ? T - q0 : kXM;
    const auto rh = make_rsrc(h_out + hoff + int64_t(q0) * d, int64_t(rows) * d * 2);
    const int nstore = d / 8;  // 1 KiB stores of the 64 x d block
    const int row_bytes = 2 * d;
#pragma unroll
    for (int u = 0; u < (DP / 8 + kXWaves - 1) / kXWaves; ++u) {
      const int n = w + kXWaves * u;
      if (n < nstore) {
        const int gb = 1024 * n + 16 * lane;
        const int r = gb / row_bytes;
        const int c = (gb - r * row_bytes) >> 4;
        const u32x4 val = *reinterpret_cast<const u32x4*>(lds + C::K_OFF + r * C::RSK + 16 * c);
        __builtin_amdgcn_raw_buffer_store_b128(val, rh, gb, 0, 0);
      }
    }
  } else if (qi < T) {
    const int64_t row = hoff + int64_t(qi) * d;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = C::QD * hh + 32 * b + 8 * rq + 4 * g;
        if (col < d) {
          float hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = acc[b][4 * rq + e] * inv;
          bf16x4 o;
          if (htilde) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)hv[e];
            *reinterpret_cast<bf16x4*>(htilde + row + col) = o;
          }
          if (ogate) {
            const bf16x4 og = *reinterpret_cast<const bf16x4*>(ogate + row + col);
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] *= 1.0f / (1.0f + __expf(-float(og[e])));
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)hv[e];
          *reinterpret_cast<bf16x4*>(h_out + row + col) = o;
        }
      }
    }
  }
}

template <int DP>
hipError_t launch_x(const void* q, const void* k, const void* v, const float* m,
                    const Workspace& ws, void* h_out, float* n_out, const Epilogue& ep, bool skip,
                    int64_t H, int64_t T, int64_t d, hipStream_t stream) {
  const int64_t row_tiles = (T + kXM - 1) / kXM;
  hipLaunchKernelGGL(tiles_wide_kernel<DP>, dim3(unsigned(row_tiles * H)), dim3(kXThreads), 0,
                     stream, static_cast<const u16*>(q), static_cast<const u16*>(k),
                     static_cast<const u16*>(v), m, ws.rowt, ws.colt, ws.colx,
                     static_cast<u16*>(h_out), ws.rowb, ws.keyb, n_out,
                     static_cast<const u16*>(ep.ogate), static_cast<u16*>(ep.htilde), ep.b, T,
                     int(d), int(ws.Tp), int(row_tiles), int(H), int(skip));
  return hipGetLastError();
}

}  // namespace

bool tiles_wide_supports(int64_t d) { return d % 16 == 0 && d >= 16 && d <= 1024; }

hipError_t launch_tiles_wide(const void* q, const void* k, const void* v, const float* m,
                             const Workspace& ws, void* h_out, float* n_out, const Epilogue& ep,
                             bool skip, int64_t H, int64_t T, int64_t d, hipStream_t stream) {
  if (!tiles_wide_supports(d)) return hipErrorInvalidValue;
  // head dims are padded up to a multiple of 128, at least 512 (zero columns add nothing)
  switch (d <= 512 ? 4 : (d + 127) / 128) {
    case 4: return launch_x<512>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, stream);
    case 5: return launch_x<640>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, stream);
    case 6: return launch_x<768>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, stream);
    case 7: return launch_x<896>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, stream);
    case 8: return launch_x<1024>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mlstm
