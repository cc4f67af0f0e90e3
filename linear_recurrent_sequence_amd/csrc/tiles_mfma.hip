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
//   S^T (32 keys x 32 queries)  = K_J  Q^T      A = K rows from LDS, B = Q^T in VGPRs
//   C~'^T = S^T (.) D'^T, row sums b from the float32 C~' (Eq. 83)
//   O^T (d x 32 queries)       += V_J^T C~'^T   A = V^T via LDS transpose reads,
//                                               B = bf16(C~'^T) straight from S^T
// In the 32x32 accumulator layout a lane holds one query column and 16 key
// rows; listed in the order the lane holds them, those 16 keys are the
// B-operand slots of the second product, and the V^T operand is gathered in
// the same key order by ds_read_b64_tr_b16 from V stored row-major in LDS.
//
// Data movement.  K, V (row-major, padded rows) and the column exponent terms
// of tile J+1 are copied global -> LDS by the load-to-LDS path
// (buffer_load_dwordx4 ... lds: no staging registers, no VALU) while tile J is
// computed from the other buffer; one barrier per tile.  A copy holds its
// wave at issue, and with one wave per SIMD nothing else feeds the matrix
// core meanwhile, so a wave's 16 row copies are spread over the matrix
// instructions of its first product, one every NS/16 of them, and each
// copy's issue overlaps the product already in flight.  The first product
// therefore runs on every tile in the loop, also where the wave's rows need
// none of it (its result is then dropped).  The copies go through buffer
// resources whose range ends at the sequence end, so rows past it and
// head-dimension padding arrive as zeros.
//
// Exponents: log2(D'_ij / sqrt(d)) = R_i + C_j with the float64 terms of the
// gate scan.  On a tile below the diagonal the exponent factors as
// 2^(R_i + keyb_J) * e_j (R_i + keyb_J summed in float64 and rounded once; e_j
// from the gate scan): one exponential per row and tile instead of one per
// entry, which with one wave per SIMD would idle the matrix core.  On the
// diagonal tile each entry takes its own exponential of R_i + C_j, summed in
// float64 and rounded once, under the causal mask.  C_j, e_j and keyb_J of the
// tile's keys travel with the tile into LDS.
//
// Fused gate scan (FUSED: 384 < d <= 512, at most 2048 positions, a multiple
// of 4).  Each workgroup scans its head's gates from position 0 to its last
// row in its prologue, as the gate-scan kernel does (its 512-thread block
// scan run by these 256 threads, two scan threads each, in the same order,
// so the terms are bitwise the same), and keeps in LDS what it reads later:
// e_j of every key before its last row, C_j of its 128 diagonal keys, the key
// tiles' bounds, and R_i, the row bounds and m of its own rows.  The whole
// forward pass is then one launch with no workspace.
#include "mlstm_internal.h"
#include "scan_common.h"
#include "tile_common.h"

namespace mlstm {
namespace {

using namespace tilecommon;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPf = 3;      // LDS fragment prefetch distance (MFMA steps)
constexpr int kFusedMaxT = scan::kScanThreads * scan::kScanPer;  // one block scan
constexpr int kQHalf = kBM / 2 / kWaves;  // Q rows per wave and tile buffer

template <int DP>
struct Cfg {
  static_assert(DP % 32 == 0 && DP >= 32 && DP <= 512, "padded head dim");
  static constexpr int CH = DP / 8;               // 16-byte chunks per row
  static constexpr int RSK = DP * 2 + 16;         // K row stride: 16 rows hit 16 distinct bank groups
  static constexpr int RSV = DP * 2 + 64;         // V row stride: transpose reads 2-way at most
  static constexpr int K_BYTES = kBN * RSK;
  static constexpr int V_BYTES = kBN * RSV;
  static constexpr int C_OFF = K_BYTES + V_BYTES;  // C_j of the tile's keys (float64)
  static constexpr int KB_OFF = C_OFF + kBN * 8;   // max of C_j over the key tile (float64)
  static constexpr int E_OFF = (KB_OFF + 8 + 15) / 16 * 16;  // e_j of the tile's keys (float32)
  static constexpr int BUF = E_OFF + kBN * 4;
};

template <int DP, bool FUSED>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void tiles_mfma_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ m_in, const double* __restrict__ rowt,
    const double* __restrict__ colt, const float* __restrict__ colx, u16* __restrict__ h_out,
    const double* __restrict__ rowb,
    const double* __restrict__ keyb, float* __restrict__ n_out, const u16* __restrict__ ogate,
    u16* __restrict__ htilde, float* __restrict__ b_out, int64_t T, int d, int64_t Tp,
    int64_t row_tiles, int64_t H, int skip, FusedGates fg) {
  using C = Cfg<DP>;
  // two distinct buffers, so the loads into one never alias reads of the other
  __shared__ __attribute__((aligned(1024))) char smem0[C::BUF];
  __shared__ __attribute__((aligned(1024))) char smem1[C::BUF];
  // FUSED: the gate terms the workgroup reads, from its own scan: e_j of
  // every key before its last row, C_j of its diagonal keys, keyb of every
  // 32-key tile, and rowb, R_i and m of its own rows
  __shared__ __attribute__((aligned(16))) float f_e[FUSED ? kFusedMaxT : 1];
  __shared__ __attribute__((aligned(16))) double f_cd[FUSED ? kBM : 1];
  __shared__ double f_kb[FUSED ? kFusedMaxT / kBoundTile : 1];
  __shared__ double f_rb[FUSED ? kBM / kBoundTile : 1];
  __shared__ __attribute__((aligned(16))) double f_r[FUSED ? kBM : 1];
  __shared__ __attribute__((aligned(16))) float f_m[FUSED ? kBM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;    // half-wave: selects 8 of the 16 reduction indices
  const int l32 = lane & 31;  // query column of this lane
  int64_t I, head;
  map_tile(blockIdx.x, row_tiles, H, I, head);
  const int64_t hoff = head * T * int64_t(d);
  const int64_t q0 = I * kBM;
  const int64_t qw = q0 + 32 * w;  // first query row of this wave
  const int64_t qi = qw + l32;     // query row of this lane
  const int dch = d / 8;           // real 16-byte chunks per row

  // Q^T fragments: B operand of S^T = K Q^T, reduction index = head dim.  The
  // workgroup's 128 query rows are staged in the two tile buffers (64 rows
  // each, one copy per row); rows past the sequence end and padded columns
  // arrive as zeros.  Each wave then reads its 32 rows' fragments (loading
  // them straight from memory, where each instruction touches 32 rows, was
  // slower).  Without FUSED the prologue's copies (Q and the first tile) are
  // the builtin ones, which the compiler sees: it can then issue the gate
  // terms' loads of the prologue ahead of them (behind copies it cannot see,
  // those loads would wait for the whole Q block).  With FUSED every copy
  // goes through inline assembly, so the compiler never sets M0 itself.
  static_assert((kBM / 2) * C::RSK <= C::BUF, "64 staged rows fit in a tile buffer");
  bf16x8 qf[DP / 16];
  const unsigned vchunk = lane < dch ? unsigned(16 * lane) : kOutOfRange;
  // rows 64 h + kQHalf w + i (i < kQHalf) of the Q block into tile buffer h
  auto copy_q_half = [&](int h) {
    char* const dst = h == 0 ? smem0 : smem1;
#pragma unroll
    for (int i = 0; i < kQHalf; ++i) {
      const int r = kQHalf * w + i;
      const int64_t row = q0 + kBM / 2 * h + r;
      if (lane < C::CH)
        copy16(rsrc_words(q + hoff + row * d, row < T ? 2 * d : 0), vchunk,
               lds_addr(dst + r * C::RSK));
    }
  };
  const int64_t t_eff = T < q0 + kBM ? T : q0 + kBM;
  // each wave's Q^T fragments from its staged rows (waves 0, 1 in buffer 0)
  auto read_q_fragments = [&]() {
    const char* qrow = (w < 2 ? smem0 : smem1) + (32 * (w & 1) + l32) * C::RSK + 16 * g;
#pragma unroll
    for (int s = 0; s < DP / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
  };
  // the wave's 8 rows of K and of V of tile J (FUSED: inline-assembly copies)
  const int row_bytes = 2 * d;
  struct TileSrc { i32x4 k, v; };
  auto tile_src = [&](int64_t J) {
    const int64_t r0 = J * kBN + w * (kBN / kWaves);
    const int64_t left = T - r0;
    const int64_t nrec =
        (left < 0 ? 0 : left < kBN / kWaves ? left : kBN / kWaves) * 2 * int64_t(d);
    return TileSrc{rsrc_words(k + hoff + r0 * d, nrec), rsrc_words(v + hoff + r0 * d, nrec)};
  };
  auto row_copy = [&](const TileSrc& ts, char* buf, auto ic) {
    constexpr int i = decltype(ic)::value;
    if (lane < C::CH) {
      if constexpr (i < 8)
        copy16_row<i & 7, (i & 7) * C::RSK>(ts.k, vchunk, row_bytes,
                                             lds_addr(buf + w * (kBN / kWaves) * C::RSK));
      else
        copy16_row<i & 7, (i & 7) * C::RSV>(
            ts.v, vchunk, row_bytes, lds_addr(buf + C::K_BYTES + w * (kBN / kWaves) * C::RSV));
    }
  };
  if constexpr (FUSED) {
    // The gate pre-activations of positions [0, t_eff) go into buffer 1 ahead
    // of the Q block's first half (buffer 0), so that they are waited for
    // alone: a wave's loads complete in order.  Lengths are divisible by 4,
    // so every head's gate row starts 16-byte aligned.
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const unsigned off = unsigned(1024 * (w + kWaves * c) + 16 * lane);
      copy16(rsrc_words(fg.fgate + head * T, t_eff * 4), off,
             lds_addr(smem1 + 1024 * (w + kWaves * c)));
      copy16(rsrc_words(fg.igate + head * T, t_eff * 4), off,
             lds_addr(smem1 + 4 * kFusedMaxT + 1024 * (w + kWaves * c)));
    }
  }
  if constexpr (FUSED) {
    copy_q_half(0);
  } else {
#pragma unroll 4
    for (int i = 0; i < kBM / kWaves; ++i) {
      const int r = (kBM / kWaves) * w + i;
      const int64_t row = q0 + r;
      if (lane < C::CH)
        dma16(make_rsrc(q + hoff + row * d, row < T ? 2 * d : 0), vchunk,
              (r < kBM / 2 ? smem0 : smem1) + (r % (kBM / 2)) * C::RSK);
    }
  }

  // ---- FUSED: the scan of the gate-scan kernel (a 512-thread block over
  // 2048 positions, 4 per thread) over positions [0, q0 + 128), thread tid
  // running threads tid and tid + 256 of that block, so that the terms are
  // bitwise the gate-scan kernel's.  The Q block's second half is copied once
  // the gates have been read.
  if constexpr (FUSED) {
    using namespace scan;
    constexpr int kHalfT = kScanThreads / 2;
    static_assert(kHalfT == kThreads, "two scan threads per thread");
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(kQHalf));
    __syncthreads();
    float fr[2][kScanPer], iv[2][kScanPer];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int vt = tid + kHalfT * u;
      const int64_t p0 = int64_t(kScanPer) * vt;
      const float4 f4 = reinterpret_cast<const float4*>(smem1)[vt];
      const float4 i4 = reinterpret_cast<const float4*>(smem1 + 4 * kFusedMaxT)[vt];
      const float fa[kScanPer] = {f4.x, f4.y, f4.z, f4.w};
      const float ia[kScanPer] = {i4.x, i4.y, i4.z, i4.w};
#pragma unroll
      for (int e = 0; e < kScanPer; ++e) {  // padding: no forgetting, no input
        fr[u][e] = p0 + e < t_eff ? fa[e] : 0.0f;
        iv[u][e] = p0 + e < t_eff ? ia[e] : -INFINITY;
      }
    }
    __syncthreads();  // buffer 1 is refilled below
    copy_q_half(1);
    // a scan wave whose positions all lie at or past the workgroup's last
    // row holds padding only: it skips the logarithms and the per-position
    // terms, which nothing reads
    double fb[2][kScanPer] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
    bool active[2];
    Elem mine[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t p0 = int64_t(kScanPer) * (tid + kHalfT * u);
      active[u] = kScanPer * 64 * (w + kWaves * u) < q0 + kBM;  // uniform across the wave
      if (active[u]) to_log_forget(p0, t_eff, fg.exp_forget, fr[u], fb[u]);
      mine[u] = thread_elem(fb[u], iv[u]);
    }
    // the Q block's first half has landed meanwhile (all but the wave's last
    // kQHalf copies): waves 0, 1 read their Q^T fragments, and the first key
    // tile is copied into buffer 0 while the scan runs (taken to be tile 0
    // until the decay bounds say otherwise: a wave's copies land in order, so
    // a later copy of the same rows is the one that stays)
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(kQHalf));
    __syncthreads();
    if (w < 2) read_q_fragments();
    __syncthreads();
    {
      const TileSrc ts0 = tile_src(0);
      static_for<16>([&](auto ic) { row_copy(ts0, smem0, ic); });
    }
    Elem before[2], total;
    block_scan_halves(mine[0], mine[1], before[0], before[1], total);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t p0 = int64_t(kScanPer) * (tid + kHalfT * u);
      Terms tm;
      if (active[u]) position_terms(identity(), before[u], fb[u], iv[u], p0, t_eff, fg.half_ln_d, tm);
      if (active[u] && p0 < q0 + kBM) {
        *reinterpret_cast<float4*>(f_e + p0) = make_float4(tm.e[0], tm.e[1], tm.e[2], tm.e[3]);
        if ((p0 & (kBoundTile - 1)) == 0) f_kb[p0 / kBoundTile] = tm.cmax;
        if (p0 >= q0) {
          const int o = int(p0 - q0);
          *reinterpret_cast<double2*>(f_cd + o) = make_double2(tm.c[0], tm.c[1]);
          *reinterpret_cast<double2*>(f_cd + o + 2) = make_double2(tm.c[2], tm.c[3]);
          *reinterpret_cast<double2*>(f_r + o) = make_double2(tm.r[0], tm.r[1]);
          *reinterpret_cast<double2*>(f_r + o + 2) = make_double2(tm.r[2], tm.r[3]);
          *reinterpret_cast<float4*>(f_m + o) = make_float4(tm.m[0], tm.m[1], tm.m[2], tm.m[3]);
          if ((o & (kBoundTile - 1)) == 0) f_rb[o / kBoundTile] = tm.rmax;
#pragma unroll
          for (int e = 0; e < kScanPer; ++e)
            if (p0 + e < T) fg.m_out[head * T + p0 + e] = tm.m[e];
        }
      }
    }
    __syncthreads();
  }
  const double r_i = FUSED ? f_r[qi - q0] : rowt[head * Tp + qi];  // R_i, qi < Tp

  f32x16 acc[DP / 32];
#pragma unroll
  for (int b = 0; b < DP / 32; ++b) acc[b] = f32x16{};
  float bsum = 0.0f;

  const int64_t n_key_tiles = (T + kBN - 1) / kBN;
  const int64_t last_tile = (4 * I + 3 < n_key_tiles - 1) ? 4 * I + 3 : n_key_tiles - 1;
  const int64_t wave_last = (4 * I + w < n_key_tiles - 1) ? 4 * I + w : n_key_tiles - 1;

  // ---- decay-aware tile skipping.  A key tile J whose exponent bound (see
  // the workspace notes) is below kSkipLog2 for a wave's 32 rows contributes
  // exactly zero to them.  The workgroup starts its key loop at the first
  // tile some wave needs, and inside the loop each wave skips the products
  // of tiles it does not need.
  const int64_t nb32 = Tp / kBoundTile;
  auto row_bound = [&](int64_t r) {  // rowb of the 32-row block of row r (of this workgroup)
    return FUSED ? f_rb[(r - q0) / kBoundTile] : rowb[head * nb32 + r / kBoundTile];
  };
  auto key_bound = [&](int64_t J) {  // keyb of 32-key tile J
    return FUSED ? f_kb[J] : keyb[head * nb32 + J];
  };
  const double rb_w = row_bound(qw);
  auto tile_needed = [&](double rb, double kb) { return rb + kb >= kSkipLog2; };
  int64_t first_tile = 0;
  if (skip) {
    __shared__ int64_t s_first[kWaves];
    double rb_rows[kWaves];
    int64_t last_w[kWaves];
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      const int64_t qu = q0 + 32 * u;
      rb_rows[u] = row_bound(qu);
      last_w[u] = (4 * I + u < n_key_tiles - 1) ? 4 * I + u : n_key_tiles - 1;
    }
    int64_t mine = last_tile;  // the diagonal tile of wave 0 bounds the answer
    for (int64_t J = tid; J < last_tile; J += kThreads) {
      const double kb = key_bound(J);
      bool need = false;
#pragma unroll
      for (int u = 0; u < kWaves; ++u)
        need = need || (J <= last_w[u] && tile_needed(rb_rows[u], kb));
      if (need) {
        mine = J;
        break;  // J grows with each iteration: the first hit is this thread's least
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const int64_t o = __shfl_xor(mine, off, 64);
      mine = o < mine ? o : mine;
    }
    if (lane == 0) s_first[w] = mine;
    __syncthreads();
    first_tile = s_first[0];
#pragma unroll
    for (int u = 1; u < kWaves; ++u) first_tile = s_first[u] < first_tile ? s_first[u] : first_tile;
  }

  // ---- global -> LDS copies of tile J: each wave copies 8 K rows and 8 V
  // rows.  The buffer ranges end at the last key of the sequence, so rows
  // past it arrive as zeros; head-dimension padding reads an out-of-range
  // offset.  load_tile (builtin copies) serves the first tile without FUSED.
  auto load_tile = [&](int64_t J, char* buf) {
    const int64_t k0 = J * kBN;
    const int64_t nrec = (T - k0 < kBN ? T - k0 : kBN) * int64_t(d) * 2;
    const auto rk = make_rsrc(k + hoff + k0 * d, nrec);
    const auto rv = make_rsrc(v + hoff + k0 * d, nrec);
#pragma unroll
    for (int i = 0; i < kBN / kWaves; ++i) {
      const int r = w * (kBN / kWaves) + i;
      if (lane < C::CH) {
        const unsigned off = lane < dch ? unsigned(r * d * 2 + 16 * lane) : kOutOfRange;
        dma16(rk, off, buf + r * C::RSK);
        dma16(rv, off, buf + C::K_BYTES + r * C::RSV);
      }
    }
    if (w == 0 && lane < kBN / 2)
      dma16(make_rsrc(colt + head * Tp + k0, kBN * 8), unsigned(16 * lane), buf + C::C_OFF);
    if (w == 1 && lane < kBN / 4)
      dma16(make_rsrc(colx + head * Tp + k0, kBN * 4), unsigned(16 * lane), buf + C::E_OFF);
    if (w == 2 && lane < 2)
      dma4(make_rsrc(keyb + head * nb32 + J, 8), unsigned(4 * lane), buf + C::KB_OFF);
  };
  // In the loop the same copies go one row at a time (row_copy, above), spread
  // over the first product: row copy i (0 <= i < 16) is K row i (i < 8) or V
  // row i - 8 of this wave's share (one buffer range each); the tile's gate
  // terms are copied by gate_copies (FUSED: held in LDS instead).
  auto gate_copies = [&](int64_t J, char* buf) {
    if (FUSED) return;
    const int64_t k0 = J * kBN;
    if (w == 0 && lane < kBN / 2)
      copy16(rsrc_words(colt + head * Tp + k0, kBN * 8), unsigned(16 * lane),
             lds_addr(buf + C::C_OFF));
    if (w == 1 && lane < kBN / 4)
      copy16(rsrc_words(colx + head * Tp + k0, kBN * 4), unsigned(16 * lane),
             lds_addr(buf + C::E_OFF));
    if (w == 2 && lane < 2)
      copy4(rsrc_words(keyb + head * nb32 + J, 8), unsigned(4 * lane), lds_addr(buf + C::KB_OFF));
  };
  // whether this wave's rows need tile J (copied into `buf`)
  auto wave_needs = [&](const char* buf, int64_t J) {
    if (J > wave_last) return false;
    if (!skip) return true;
    const double kb = FUSED ? f_kb[J] : *reinterpret_cast<const double*>(buf + C::KB_OFF);
    return tile_needed(rb_w, kb);
  };

  // per-lane LDS offsets of the operand reads
  const int koff = l32 * C::RSK + 16 * g;
  const int j16 = l32 & 15;
  const int voff = (4 * g + (j16 >> 2)) * C::RSV + 32 * (l32 >> 4) + 8 * (j16 & 3);

  // tile J from `buf`; during its first product the row copies of tile J + 1
  // (sources `ts`) go into `nxt` when `more`; the rest only when `needs`
  auto compute = [&](const char* buf, int64_t J, char* nxt, bool more, const TileSrc& ts,
                     bool needs) {
    // S^T = K_J Q^T, K fragments read kPf steps ahead (the scheduling
    // barriers stop the compiler from hoisting every LDS read of the
    // unrolled loop, which would cost a register per read)
    f32x16 st = f32x16{};
    {
      const char* kp = buf + koff;
      constexpr int NS = DP / 16;
      bf16x8 kf[kPf + 1];
#pragma unroll
      for (int t = 0; t < kPf && t < NS; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(kp + 32 * t);
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        if (t + kPf < NS)
          kf[(t + kPf) % (kPf + 1)] = *reinterpret_cast<const bf16x8*>(kp + 32 * (t + kPf));
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % (kPf + 1)], qf[t], st, 0, 0, 0);
        static_for<16>([&](auto ic) {
          if ((decltype(ic)::value * NS) / 16 == t && more) row_copy(ts, nxt, ic);
        });
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // A wave that needs none of the tile stops here.  (Issuing its copies
    // back to back instead of running the first product would be a second
    // copy site, and that makes the compiler spill the Q^T fragments.)
    if (!needs) return;
    // lane (g, l32), register r holds S^T[key 8(r/4) + 4g + r%4][query l32]
    const bool diag = (J * kBN == qw);
    float cv[16];
    if (diag) {
      // the diagonal tile: each entry's own exponential 2^(R_i + C_j) under
      // the causal mask (Eq. 71); the tile's column terms are read together,
      // before any is used
      const double* cb =
          FUSED ? f_cd + (J * kBN - q0) : reinterpret_cast<const double*>(buf + C::C_OFF);
      double2 cd[8];
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        cd[2 * rq] = *reinterpret_cast<const double2*>(cb + 8 * rq + 4 * g);
        cd[2 * rq + 1] = *reinterpret_cast<const double2*>(cb + 8 * rq + 4 * g + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const double2 c01 = cd[2 * rq], c23 = cd[2 * rq + 1];
        const double cc[4] = {c01.x, c01.y, c23.x, c23.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 8 * rq + 4 * g + e;
          const float ex = key > l32 ? -INFINITY : float(r_i + cc[e]);
          const float c = st[4 * rq + e] * __builtin_amdgcn_exp2f(ex);  // C~' (Eq. 82)
          bsum += c;                                                 // b (Eq. 83)
          cv[4 * rq + e] = c;
        }
      }
    } else {
      // below the diagonal the exponent factors as 2^(R_i + keyb_J) * e_j:
      // one exponential per row and tile; the tile's key factors and bound
      // are read together, before any is used
      const float* ge = FUSED ? f_e + J * kBN : reinterpret_cast<const float*>(buf + C::E_OFF);
      float4 e4[4];
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) e4[rq] = *reinterpret_cast<const float4*>(ge + 8 * rq + 4 * g);
      const double kb = FUSED ? f_kb[J] : *reinterpret_cast<const double*>(buf + C::KB_OFF);
      __builtin_amdgcn_sched_barrier(0);
      const float ei = __builtin_amdgcn_exp2f(float(r_i + kb));
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float ee[4] = {e4[rq].x, e4[rq].y, e4[rq].z, e4[rq].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = st[4 * rq + e] * (ei * ee[e]);  // C~' (Eq. 82)
          bsum += c;                                      // b (Eq. 83)
          cv[4 * rq + e] = c;
        }
      }
    }
    bf16x8 p[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[0][e] = (__bf16)cv[e];
      p[1][e] = (__bf16)cv[8 + e];
    }
    // O^T += V_J^T C~'^T.  Step t = (column block b, key half s): the A operand
    // holds V[16s + 4g + 0..3][32b + l32] and V[16s + 8 + 4g + 0..3][32b + l32],
    // the keys of B-operand registers 8s..8s+7.
    {
      const char* vp = buf + C::K_BYTES + voff;
      constexpr int NV = DP / 16;
      i16x4 vlo[kPf + 1], vhi[kPf + 1];
      auto vaddr = [&](int t) { return vp + 16 * (t & 1) * C::RSV + 64 * (t >> 1); };
#pragma unroll
      for (int t = 0; t < kPf && t < NV; ++t) {
        vlo[t] = tr_read(vaddr(t));
        vhi[t] = tr_read(vaddr(t) + 8 * C::RSV);
      }
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const int tn = t + kPf;
        if (tn < NV) {
          vlo[tn % (kPf + 1)] = tr_read(vaddr(tn));
          vhi[tn % (kPf + 1)] = tr_read(vaddr(tn) + 8 * C::RSV);
        }
        const i16x8 a16 = __builtin_shufflevector(vlo[t % (kPf + 1)], vhi[t % (kPf + 1)], 0, 1,
                                                  2, 3, 4, 5, 6, 7);
        acc[t >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a16), p[t & 1], acc[t >> 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (!FUSED || w >= 2) read_q_fragments();
  __syncthreads();  // the buffers are refilled below
  if constexpr (FUSED) {
    if (first_tile != 0) {
      const TileSrc ts = tile_src(first_tile);
      static_for<16>([&](auto ic) { row_copy(ts, smem0, ic); });
    }
  } else {
    load_tile(first_tile, smem0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // No plain global load is issued inside the loop: everything a tile needs
  // (K, V and its gate terms) arrives by the copies into LDS or is there from
  // the prologue's scan, so the waits on those copies stay exact.
  // one tile: its first product carries the row copies of the next tile
  auto step = [&](const char* buf, int64_t J, char* nxt) {
    const bool more = J + 1 <= last_tile;
    const TileSrc ts = tile_src(J + 1);
    if (more) gate_copies(J + 1, nxt);
    compute(buf, J, nxt, more, ts, wave_needs(buf, J));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int64_t J = first_tile; J <= last_tile; J += 2) {
    step(smem0, J, smem1);  // even tile from smem0, prefetch into smem1
    if (J + 1 > last_tile) break;
    step(smem1, J + 1, smem0);  // odd tile from smem1, prefetch into smem0
  }

  // ---- epilogue: n (Eq. 84), h~ = acc / n (Eqs. 85, 86), and with an
  // output gate H = sigma(O~) (.) h~ (Eq. 78) from the float32 h~ ----
  bsum += __shfl_xor(bsum, 32, 64);
  const float m_q = qi < T ? (FUSED ? f_m[qi - q0] : m_in[head * T + qi]) : 0.0f;
  const float nn = fmaxf(fabsf(bsum), expf(-m_q));
  const float inv = 1.0f / nn;
  if (qi < T && g == 0) {
    n_out[head * T + qi] = nn;
    if (b_out) b_out[head * T + qi] = bsum;
  }
  if (ogate == nullptr && htilde == nullptr) {
    // bf16(h~) goes through LDS (the tile buffers are free now): the block's
    // rows at the K rows' padded stride, rows 0..63 in buffer 0 and 64..127
    // in buffer 1, columns in order; then the block's rows, contiguous in
    // memory, are stored 1 KiB per instruction.  Rows past the sequence end
    // fall outside the buffer range and are not written.
    char* const obuf = (w < 2 ? smem0 : smem1) + (32 * (w & 1) + l32) * C::RSK;
#pragma unroll
    for (int b = 0; b < DP / 32; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = 32 * b + 8 * rq + 4 * g;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[b][4 * rq + e] * inv);
        *reinterpret_cast<bf16x4*>(obuf + 2 * col) = o;
      }
    }
    __syncthreads();
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const int64_t rows = T - q0 < kBM ? T - q0 : kBM;
    const auto rh = make_rsrc(h_out + hoff + q0 * d, rows * d * 2);
    const int nstore = d / 4;  // 1 KiB stores of the 128 x d block
#pragma unroll
    for (int u = 0; u < (DP / 4 + kWaves - 1) / kWaves; ++u) {
      const int n = w + kWaves * u;
      if (n < nstore) {
        const int gb = 1024 * n + 16 * lane;
        const int r = gb / row_bytes;
        const int c = (gb - r * row_bytes) >> 4;
        const u32x4 val = *reinterpret_cast<const u32x4*>(
            (r < kBM / 2 ? smem0 : smem1) + (r % (kBM / 2)) * C::RSK + 16 * c);
        __builtin_amdgcn_raw_buffer_store_b128(val, rh, gb, 0, 0);
      }
    }
  } else if (qi < T) {
    const int64_t row = hoff + qi * d;
#pragma unroll
    for (int b = 0; b < DP / 32; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = 32 * b + 8 * rq + 4 * g;
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

template <int DP, bool FUSED>
hipError_t launch_dp(const void* q, const void* k, const void* v, const float* m,
                     const Workspace& ws, void* h_out, float* n_out, const Epilogue& ep,
                     bool skip, int64_t H, int64_t T, int64_t d, const FusedGates& fg,
                     hipStream_t stream) {
  const int64_t row_tiles = (T + kBM - 1) / kBM;
  hipLaunchKernelGGL((tiles_mfma_kernel<DP, FUSED>), dim3(unsigned(row_tiles * H)),
                     dim3(kThreads), 0, stream, static_cast<const u16*>(q),
                     static_cast<const u16*>(k), static_cast<const u16*>(v), m, ws.rowt, ws.colt,
                     ws.colx, static_cast<u16*>(h_out), ws.rowb, ws.keyb, n_out,
                     static_cast<const u16*>(ep.ogate), static_cast<u16*>(ep.htilde), ep.b, T,
                     int(d), ws.Tp, row_tiles, H, int(skip), fg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tiles_mfma(const void* q, const void* k, const void* v, const float* m,
                             const Workspace& ws, void* h_out, float* n_out,
                             const Epilogue& ep, bool skip, int64_t H, int64_t T,
                             int64_t d, hipStream_t stream) {
  const FusedGates none{};
#define MLSTM_DP(n) launch_dp<32 * n, false>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, none, stream)
  // head dims are padded up to a multiple of 32 (zero columns add nothing)
  switch ((d + 31) / 32) {
    case 1: return MLSTM_DP(1);
    case 2: return MLSTM_DP(2);
    case 3: return MLSTM_DP(3);
    case 4: return MLSTM_DP(4);
    case 5: return MLSTM_DP(5);
    case 6: return MLSTM_DP(6);
    case 7: return MLSTM_DP(7);
    case 8: return MLSTM_DP(8);
    case 9: return MLSTM_DP(9);
    case 10: return MLSTM_DP(10);
    case 11: return MLSTM_DP(11);
    case 12: return MLSTM_DP(12);
    case 13: return MLSTM_DP(13);
    case 14: return MLSTM_DP(14);
    case 15: return MLSTM_DP(15);
    case 16: return MLSTM_DP(16);
    default: return hipErrorInvalidValue;
  }
#undef MLSTM_DP
}

bool tiles_mfma_fused_supports(int64_t T, int64_t d) {
  return d > 384 && d <= 512 && d % 16 == 0 && T >= 1 && T <= kFusedMaxT && T % 4 == 0;
}

hipError_t launch_tiles_mfma_fused(const void* q, const void* k, const void* v,
                                   const float* igate, const float* fgate, void* h_out,
                                   float* m_out, float* n_out, const Epilogue& ep,
                                   bool exp_forget, int64_t H, int64_t T, int64_t d,
                                   hipStream_t stream) {
  if (!tiles_mfma_fused_supports(T, d)) return hipErrorInvalidValue;
  Workspace none{};
  none.Tp = padded_len(T);
  FusedGates fg;
  fg.igate = igate;
  fg.fgate = fgate;
  fg.m_out = m_out;
  fg.half_ln_d = 0.5 * log(double(d));
  fg.exp_forget = int(exp_forget);
#define MLSTM_DP(n) launch_dp<32 * n, true>(q, k, v, nullptr, none, h_out, n_out, ep, true, H, T, d, fg, stream)
  switch ((d + 31) / 32) {
    case 13: return MLSTM_DP(13);
    case 14: return MLSTM_DP(14);
    case 15: return MLSTM_DP(15);
    case 16: return MLSTM_DP(16);
    default: return hipErrorInvalidValue;
  }
#undef MLSTM_DP
}

}  // namespace mlstm
