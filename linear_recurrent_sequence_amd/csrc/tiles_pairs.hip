// Stage 2, bf16 matrix-core variant with two waves per SIMD: Eqs. 81-86 of
// the xLSTM appendix over causal tiles, both contractions on gfx950 MFMA
// (v_mfma_f32_32x32x16_bf16, float32 accumulation).
//
// Why two waves per SIMD.  A wave that issues a global -> LDS copy, or a run
// of exponentials, cannot issue matrix instructions meanwhile; with one wave
// per SIMD the matrix core idles for that time.  With two, one wave's copies
// and exponentials run while the other wave's products keep the matrix core
// busy.  The register file then holds two waves of at most 256 registers, so
// a wave cannot keep both all of its queries' Q^T fragments and all of their
// output columns; the two waves of a SIMD share 32 query rows instead.
//
// Work decomposition.  A workgroup of 8 waves owns 128 query rows of one head.
// Wave w serves query block pq = w % 4 (rows 32 pq .. 32 pq + 31) as member
// hh = w / 4 of a pair.  The key axis is walked in super-steps of 64 keys;
// member hh owns key tile hh (32 keys) of each super-step for the first
// product and the 32-column output blocks 2b + hh for the second:
//   S^T_hh  = K_hh Q^T                      32 keys x 32 queries, full head dim
//   C~'^T_hh = S^T_hh (.) D'^T_hh,  b += column sums            (Eqs. 81-83)
//   members swap bf16(C~'^T) through LDS (2 KiB each)
//   O^T[own columns] += V^T[own columns, 64 keys] C~'^T[64 keys]
// so the matrix-core work per SIMD equals that of one wave with all columns,
// nothing is computed twice, and a wave holds the full Q^T (the B operand of
// the first product) but only half of the accumulators.  The row sums b of
// the two members are added once, at the end, in a fixed order.
//
// Data movement.  One K tile and one V tile of 64 keys live in LDS, each
// refilled while the other is read: during the first product of super-step
// s the copies bring V_s, during the second they bring K_{s+1} and its gate
// terms; each refill is spread over the matrix instructions of that phase.
// Copies are buffer_load_dwordx4 ... lds (global -> LDS, no registers), one
// padded row per instruction, issued through inline assembly so that the
// compiler does not wait for them before unrelated LDS reads; the kernel
// waits for its own copies (vmcnt) before each barrier.  In the key loop a
// wave's 8 rows of a tile share one buffer range and each copy forms its
// row's offsets itself, so a copy costs three scalar instructions besides the
// load rather than a buffer descriptor of its own.
//
// Exponents.  On a tile below the diagonal the exponent factors as
// 2^(R_i + keyb_J) * e_j with e_j from the gate scan (one exponential per
// query row and tile); on a diagonal tile every entry takes its own
// exponential 2^(R_i + C_j) under the causal mask (Eq. 71).  Each exponent is
// summed in float64 and rounded to float32 once.
//
// Fused gate scan (FUSED: at most 2048 positions, a multiple of 4).  Instead
// of reading the gate scan's terms from a workspace, each workgroup scans its
// head's gates from position 0 to its last row in its prologue, with the
// scan code of the gate-scan kernel (the same block structure, so the terms
// are bitwise the same), and keeps C_j, e_j and the tile bounds of all its
// keys in LDS; it writes m of its own rows.  The gate rows are copied into
// LDS ahead of the Q block, so the scan overlaps the Q copies.  The whole
// forward pass is then one launch with no workspace.
#include "mlstm_internal.h"
#include "scan_common.h"
#include "tile_common.h"

namespace mlstm {
namespace {

using namespace tilecommon;

constexpr int kWThreads = 512;  // 8 waves: two per SIMD
constexpr int kWWaves = kWThreads / 64;
constexpr int kSK = 64;   // keys per super-step (two 32-key tiles)
constexpr int kWPf = 3;   // LDS fragment prefetch distance (MFMA steps)
constexpr int kFusedMaxT = 2048;  // longest sequence of the fused gate scan (one scan chunk)
constexpr int kQCopies = 16;      // row copies per wave of the workgroup's Q block
constexpr int kWaitAllButQCopies = wait_vmcnt(kQCopies);
static_assert(kFusedMaxT == scan::kScanThreads * scan::kScanPer, "one block scan");

// LDS layout: rows are padded so that the fragment reads are free of bank
// conflicts (LDS serves 256 bytes per clock in 64 banks; a 16-byte read of
// 16 lanes, or an 8-byte read of 32 lanes, is conflict-free when the lanes hit
// distinct 16-byte, resp. 8-byte, slots modulo 256 bytes):
//  K rows (and the staged Q and output blocks): stride 2 DP + 16; the K
//   fragment read takes one 16-byte chunk of 16 consecutive rows, which then
//   start 16 (CH + 1) bytes apart with CH + 1 odd: 16 distinct slots.
//  V rows: stride 2 DP + 64; the transpose read takes one 64-byte group of
//   each of the 4 rows of an aligned quad, 64 (DP / 32 + 1) bytes apart with
//   DP / 32 + 1 odd: 4 distinct groups.
// Each row is copied by one instruction whose lanes fetch consecutive 16-byte
// chunks, so a copy needs no per-lane address arithmetic.
template <int DP, bool FUSED>
struct WCfg {
  static_assert(DP % 64 == 0 && DP >= 64 && DP <= 384, "head dim of the two-wave kernel");
  static constexpr int CH = DP / 8;          // 16-byte chunks per row
  static constexpr int RSK = 2 * DP + 16;    // K row stride (bytes)
  static constexpr int RSV = 2 * DP + 64;    // V row stride
  static constexpr int NB = DP / 64;         // 32-column output blocks per wave
  static constexpr int NS = DP / 16;         // MFMA steps of S^T
  static constexpr int RPW = kSK / kWWaves;  // rows of a 64-key tile copied per wave
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = kSK * RSK;
  static constexpr int GC = V_OFF + kSK * RSV;  // C_j of the K tile's 64 keys (float64)
  static constexpr int GE = GC + 512;        // e_j (float32)
  static constexpr int GB = GC + 768;        // keyb of the two 32-key tiles (float64)
  static constexpr int X_OFF = GC + 784;     // bf16(C~'^T) exchange, 2 KiB per wave
  // fused gate scan: the terms of every key and the workgroup's rows
  static constexpr int F_C = X_OFF + kWWaves * 2048;  // C_j of keys [0, 2048) (float64)
  static constexpr int F_E = F_C + kFusedMaxT * 8;    // e_j (float32)
  static constexpr int F_KB = F_E + kFusedMaxT * 4;   // keyb of each 32-key tile (float64)
  static constexpr int F_RB = F_KB + kFusedMaxT / 4;  // rowb of each 32-row block (float64)
  static constexpr int F_R = F_RB + kFusedMaxT / 4;   // R_i of the workgroup's 128 rows (float64)
  static constexpr int F_M = F_R + kBM * 8;           // m of those rows (float32)
  static constexpr int BYTES = FUSED ? F_M + kBM * 4 : X_OFF + kWWaves * 2048;
  static_assert(2 * kSK * RSK <= GC, "the staged Q block fits in the K and V regions");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int DP, bool FUSED>
__global__ __attribute__((amdgpu_flat_work_group_size(kWThreads, kWThreads),
                          amdgpu_waves_per_eu(2, 2))) void tiles_pairs_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ m_in, const double* __restrict__ rowt,
    const double* __restrict__ colt, const float* __restrict__ colx, u16* __restrict__ h_out,
    const double* __restrict__ rowb, const double* __restrict__ keyb, float* __restrict__ n_out,
    const u16* __restrict__ ogate, u16* __restrict__ htilde, float* __restrict__ b_out, int T,
    int d, int Tp, int row_tiles, int H, int skip, FusedGates fg) {
  using C = WCfg<DP, FUSED>;
  __shared__ __attribute__((aligned(1024))) char lds[C::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pq = w & 3;       // query block of this wave's pair
  const int hh = w >> 2;      // member: key tile of each super-step, output-column half
  const int g = lane >> 5;    // half-wave: selects 8 of the 16 reduction indices
  const int l32 = lane & 31;  // query column of this lane
  const int j16 = l32 & 15;
  int64_t I64, head64;
  map_tile(blockIdx.x, row_tiles, H, I64, head64);
  const int I = int(I64), head = int(head64);
  const int64_t hoff = int64_t(head) * T * d;
  const int q0 = I * kBM;
  const int qw = q0 + 32 * pq;  // first query row of this pair
  const int qi = qw + l32;      // query row of this lane
  const int dch = d / 8;            // real 16-byte chunks per row

  // Q^T fragments (full head dim): B operand of S^T = K Q^T, read from the
  // workgroup's Q block staged in LDS by the prologue
  bf16x8 qf[C::NS];

  f32x16 acc[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) acc[b] = f32x16{};
  float bsum = 0.0f;

  const int n_key_tiles = int((T + kBN - 1) / kBN);
  const int It = int(I);
  const int last_tile = (4 * It + 3 < n_key_tiles - 1) ? 4 * It + 3 : n_key_tiles - 1;
  const int pair_last = (4 * It + pq < n_key_tiles - 1) ? 4 * It + pq : n_key_tiles - 1;

  const int nb32 = Tp / kBoundTile;
  // ---- copies.  Tile of super-step s: key rows [64 s, 64 s + 64); the
  // buffer range ends at the sequence end, so rows past it arrive as zeros.
  // one row per copy: lanes [0, CH) fetch the row's 16-byte chunks (chunks
  // past the real head dimension read as zeros), lanes past CH stay idle.  A
  // row past the sequence end gets an empty buffer range and arrives as zeros.
  const unsigned vchunk = lane < dch ? unsigned(16 * lane) : kOutOfRange;
  auto copy_row = [&](const u16* src, int row, unsigned dst) {
    const i32x4 rs = rsrc_words(src + hoff + int64_t(row) * d, row < T ? 2 * d : 0);
    if (lane < C::CH) copy16(rs, vchunk, dst);
  };
  // row i (0 <= i < RPW) of this wave's share of the 64-key tile of super-step s
  // (prologue copies)
  auto copy_k = [&](int s, int i) {
    const int r = w + kWWaves * i;
    copy_row(k, s * kSK + r, lds_addr(lds + C::K_OFF + r * C::RSK));
  };
  // In the key loop a wave's RPW rows w + 8 i of a 64-key tile share one
  // buffer range, which ends before the first of them past the sequence end;
  // each row's offsets are formed inside its copy (copy16_row).
  const int row_step = kWWaves * 2 * d;  // bytes from one of a wave's rows to the next
  auto wave_rows = [&](const u16* src, int s) {
    const int r0 = s * kSK + w;
    const int left = T - r0;
    const int nv = left <= 0 ? 0 : (left + kWWaves - 1) / kWWaves;
    return rsrc_words(src + hoff + int64_t(r0) * d,
                      int64_t(nv < C::RPW ? nv : C::RPW) * row_step);
  };
  // the wave's row copies i with (i n) / RPW == t (all of them for t < 0):
  // its RPW row copies are spread over the n matrix instructions of a phase
  auto rows_at = [&](int t, int n, i32x4 rs, unsigned lds_base, auto stride) {
    static_for<C::RPW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if ((t < 0 || (i * n) / C::RPW == t) && lane < C::CH)
        copy16_row<i, i * kWWaves * decltype(stride)::value>(rs, vchunk, row_step, lds_base);
    });
  };
  using KStride = std::integral_constant<int, C::RSK>;
  using VStride = std::integral_constant<int, C::RSV>;
  const unsigned lds_k = lds_addr(lds + C::K_OFF + w * C::RSK);
  const unsigned lds_v = lds_addr(lds + C::V_OFF + w * C::RSV);

  // gate terms of super-step s: one small copy each for waves 0..2 (the
  // fused variant holds every key's terms in LDS from its prologue)
  auto copy_gates = [&](int s) {
    if (FUSED) return;
    const int k0 = s * kSK;
    if (w == 0 && lane < 32)
      copy16(rsrc_words(colt + int64_t(head) * Tp + k0, kSK * 8), unsigned(16 * lane),
             lds_addr(lds + C::GC));
    if (w == 1 && lane < 16)
      copy16(rsrc_words(colx + int64_t(head) * Tp + k0, kSK * 4), unsigned(16 * lane),
             lds_addr(lds + C::GE));
    if (w == 2 && lane < 1)
      copy16(rsrc_words(keyb + int64_t(head) * nb32 + k0 / kBoundTile, 16), 0u,
             lds_addr(lds + C::GB));
  };

  // ---- fused: the gate pre-activations of positions [0, t_eff) are copied
  // into LDS (the C_j region, which the scan rewrites only after reading
  // them) ahead of the Q block.  A wave's loads complete in order: a load
  // issued after the Q copies would wait for all of them, while these are
  // waited for alone (all but the wave's last kQCopies copies).  The fused
  // variant takes lengths divisible by 4 only, so that every head's gate row
  // starts 16-byte aligned.
  const int t_eff = T < q0 + kBM ? T : q0 + kBM;
  if constexpr (FUSED) {
    const unsigned off = unsigned(1024 * w + 16 * lane);
    copy16(rsrc_words(fg.fgate + int64_t(head) * T, int64_t(t_eff) * 4), off,
           lds_addr(lds + C::F_C + 1024 * w));
    copy16(rsrc_words(fg.igate + int64_t(head) * T, int64_t(t_eff) * 4), off,
           lds_addr(lds + C::F_C + 4 * kFusedMaxT + 1024 * w));
  }

  // ---- the workgroup's Q block (128 rows, contiguous in memory) is copied
  // into the K and V regions with the tiles' chunk permutation, overlapping
  // the gate scan and the first-tile search; the prologue reads the Q^T
  // fragments from there.
#pragma unroll
  for (int i = 0; i < kBM / kWWaves; ++i) {
    const int r = w + kWWaves * i;
    copy_row(q, q0 + r, lds_addr(lds + C::K_OFF + r * C::RSK));
  }

  // each wave's Q^T fragments (like K fragments) from the staged Q block
  auto read_q_fragments = [&]() {
    const int qrow = C::K_OFF + (32 * pq + l32) * C::RSK + 16 * g;
#pragma unroll
    for (int t = 0; t < C::NS; ++t) qf[t] = *reinterpret_cast<const bf16x8*>(lds + qrow + 32 * t);
  };

  // ---- fused gate scan of positions [0, q0 + 128) of the head while the Q
  // copies are in flight: thread tid owns positions 4 tid .. 4 tid + 3
  if constexpr (FUSED) {
    using namespace scan;
    const int64_t p0 = int64_t(kScanPer) * tid;
    static_assert(kBM / kWWaves == kQCopies, "Q copies per wave");
    __builtin_amdgcn_s_waitcnt(kWaitAllButQCopies);
    __syncthreads();
    const float4 f4 = reinterpret_cast<const float4*>(lds + C::F_C)[tid];
    const float4 i4 = reinterpret_cast<const float4*>(lds + C::F_C + 4 * kFusedMaxT)[tid];
    const float fa[kScanPer] = {f4.x, f4.y, f4.z, f4.w};
    const float ia[kScanPer] = {i4.x, i4.y, i4.z, i4.w};
    float fr[kScanPer], iv[kScanPer];
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {  // padding: no forgetting, no input
      fr[e] = p0 + e < t_eff ? fa[e] : 0.0f;
      iv[e] = p0 + e < t_eff ? ia[e] : -INFINITY;
    }
    // a wave whose positions all lie at or past the workgroup's last row
    // holds padding only (log f = 0, i~ = -inf): it skips the logarithms and
    // the per-position terms, which nothing reads
    const bool active = kScanPer * 64 * w < q0 + kBM;  // uniform across the wave
    double fb[kScanPer] = {0.0, 0.0, 0.0, 0.0};
    if (active) to_log_forget(p0, t_eff, fg.exp_forget, fr, fb);
    const Elem mine = thread_elem(fb, iv);
    // the Q block has landed meanwhile: its Q^T fragments are read, and the
    // first K tile is copied before the rest of the scan runs (the first
    // super-step is taken to be 0 until the decay bounds say otherwise)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    read_q_fragments();
    __syncthreads();  // the region is refilled below
#pragma unroll
    for (int i = 0; i < C::RPW; ++i) copy_k(0, i);
    Elem total;
    const Elem before = block_scan(mine, total);
    Terms tm;
    if (active) position_terms(identity(), before, fb, iv, p0, t_eff, fg.half_ln_d, tm);
    if (active && p0 < q0 + kBM) {
      double* fc = reinterpret_cast<double*>(lds + C::F_C) + p0;
      *reinterpret_cast<double2*>(fc) = make_double2(tm.c[0], tm.c[1]);
      *reinterpret_cast<double2*>(fc + 2) = make_double2(tm.c[2], tm.c[3]);
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(lds + C::F_E) + p0) =
          make_float4(tm.e[0], tm.e[1], tm.e[2], tm.e[3]);
      if ((p0 & (kBoundTile - 1)) == 0) {
        reinterpret_cast<double*>(lds + C::F_KB)[p0 / kBoundTile] = tm.cmax;
        reinterpret_cast<double*>(lds + C::F_RB)[p0 / kBoundTile] = tm.rmax;
      }
      if (p0 >= q0) {
        const int o = int(p0) - q0;
        double* fr2 = reinterpret_cast<double*>(lds + C::F_R) + o;
        *reinterpret_cast<double2*>(fr2) = make_double2(tm.r[0], tm.r[1]);
        *reinterpret_cast<double2*>(fr2 + 2) = make_double2(tm.r[2], tm.r[3]);
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(lds + C::F_M) + o) =
            make_float4(tm.m[0], tm.m[1], tm.m[2], tm.m[3]);
#pragma unroll
        for (int e = 0; e < kScanPer; ++e)
          if (p0 + e < T) fg.m_out[int64_t(head) * T + p0 + e] = tm.m[e];
      }
    }
    __syncthreads();
  }
  const double r_i = FUSED ? reinterpret_cast<const double*>(lds + C::F_R)[qi - q0]
                           : rowt[int64_t(head) * Tp + qi];  // R_i, qi < Tp
  auto row_bound = [&](int r) {  // rowb of the 32-row block of row r
    return FUSED ? reinterpret_cast<const double*>(lds + C::F_RB)[r / kBoundTile]
                 : rowb[int64_t(head) * nb32 + r / kBoundTile];
  };
  auto key_bound = [&](int J) {  // keyb of 32-key tile J
    return FUSED ? reinterpret_cast<const double*>(lds + C::F_KB)[J]
                 : keyb[int64_t(head) * nb32 + J];
  };

  // ---- decay-aware start of the key loop: the first 32-key tile some pair
  // needs (the bound of mlstm_internal.h); inside the loop each member skips
  // the products of tiles its rows do not need.
  const double rb_w = row_bound(qw);  // uniform across the wave
  auto tile_needed = [&](double rb, double kb) { return rb + kb >= kSkipLog2; };
  int first_tile = 0;
  if (skip) {
    __shared__ int s_first[kWWaves];
    double rb_rows[4];
    int last_p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int qu = q0 + 32 * u;
      rb_rows[u] = row_bound(qu);
      last_p[u] = (4 * It + u < n_key_tiles - 1) ? 4 * It + u : n_key_tiles - 1;
    }
    // the wave's least needed tile: lanes test J0 + tid in blocks of the
    // workgroup's threads; the first block with a hit in the wave holds it,
    // at its lowest hitting lane (a ballot, no lane-to-lane moves)
    int mine = last_tile;
    for (int J0 = 0; J0 < last_tile; J0 += kWThreads) {
      const int J = J0 + tid;
      bool need = false;
      if (J < last_tile) {
        const double kb = key_bound(J);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          need = need || (J <= last_p[u] && tile_needed(rb_rows[u], kb));
      }
      const uint64_t hits = __builtin_amdgcn_ballot_w64(need);
      if (hits != 0) {
        mine = J0 + 64 * w + int(__builtin_ctzll(hits));
        break;
      }
    }
    if (lane == 0) s_first[w] = mine;
    __syncthreads();
    first_tile = s_first[0];
#pragma unroll
    for (int u = 1; u < kWWaves; ++u) first_tile = s_first[u] < first_tile ? s_first[u] : first_tile;
    first_tile = __builtin_amdgcn_readfirstlane(first_tile);
  }
  const int s_first_step = first_tile / 2;
  const int s_last_step = last_tile / 2;

  // per-lane LDS offsets of the fragment reads.
  // K: row 32 hh + l32, bytes 32 t + 16 g for MFMA step t (immediate offsets).
  const int krow = C::K_OFF + (32 * hh + l32) * C::RSK + 16 * g;
  // V^T gather (ds_read_b64_tr_b16, as in the one-wave kernel): rows
  // 16 c + 4 g + j16 / 4 (+ 8) of a key tile, bytes 64 m + 32 (l32 / 16) +
  // 8 (j16 % 4), with m = 2 b + hh the 64-byte index of this member's
  // 32-column block b.
  const int vrow = C::V_OFF + (4 * g + (j16 >> 2)) * C::RSV + 32 * (l32 >> 4) + 8 * (j16 & 3) +
                   64 * hh;
  const int vown = vrow + 32 * hh * C::RSV;
  const int vpart = vrow + 32 * (hh ^ 1) * C::RSV;
  char* const xmine = lds + C::X_OFF + 2048 * w;
  const char* const xpart = lds + C::X_OFF + 2048 * (w ^ 4);

  // ---- prologue: each wave reads its Q^T fragments (like K fragments) from
  // the staged Q block; then K and the gate terms of the first super-step are
  // copied into the K region.  The fused variant read its fragments and
  // copied K_0 during the scan: it copies again only when the first
  // super-step is not 0 (a wave's copies land in order, so the later copy of
  // the same rows is the one that stays).
  if constexpr (!FUSED) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    read_q_fragments();
    __syncthreads();  // the region is refilled below
  }
  {
    if (!FUSED || s_first_step != 0) {
#pragma unroll
      for (int i = 0; i < C::RPW; ++i) copy_k(s_first_step, i);
      copy_gates(s_first_step);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  for (int s = s_first_step; s <= s_last_step; ++s) {
    // ===== phase 1: K_s and its gate terms are resident; copies bring V_s =====
    // the gate terms of the super-step's 64 keys (C_j, e_j, keyb of its tiles)
    const char* const g_c = FUSED ? lds + C::F_C + 8 * kSK * s : lds + C::GC;
    const char* const g_e = FUSED ? lds + C::F_E + 4 * kSK * s : lds + C::GE;
    const char* const g_b = FUSED ? lds + C::F_KB + 16 * s : lds + C::GB;
    // whether this member's and the partner's key tiles reach the pair's rows
    auto member_needs = [&](int hk) {
      const int J = 2 * s + hk;
      const double kb = *reinterpret_cast<const double*>(g_b + 8 * hk);
      const bool nd = J <= pair_last && (!skip || tile_needed(rb_w, kb));
      return __builtin_amdgcn_readfirstlane(int(nd)) != 0;
    };
    const bool need_own = member_needs(hh);
    const bool need_part = member_needs(hh ^ 1);
    const i32x4 rs_v = wave_rows(v, s);
    bf16x8 pown[2];
    if (need_own) {
      f32x16 st = f32x16{};
      bf16x8 kf[kWPf + 1];
      auto kaddr = [&](int t) { return lds + krow + 32 * t; };
#pragma unroll
      for (int t = 0; t < kWPf && t < C::NS; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(kaddr(t));
#pragma unroll
      for (int t = 0; t < C::NS; ++t) {
        if (t + kWPf < C::NS)
          kf[(t + kWPf) % (kWPf + 1)] = *reinterpret_cast<const bf16x8*>(kaddr(t + kWPf));
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % (kWPf + 1)], qf[t], st, 0, 0, 0);
        rows_at(t, C::NS, rs_v, lds_v, VStride{});
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane (g, l32), register r holds S^T[key 8(r/4) + 4g + r%4][query l32]
      const bool diag = (2 * s + hh) * kBN == qw;
      const double* gc = reinterpret_cast<const double*>(g_c) + 32 * hh;
      const float* ge = reinterpret_cast<const float*>(g_e) + 32 * hh;
      // C~' = S (.) D' in place of S (Eq. 82), b += C~' (Eq. 83)
      if (diag) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const double2 c01 = *reinterpret_cast<const double2*>(gc + 8 * rq + 4 * g);
          const double2 c23 = *reinterpret_cast<const double2*>(gc + 8 * rq + 4 * g + 2);
          const double cc[4] = {c01.x, c01.y, c23.x, c23.y};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = 8 * rq + 4 * g + e;
            // causal mask (Eq. 71)
            const float ex = key > l32 ? -INFINITY : float(r_i + cc[e]);
            st[4 * rq + e] *= __builtin_amdgcn_exp2f(ex);
            bsum += st[4 * rq + e];
          }
        }
      } else {
        // the tile's key factors and bound are read together, before any is
        // used: one LDS round trip instead of one per register group
        float4 e4[4];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) e4[rq] = *reinterpret_cast<const float4*>(ge + 8 * rq + 4 * g);
        const double kb = *reinterpret_cast<const double*>(g_b + 8 * hh);
        __builtin_amdgcn_sched_barrier(0);
        const float ei = __builtin_amdgcn_exp2f(float(r_i + kb));
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const float ee[4] = {e4[rq].x, e4[rq].y, e4[rq].z, e4[rq].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            st[4 * rq + e] *= ei * ee[e];
            bsum += st[4 * rq + e];
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pown[0][e] = (__bf16)st[e];
        pown[1][e] = (__bf16)st[8 + e];
      }
      *reinterpret_cast<bf16x8*>(xmine + 16 * lane) = pown[0];
      *reinterpret_cast<bf16x8*>(xmine + 1024 + 16 * lane) = pown[1];
    } else {
      rows_at(-1, 1, rs_v, lds_v, VStride{});
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ===== phase 2: V_s is resident; copies bring K_{s+1} and its gate terms =====
    const bool more = s < s_last_step;
    const i32x4 rs_k = wave_rows(k, s + 1);

    // The products run even when neither key tile reaches the pair's rows
    // (their operands are then zero): a branch around them would make the
    // compiler copy the accumulators.
    {
      const bf16x8 zero8 = bf16x8{};
      bf16x8 ppart[2] = {zero8, zero8};
      if (need_part) {
        ppart[0] = *reinterpret_cast<const bf16x8*>(xpart + 16 * lane);
        ppart[1] = *reinterpret_cast<const bf16x8*>(xpart + 1024 + 16 * lane);
      }
      if (!need_own) pown[0] = pown[1] = zero8;
      // O^T[own columns] += V^T C~'^T over the 64 keys, this member's key
      // tile first.  Step t = (column block b, key quarter c4): quarters 0, 1
      // are the own tile's keys 16 c + [0, 16), quarters 2, 3 the partner's;
      // the A operand holds V[16 c + 4g + 0..3][col + l32] and
      // V[16 c + 8 + 4g + 0..3][col + l32] of that tile.
      constexpr int NV = 4 * C::NB;

      auto vaddr = [&](int t) {
        const int b = t >> 2, c4 = t & 3;
        return lds + (c4 < 2 ? vown : vpart) + 128 * b + 16 * (c4 & 1) * C::RSV;
      };
      i16x4 vlo[kWPf + 1], vhi[kWPf + 1];
#pragma unroll
      for (int t = 0; t < kWPf && t < NV; ++t) {
        vlo[t] = tr_read(vaddr(t));
        vhi[t] = tr_read(vaddr(t) + 8 * C::RSV);
      }
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const int tn = t + kWPf;
        if (tn < NV) {
          vlo[tn % (kWPf + 1)] = tr_read(vaddr(tn));
          vhi[tn % (kWPf + 1)] = tr_read(vaddr(tn) + 8 * C::RSV);
        }
        const i16x8 a16 = __builtin_shufflevector(vlo[t % (kWPf + 1)], vhi[t % (kWPf + 1)], 0, 1,
                                                  2, 3, 4, 5, 6, 7);
        const int c4 = t & 3;
        const bf16x8 bop = c4 == 0 ? pown[0] : c4 == 1 ? pown[1] : c4 == 2 ? ppart[0] : ppart[1];
        acc[t >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16), bop,
                                                              acc[t >> 2], 0, 0, 0);
        if (more) rows_at(t, NV, rs_k, lds_k, KStride{});
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (more) copy_gates(s + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: b of the pair (member 0's keys first), n (Eq. 84),
  // h~ = acc / n (Eqs. 85, 86), output gate (Eq. 78) on this member's columns
  bsum += __shfl_xor(bsum, 32, 64);
  const float m_q = FUSED ? reinterpret_cast<const float*>(lds + C::F_M)[qi - q0]
                          : (qi < T ? m_in[int64_t(head) * T + qi] : 0.0f);
  reinterpret_cast<float*>(xmine)[lane] = bsum;
  __syncthreads();
  const float bpart = reinterpret_cast<const float*>(xpart)[lane];
  const float btot = hh == 0 ? bsum + bpart : bpart + bsum;
  const float nn = fmaxf(fabsf(btot), expf(-m_q));
  const float inv = 1.0f / nn;
  if (qi < T && g == 0 && hh == 0) {
    n_out[int64_t(head) * T + qi] = nn;
    if (b_out) b_out[int64_t(head) * T + qi] = btot;
  }
  if (ogate == nullptr && htilde == nullptr) {
    // bf16(h~) goes through LDS (the tile regions are free now): row
    // 32 pq + l32 of the block at the K rows' padded stride, columns in
    // order; then the block's rows, contiguous in memory, are stored 1 KiB
    // per instruction.  Rows past the sequence end fall outside the buffer
    // range and are not written.
    const int orow = C::K_OFF + (32 * pq + l32) * C::RSK;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = 32 * (2 * b + hh) + 8 * rq + 4 * g;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[b][4 * rq + e] * inv);
        *reinterpret_cast<bf16x4*>(lds + orow + 2 * col) = o;
      }
    }
    __syncthreads();
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const int rows = T - q0 < kBM ? T - q0 : kBM;
    const auto rh = make_rsrc(h_out + hoff + int64_t(q0) * d, int64_t(rows) * d * 2);
    const int nstore = d / 4;  // 1 KiB stores of the 128 x d block
    const int row_bytes = 2 * d;
#pragma unroll
    for (int u = 0; u < (DP / 4 + kWWaves - 1) / kWWaves; ++u) {
      const int n = w + kWWaves * u;
      if (n < nstore) {
        const int gb = 1024 * n + 16 * lane;
        const int r = gb / row_bytes;
        const int c = (gb - r * row_bytes) >> 4;
        const u32x4 val = *reinterpret_cast<const u32x4*>(
            lds + C::K_OFF + r * C::RSK + 16 * c);
        __builtin_amdgcn_raw_buffer_store_b128(val, rh, gb, 0, 0);
      }
    }
  } else if (qi < T) {
    const int64_t row = hoff + int64_t(qi) * d;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = 32 * (2 * b + hh) + 8 * rq + 4 * g;
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
hipError_t launch_w(const void* q, const void* k, const void* v, const float* m,
                    const Workspace& ws, void* h_out, float* n_out, const Epilogue& ep, bool skip,
                    int64_t H, int64_t T, int64_t d, const FusedGates& fg, hipStream_t stream) {
  const int64_t row_tiles = (T + kBM - 1) / kBM;
  hipLaunchKernelGGL((tiles_pairs_kernel<DP, FUSED>), dim3(unsigned(row_tiles * H)),
                     dim3(kWThreads), 0, stream, static_cast<const u16*>(q),
                     static_cast<const u16*>(k), static_cast<const u16*>(v), m, ws.rowt, ws.colt,
                     ws.colx, static_cast<u16*>(h_out), ws.rowb, ws.keyb, n_out,
                     static_cast<const u16*>(ep.ogate), static_cast<u16*>(ep.htilde), ep.b,
                     int(T), int(d), int(ws.Tp), int(row_tiles), int(H), int(skip), fg);
  return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_any(const void* q, const void* k, const void* v, const float* m,
                      const Workspace& ws, void* h_out, float* n_out, const Epilogue& ep,
                      bool skip, int64_t H, int64_t T, int64_t d, const FusedGates& fg,
                      hipStream_t stream) {
  // head dims are padded up to a multiple of 64 (zero columns add nothing)
  switch ((d + 63) / 64) {
    case 1: return launch_w<64, FUSED>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, fg, stream);
    case 2: return launch_w<128, FUSED>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, fg, stream);
    case 3: return launch_w<192, FUSED>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, fg, stream);
    case 4: return launch_w<256, FUSED>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, fg, stream);
    case 5: return launch_w<320, FUSED>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, fg, stream);
    case 6: return launch_w<384, FUSED>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, fg, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool tiles_pairs_supports(int64_t d) { return d % 16 == 0 && d >= 16 && d <= 384; }

bool tiles_pairs_fused_supports(int64_t T, int64_t d) {
  return tiles_pairs_supports(d) && T >= 1 && T <= kFusedMaxT && T % 4 == 0;
}

hipError_t launch_tiles_pairs(const void* q, const void* k, const void* v, const float* m,
                              const Workspace& ws, void* h_out, float* n_out, const Epilogue& ep,
                              bool skip, int64_t H, int64_t T, int64_t d, hipStream_t stream) {
  if (!tiles_pairs_supports(d)) return hipErrorInvalidValue;
  return launch_any<false>(q, k, v, m, ws, h_out, n_out, ep, skip, H, T, d, FusedGates{}, stream);
}

hipError_t launch_tiles_pairs_fused(const void* q, const void* k, const void* v,
                                    const float* igate, const float* fgate, void* h_out,
                                    float* m_out, float* n_out, const Epilogue& ep,
                                    bool exp_forget, int64_t H, int64_t T, int64_t d,
                                    hipStream_t stream) {
  if (!tiles_pairs_fused_supports(T, d)) return hipErrorInvalidValue;
  Workspace none{};
  none.Tp = padded_len(T);
  FusedGates fg;
  fg.igate = igate;
  fg.fgate = fgate;
  fg.m_out = m_out;
  fg.half_ln_d = 0.5 * log(double(d));
  fg.exp_forget = int(exp_forget);
  return launch_any<true>(q, k, v, nullptr, none, h_out, n_out, ep, true, H, T, d, fg, stream);
}

}  // namespace mlstm
