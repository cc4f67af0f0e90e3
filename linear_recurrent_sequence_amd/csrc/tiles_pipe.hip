// Stage 2 fused with stage 1, bf16 matrix-core variant with a software-
// pipelined key loop: Eqs. 79-86 of the xLSTM appendix ("Parallel mLSTM
// Forward Pass") over causal tiles, both contractions on gfx950 MFMA
// (v_mfma_f32_32x32x16_bf16, float32 accumulation), for head dimensions that
// are multiples of 64 up to 384 and sequences of at most 2048 positions.
// The forward pass takes it for d <= 192, where it is the fastest kernel
// (1.5x the two-wave pair kernel at d = 64, 1.25x at d = 128, 1.05x at
// d = 192 on 2048 positions); above that its register file runs out (the
// Q^T fragments, the d / 2 accumulators, the staged pieces and the operand
// prefetch of one wave per SIMD fill all 512 registers at d = 384) and the
// pair kernel, whose second wave per SIMD hides the latencies this one must
// cover alone, is faster.
//
// Work decomposition.  A workgroup of 4 waves (one per SIMD) owns 128 query
// rows of one head, 32 per wave (the N = 32 side of every MFMA), and walks
// the key axis in tiles of 32 keys up to its diagonal.  A wave holds its
// rows' Q^T fragments (the B operand of S^T = K Q^T) and all d output columns
// of O^T = V^T C~'^T, so no two waves exchange anything but the K and V tiles
// they share through LDS.
//
// Software pipeline.  Iteration J forms S_J = K_J Q^T and accumulates
// O += V_{J-1} P_{J-1} with the bf16 C~' of the previous tile (P), so the
// matrix core always has independent products in flight: the factor of
// every entry of tile J (Eq. 82) is formed while S_J runs, and each entry's
// product, row-sum term (Eq. 83) and bf16 rounding while the V product of the
// previous tile runs.  K and V each have two LDS buffers: iteration J reads
// K_J and V_{J-1} and fills the others with K_{J+1} and V_J.  One barrier
// per iteration.
//
// Staged copies.  A tile's K (or V) rows are one contiguous block of
// 64 d bytes in memory.  Each wave loads its share in 1 KiB pieces with
// ordinary buffer loads into registers, one iteration ahead, and writes them
// into the padded LDS rows at the start of the next iteration (ds_write_b128),
// so a copy costs two issue slots and the loads have a whole iteration to
// land; nothing waits on them at the barrier.  Buffer ranges end at the
// sequence end: rows past it arrive as zeros.
//
// Exponents, as in the other tile kernels: log2(D'_ij / sqrt(d)) = R_i + C_j
// with float64 terms from the gate scan.  Below the diagonal the factor is
// 2^(R_i + keyb_J) e_j (one exponential per row and tile); on the diagonal
// tile each entry takes its own exponential of R_i + C_j under the causal mask
// (Eq. 71).  Each exponent is summed in float64 and rounded once.  A tile whose
// bound is below kSkipLog2 for a wave's rows gets the factor 0 (its C~' is
// exactly zero).
//
// Gate scan.  Each workgroup scans its head's gates from position 0 to its
// last row in its prologue with the gate-scan kernel's block scan (512 scan
// threads over 2048 positions, two per thread, the same combinations in the
// same order, so every term is bitwise the gate-scan kernel's) and keeps e_j
// of every key before its last row, C_j of its diagonal keys, the key tiles'
// bounds, and R_i, the row bounds and m of its own rows in LDS.  The whole
// forward pass is one launch with no workspace.
#include "mlstm_internal.h"
#include "scan_common.h"
#include "tile_common.h"

namespace mlstm {
namespace {

using namespace tilecommon;

constexpr int kPThreads = 256;
constexpr int kPWaves = kPThreads / 64;
constexpr int kPPf = 3;  // LDS fragment prefetch distance of K (MFMA steps)
constexpr int kVPf = 3;  // and of V^T
constexpr int kPMaxT = scan::kScanThreads * scan::kScanPer;  // one block scan: 2048
constexpr int kPQRows = kBM / kPWaves;                        // Q rows copied per wave

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSgValu = 0x2;
constexpr int kSgMfma = 0x8;
constexpr int kSgVmemRead = 0x20;
constexpr int kSgDsRead = 0x100;
constexpr int kSgDsWrite = 0x200;

// LDS rows are padded as in the other tile kernels, so that the fragment
// reads are free of bank conflicts: K rows (and the staged Q block) at
// 2 d + 16 bytes, V rows at 2 d + 64 bytes.
template <int DP>
struct PCfg {
  static_assert(DP % 64 == 0 && DP >= 64 && DP <= 384, "head dim of the pipelined kernel");
  static constexpr int CH = DP / 8;       // 16-byte chunks per row
  static constexpr int ROWB = 2 * DP;     // bytes of a row in memory
  static constexpr int RSK = ROWB + 16;   // K row stride in LDS
  static constexpr int RSV = ROWB + 64;   // V row stride in LDS
  static constexpr int KT = kBN * RSK;    // one K tile
  static constexpr int VT = kBN * RSV;    // one V tile
  static constexpr int KB0 = 0, KB1 = KT, VB0 = 2 * KT, VB1 = 2 * KT + VT;
  static constexpr int RING = 2 * KT + 2 * VT;
  static constexpr int NS = DP / 16;      // MFMA steps of either product
  static constexpr int NCH = DP / 64;     // 1 KiB pieces per wave of a K (or V) tile
  // Q^T fragments held in accumulation registers: as many as fit beside
  // the d / 2 accumulation registers of O^T and the 16 of S^T (256 in all)
  static constexpr int NQA = (256 - DP / 2 - 16) / 4 < NS ? (256 - DP / 2 - 16) / 4 : NS;
  static_assert(kBM * RSK <= RING, "the staged Q block fits in the tile buffers");
};

// the LDS buffers an iteration uses: K_J (kc), K_{J+1} (kn), V_{J-1} (vp), V_J (vn)
struct Bufs {
  int kc, kn, vp, vn;
};

template <int DP>
__global__ __attribute__((amdgpu_flat_work_group_size(kPThreads, kPThreads),
                          amdgpu_waves_per_eu(1, 1))) void tiles_pipe_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    u16* __restrict__ h_out, float* __restrict__ n_out, const u16* __restrict__ ogate,
    u16* __restrict__ htilde, float* __restrict__ b_out, int T, int row_tiles, int H,
    FusedGates fg) {
  using C = PCfg<DP>;
  __shared__ __attribute__((aligned(1024))) char ring[C::RING];
  __shared__ __attribute__((aligned(16))) float gst[2 * kPMaxT];  // f~, i~ of the scan
  __shared__ __attribute__((aligned(16))) float f_e[kPMaxT];      // e_j of every key
  __shared__ __attribute__((aligned(16))) double f_cd[kBM];       // C_j of the diagonal keys
  __shared__ double f_kb[kPMaxT / kBoundTile];                    // keyb of every key tile
  __shared__ double f_rb[kBM / kBoundTile];                       // rowb of the row blocks
  __shared__ __attribute__((aligned(16))) double f_r[kBM];        // R_i of the rows
  __shared__ __attribute__((aligned(16))) float f_m[kBM];         // m of the rows
  __shared__ int s_first[kPWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;    // half-wave: selects 8 of the 16 reduction indices
  const int l32 = lane & 31;  // query column of this lane
  int64_t I64, head64;
  map_tile(blockIdx.x, row_tiles, H, I64, head64);
  const int I = int(I64), head = int(head64);
  const int64_t hoff = int64_t(head) * T * DP;
  const int q0 = I * kBM;
  const int qw = q0 + 32 * w;  // first query row of this wave
  const int qi = qw + l32;     // query row of this lane
  const int t_eff = T < q0 + kBM ? T : q0 + kBM;

  // ---- prologue copies (global -> LDS, no registers): the gate
  // pre-activations of positions [0, t_eff), then the workgroup's Q block,
  // 32 rows per wave.  A wave's loads complete in order, so the gates are
  // waited for alone (all but the wave's last kPQRows copies).
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const unsigned off = unsigned(1024 * (w + kPWaves * c) + 16 * lane);
    copy16(rsrc_words(fg.fgate + int64_t(head) * T, int64_t(t_eff) * 4), off,
           lds_addr(reinterpret_cast<char*>(gst) + 1024 * (w + kPWaves * c)));
    copy16(rsrc_words(fg.igate + int64_t(head) * T, int64_t(t_eff) * 4), off,
           lds_addr(reinterpret_cast<char*>(gst) + 4 * kPMaxT + 1024 * (w + kPWaves * c)));
  }
  const unsigned vchunk = unsigned(16 * lane);
  {
    const int r0 = q0 + kPQRows * w;
    const int left = T - r0;
    const int nrows = left <= 0 ? 0 : (left < kPQRows ? left : kPQRows);
    const i32x4 rs = rsrc_words(q + hoff + int64_t(r0) * DP, int64_t(nrows) * C::ROWB);
    const unsigned base = lds_addr(ring + kPQRows * w * C::RSK);
    static_for<kPQRows>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (lane < C::CH) copy16_row<i, i * C::RSK>(rs, vchunk, C::ROWB, base);
    });
  }

  // ---- the scan of the gate-scan kernel over positions [0, q0 + 128),
  // thread tid running scan threads tid and tid + 256
  using namespace scan;
  constexpr int kHalfT = kScanThreads / 2;
  static_assert(kHalfT == kPThreads, "two scan threads per thread");
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(kPQRows));
  __syncthreads();
  float fr[2][kScanPer], iv[2][kScanPer];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int vt = tid + kHalfT * u;
    const int p0 = kScanPer * vt;
    const float4 f4 = reinterpret_cast<const float4*>(gst)[vt];
    const float4 i4 = reinterpret_cast<const float4*>(gst + kPMaxT)[vt];
    const float fa[kScanPer] = {f4.x, f4.y, f4.z, f4.w};
    const float ia[kScanPer] = {i4.x, i4.y, i4.z, i4.w};
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {  // padding: no forgetting, no input
      fr[u][e] = p0 + e < t_eff ? fa[e] : 0.0f;
      iv[u][e] = p0 + e < t_eff ? ia[e] : -INFINITY;
    }
  }
  // a scan wave whose positions all lie at or past the workgroup's last row
  // holds padding only: it skips the logarithms and the per-position terms
  double fb[2][kScanPer] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  bool active[2];
  Elem mine[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p0 = kScanPer * (tid + kHalfT * u);
    active[u] = kScanPer * 64 * (w + kPWaves * u) < q0 + kBM;  // uniform across the wave
    if (active[u]) to_log_forget(p0, t_eff, fg.exp_forget, fr[u], fb[u]);
    mine[u] = thread_elem(fb[u], iv[u]);
  }

  // the Q block has landed meanwhile: each wave reads its rows' Q^T
  // fragments (like K fragments: 16 bytes of one row per lane)
  bf16x8 qf[C::NS];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  {
    // read into accumulation registers (the matrix instructions take their
    // B operand from there as well), which leaves the vector registers to
    // the staged copies; each read is waited for inside its own statement
    const unsigned qrow = lds_addr(ring + (kPQRows * w + l32) * C::RSK + 16 * g);
#pragma unroll
    for (int t = 0; t < C::NS; ++t) {
      if (t < C::NQA)
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                     : "=a"(qf[t])
                     : "v"(qrow + 32 * t)
                     : "memory");
      else
        qf[t] = *reinterpret_cast<const bf16x8*>(ring + (kPQRows * w + l32) * C::RSK + 16 * g +
                                                 32 * t);
    }
  }
  __syncthreads();  // the tile buffers are filled from here on

  // ---- staged copies.  Wave w moves rows 8 w .. 8 w + 7 of a 32-key tile
  // in NCH pieces of 1 KiB: lanes in groups of SEG, each group one run of
  // SEG 16-byte chunks of a row (256 bytes when the row allows, so that a
  // group's LDS write covers every bank once), RPP rows per piece.
  const int n_key_tiles = (T + kBN - 1) / kBN;
  const int last = (4 * I + 3 < n_key_tiles - 1) ? 4 * I + 3 : n_key_tiles - 1;
  const int wave_last = (4 * I + w < n_key_tiles - 1) ? 4 * I + w : n_key_tiles - 1;
  constexpr int SEG = C::CH % 16 == 0 ? 16 : 8;  // lanes per run
  constexpr int RPP = 64 / SEG;                  // rows per piece
  constexpr int PPR = C::CH / SEG;               // pieces per row group
  static_assert((8 / RPP) * PPR == C::NCH, "pieces cover the wave's 8 rows");
  const int prow = 8 * w + lane / SEG;  // row of this lane in the piece's first row group
  const unsigned goff = unsigned((lane / SEG) * C::ROWB + 16 * (lane % SEG));
  const unsigned kdst = unsigned(prow * C::RSK + 16 * (lane % SEG));
  const unsigned vdst = unsigned(prow * C::RSV + 16 * (lane % SEG));
  // offsets of piece i relative to the lane's first one
  auto piece_g = [](int i) { return (i / PPR) * RPP * C::ROWB + 16 * SEG * (i % PPR); };
  auto piece_k = [](int i) { return (i / PPR) * RPP * C::RSK + 16 * SEG * (i % PPR); };
  auto piece_v = [](int i) { return (i / PPR) * RPP * C::RSV + 16 * SEG * (i % PPR); };
  // this wave's rows of key tile J that the loop reads (none past `last`)
  auto tile_rsrc = [&](const u16* base, int J) {
    const int r0 = J * kBN + 8 * w;
    const int left = (J <= last ? T : 0) - r0;
    const int rows = left <= 0 ? 0 : (left < 8 ? left : 8);
    // uniform: kept in scalar registers (a range in vector registers would
    // make the compiler loop over the lanes' values around every load)
    const int nrec = __builtin_amdgcn_readfirstlane(rows * C::ROWB);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(base + hoff + int64_t(r0) * DP), 0,
                                             nrec, kRsrcFlags);
  };
  u32x4 stk[C::NCH], stv[C::NCH];
  auto load_k = [&](int J) {
    const auto rs = tile_rsrc(k, J);
#pragma unroll
    for (int i = 0; i < C::NCH; ++i)
      stk[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, goff + unsigned(piece_g(i)), 0, 0);
  };
  auto load_v = [&](int J) {
    const auto rs = tile_rsrc(v, J);
#pragma unroll
    for (int i = 0; i < C::NCH; ++i)
      stv[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, goff + unsigned(piece_g(i)), 0, 0);
  };
  // tile 0 is the first tile unless the decay bounds say otherwise
  load_k(0);
  load_v(0);

  Elem before[2], total;
  block_scan_halves(mine[0], mine[1], before[0], before[1], total);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p0 = kScanPer * (tid + kHalfT * u);
    Terms tm;
    if (active[u]) position_terms(identity(), before[u], fb[u], iv[u], p0, t_eff, fg.half_ln_d, tm);
    if (active[u] && p0 < q0 + kBM) {
      *reinterpret_cast<float4*>(f_e + p0) = make_float4(tm.e[0], tm.e[1], tm.e[2], tm.e[3]);
      if ((p0 & (kBoundTile - 1)) == 0) f_kb[p0 / kBoundTile] = tm.cmax;
      if (p0 >= q0) {
        const int o = p0 - q0;
        *reinterpret_cast<double2*>(f_cd + o) = make_double2(tm.c[0], tm.c[1]);
        *reinterpret_cast<double2*>(f_cd + o + 2) = make_double2(tm.c[2], tm.c[3]);
        *reinterpret_cast<double2*>(f_r + o) = make_double2(tm.r[0], tm.r[1]);
        *reinterpret_cast<double2*>(f_r + o + 2) = make_double2(tm.r[2], tm.r[3]);
        *reinterpret_cast<float4*>(f_m + o) = make_float4(tm.m[0], tm.m[1], tm.m[2], tm.m[3]);
        if ((o & (kBoundTile - 1)) == 0) f_rb[o / kBoundTile] = tm.rmax;
#pragma unroll
        for (int e = 0; e < kScanPer; ++e)
          if (p0 + e < T) fg.m_out[int64_t(head) * T + p0 + e] = tm.m[e];
      }
    }
  }
  __syncthreads();
  const double r_i = f_r[qi - q0];  // R_i
  const double rb_w = f_rb[w];      // rowb of this wave's rows (uniform)

  // ---- decay-aware start: the first 32-key tile some wave needs (the bound
  // of mlstm_internal.h); each wave gives a tile it does not need the factor 0
  auto tile_needed = [&](double rb, double kb) { return rb + kb >= kSkipLog2; };
  int first = 0;
  {
    double rb_rows[kPWaves];
    int last_w[kPWaves];
#pragma unroll
    for (int u = 0; u < kPWaves; ++u) {
      rb_rows[u] = f_rb[u];
      last_w[u] = (4 * I + u < n_key_tiles - 1) ? 4 * I + u : n_key_tiles - 1;
    }
    int mine_t = last;
    for (int J0 = 0; J0 < last; J0 += kPThreads) {
      const int J = J0 + tid;
      bool need = false;
      if (J < last) {
        const double kb = f_kb[J];
#pragma unroll
        for (int u = 0; u < kPWaves; ++u) need = need || (J <= last_w[u] && tile_needed(rb_rows[u], kb));
      }
      const uint64_t hits = __builtin_amdgcn_ballot_w64(need);
      if (hits != 0) {
        mine_t = J0 + 64 * w + int(__builtin_ctzll(hits));
        break;
      }
    }
    if (lane == 0) s_first[w] = mine_t;
    __syncthreads();
    first = s_first[0];
#pragma unroll
    for (int u = 1; u < kPWaves; ++u) first = s_first[u] < first ? s_first[u] : first;
    first = __builtin_amdgcn_readfirstlane(first);
  }
  if (first != 0) {
    load_k(first);
    load_v(first);
  }
  // K_first goes into K buffer 0 now; V_first and K_{first+1} are written by
  // the first iteration
#pragma unroll
  for (int i = 0; i < C::NCH; ++i)
    *reinterpret_cast<u32x4*>(ring + C::KB0 + kdst + piece_k(i)) = stk[i];
  load_k(first + 1);

  f32x16 acc[C::NS / 2];
#pragma unroll
  for (int b = 0; b < C::NS / 2; ++b) acc[b] = f32x16{};
  float bsum = 0.0f;
  bf16x8 pprev[2] = {bf16x8{}, bf16x8{}};  // bf16 C~'^T of the previous tile (B operand)

  // per-lane LDS offsets of the operand reads
  const int koff = l32 * C::RSK + 16 * g;
  const int j16 = l32 & 15;
  const int voff = (4 * g + (j16 >> 2)) * C::RSV + 32 * (l32 >> 4) + 8 * (j16 & 3);
  const int diag_tile = qw / kBN;  // this wave's diagonal tile

  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // One iteration: HS = tile J exists (S_J, its factors and C~', the staged
  // copies), HPV = tile J - 1 exists (its V product), TAIL = J may be some
  // wave's diagonal tile.
  auto iter = [&](auto hs_c, auto hpv_c, auto tail_c, int J, Bufs bf) {
    constexpr bool HS = decltype(hs_c)::value;
    constexpr bool HPV = decltype(hpv_c)::value;
    constexpr bool TAIL = decltype(tail_c)::value;
    f32x16 st = f32x16{};
    // entry e of the tile gets the factor ei * fct[e]: below the diagonal
    // fct holds e_j and ei = 2^(R_i + keyb_J); on the diagonal tile fct holds
    // each entry's exponential and ei = 1; a tile the wave does not need gets
    // ei = 0
    float fct[16];
    double kb = 0.0;
    float ei = 0.0f;
    // ---- S_J = K_J Q^T; the staged pieces (K_{J+1}, V_J) are written and
    // the next ones (K_{J+2}, V_{J+1}) loaded, spread over its steps; the
    // factors of tile J are formed meanwhile
    if constexpr (HS) {
      const char* kp = ring + bf.kc + koff;
      bf16x8 kf[kPPf + 1];
#pragma unroll
      for (int t = 0; t < kPPf && t < C::NS; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(kp + 32 * t);
      const auto rk = tile_rsrc(k, J + 2);
      const auto rv = tile_rsrc(v, J + 1);
      static_for<C::NS>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr (t + kPPf < C::NS)
          kf[(t + kPPf) % (kPPf + 1)] = *reinterpret_cast<const bf16x8*>(kp + 32 * (t + kPPf));
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % (kPPf + 1)], qf[t], st, 0, 0, 0);
        // piece c (K pieces first, then V) at step (c NS) / (2 NCH)
        static_for<2 * C::NCH>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if constexpr ((c * C::NS) / (2 * C::NCH) == t) {
            if constexpr (c < C::NCH) {
              *reinterpret_cast<u32x4*>(ring + bf.kn + kdst + piece_k(c)) = stk[c];
              stk[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, goff + unsigned(piece_g(c)), 0, 0);
            } else {
              constexpr int i = c - C::NCH;
              *reinterpret_cast<u32x4*>(ring + bf.vn + vdst + piece_v(i)) = stv[i];
              stv[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, goff + unsigned(piece_g(i)), 0, 0);
            }
          }
        });
        // the tile's key factors and bound (read together), then the row factor
        if constexpr (t == 0) {
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const float4 e4 = *reinterpret_cast<const float4*>(f_e + J * kBN + 8 * rq + 4 * g);
            fct[4 * rq] = e4.x;
            fct[4 * rq + 1] = e4.y;
            fct[4 * rq + 2] = e4.z;
            fct[4 * rq + 3] = e4.w;
          }
          kb = f_kb[J];
        }
        constexpr int t_ei = C::NS - 1 < 2 ? C::NS - 1 : 2;
        if constexpr (t == t_ei) {
          const bool need = J <= wave_last && tile_needed(rb_w, kb);
          ei = need ? __builtin_amdgcn_exp2f(float(r_i + kb)) : 0.0f;
        }
        // the order the scheduler keeps: this step's matrix instruction,
        // then its LDS reads, its piece's write and load, and VALU work
        constexpr int n_pieces = ((((t + 1) * 2 * C::NCH) + C::NS - 1) / C::NS) -
                                 (((t * 2 * C::NCH) + C::NS - 1) / C::NS);
        constexpr int n_reads = (t + kPPf < C::NS ? 1 : 0) + (t == 0 ? 5 : 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if constexpr (n_reads > 0) __builtin_amdgcn_sched_group_barrier(kSgDsRead, n_reads, 0);
        if constexpr (n_pieces > 0) {
          __builtin_amdgcn_sched_group_barrier(kSgDsWrite, n_pieces, 0);
          __builtin_amdgcn_sched_group_barrier(kSgVmemRead, n_pieces, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSgValu, 4, 0);
      });
      __builtin_amdgcn_sched_barrier(0);
      // Where a branch follows (the diagonal tile's factors, or the entries
      // right away in the first iteration), the compiler's own wait before
      // the first read of S^T has been measured too short (the last
      // registers of the tile read stale values); wait 24 cycles first.
      if constexpr (TAIL || !HPV) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (TAIL) {
        if (J == diag_tile) {
          // the diagonal tile: each entry's own exponential 2^(R_i + C_j)
          // under the causal mask (Eq. 71)
          const double* cb = f_cd + (J * kBN - q0);
          double2 cd[8];
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            cd[2 * rq] = *reinterpret_cast<const double2*>(cb + 8 * rq + 4 * g);
            cd[2 * rq + 1] = *reinterpret_cast<const double2*>(cb + 8 * rq + 4 * g + 2);
          }
          const bool need = J <= wave_last && tile_needed(rb_w, kb);
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const double cc4[4] = {cd[2 * rq].x, cd[2 * rq].y, cd[2 * rq + 1].x, cd[2 * rq + 1].y};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = 8 * rq + 4 * g + e;
              const float ex = key > l32 ? -INFINITY : float(r_i + cc4[e]);
              fct[4 * rq + e] = __builtin_amdgcn_exp2f(ex);
            }
          }
          ei = need ? 1.0f : 0.0f;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- O^T += V_{J-1}^T P_{J-1}^T; meanwhile C~' of tile J (Eq. 82), its
    // row-sum terms (Eq. 83, float32, before rounding) and bf16(C~'^T).
    // Step t = (column block b, key half s): the A operand holds
    // V[16 s + 4 g + 0..3][32 b + l32] and V[16 s + 8 + 4 g + 0..3][32 b + l32],
    // the keys of B-operand registers 8 s .. 8 s + 7.
    bf16x8 pnew[2];
    auto entry = [&](int e) {
      const float c = st[e] * (ei * fct[e]);  // C~' (Eq. 82)
      bsum += c;                       // b (Eq. 83)
      pnew[e >> 3][e & 7] = (__bf16)c;
    };
    if constexpr (HPV) {
      const char* vp = ring + bf.vp + voff;
      i16x4 vlo[kVPf + 1], vhi[kVPf + 1];
      auto vaddr = [&](int t) { return vp + 16 * (t & 1) * C::RSV + 64 * (t >> 1); };
#pragma unroll
      for (int t = 0; t < kVPf && t < C::NS; ++t) {
        vlo[t] = tr_read(vaddr(t));
        vhi[t] = tr_read(vaddr(t) + 8 * C::RSV);
      }
      static_for<C::NS>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr (t + kVPf < C::NS) {
          vlo[(t + kVPf) % (kVPf + 1)] = tr_read(vaddr(t + kVPf));
          vhi[(t + kVPf) % (kVPf + 1)] = tr_read(vaddr(t + kVPf) + 8 * C::RSV);
        }
        const i16x8 a16 = __builtin_shufflevector(vlo[t % (kVPf + 1)], vhi[t % (kVPf + 1)], 0, 1,
                                                  2, 3, 4, 5, 6, 7);
        acc[t >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16),
                                                              pprev[t & 1], acc[t >> 1], 0, 0, 0);
        if constexpr (HS) {
          // entry e at step 1 + (e (NS - 1)) / 16
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (t == 1 + (e * (C::NS - 1)) / 16) entry(e);
        }
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if constexpr (t + kVPf < C::NS) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSgValu, 6, 0);
      });
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (HS) {
#pragma unroll
      for (int e = 0; e < 16; ++e) entry(e);
    }
    if constexpr (HS) {
      pprev[0] = pnew[0];
      pprev[1] = pnew[1];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  using TrueC = std::integral_constant<bool, true>;
  using FalseC = std::integral_constant<bool, false>;
  // buffers by iteration parity x = J - first: K_J in K buffer x & 1, V_J in
  // V buffer x & 1
  constexpr Bufs kEven{C::KB0, C::KB1, C::VB1, C::VB0};
  constexpr Bufs kOdd{C::KB1, C::KB0, C::VB0, C::VB1};
  auto bufs_of = [&](int J) { return ((J - first) & 1) ? kOdd : kEven; };
  const int main_end = (last < 4 * I - 1) ? last : 4 * I - 1;  // tiles below every diagonal
  if (first >= 4 * I)
    iter(TrueC{}, FalseC{}, TrueC{}, first, kEven);
  else
    iter(TrueC{}, FalseC{}, FalseC{}, first, kEven);
  int J = first + 1;
  for (; J + 1 <= main_end; J += 2) {
    iter(TrueC{}, TrueC{}, FalseC{}, J, kOdd);
    iter(TrueC{}, TrueC{}, FalseC{}, J + 1, kEven);
  }
  if (J <= main_end) {
    iter(TrueC{}, TrueC{}, FalseC{}, J, kOdd);
    ++J;
  }
  for (; J <= last; ++J) iter(TrueC{}, TrueC{}, TrueC{}, J, bufs_of(J));
  iter(FalseC{}, TrueC{}, FalseC{}, last + 1, bufs_of(last + 1));

  // ---- epilogue: n (Eq. 84), h~ = acc / n (Eqs. 85, 86), and with an
  // output gate H = sigma(O~) (.) h~ (Eq. 78) from the float32 h~
  bsum += __shfl_xor(bsum, 32, 64);
  const float m_q = f_m[qi - q0];
  const float nn = fmaxf(fabsf(bsum), expf(-m_q));
  const float inv = 1.0f / nn;
  if (qi < T && g == 0) {
    n_out[int64_t(head) * T + qi] = nn;
    if (b_out) b_out[int64_t(head) * T + qi] = bsum;
  }
  if (ogate == nullptr && htilde == nullptr) {
    // bf16(h~) goes through LDS (the tile buffers are free after the last
    // barrier): the block's rows at the K rows' padded stride, columns in
    // order; then the block's rows, contiguous in memory, are stored 1 KiB
    // per instruction.  Rows past the sequence end fall outside the buffer
    // range and are not written.
    char* const obuf = ring + (32 * w + l32) * C::RSK;
#pragma unroll
    for (int b = 0; b < C::NS / 2; ++b) {
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
    const int rows = T - q0 < kBM ? T - q0 : kBM;
    const auto rh = make_rsrc(h_out + hoff + int64_t(q0) * DP, int64_t(rows) * C::ROWB);
    constexpr int nstore = DP / 4;  // 1 KiB stores of the 128 x d block
#pragma unroll
    for (int u = 0; u < (nstore + kPWaves - 1) / kPWaves; ++u) {
      const int n = w + kPWaves * u;
      if (n < nstore) {
        const int gb = 1024 * n + 16 * lane;
        const int r = gb / C::ROWB;
        const int c = (gb - r * C::ROWB) >> 4;
        const u32x4 val = *reinterpret_cast<const u32x4*>(ring + r * C::RSK + 16 * c);
        __builtin_amdgcn_raw_buffer_store_b128(val, rh, gb, 0, 0);
      }
    }
  } else if (qi < T) {
    const int64_t row = hoff + int64_t(qi) * DP;
#pragma unroll
    for (int b = 0; b < C::NS / 2; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = 32 * b + 8 * rq + 4 * g;
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

template <int DP>
hipError_t launch_p(const void* q, const void* k, const void* v, void* h_out, float* n_out,
                    const Epilogue& ep, int64_t H, int64_t T, const FusedGates& fg,
                    hipStream_t stream) {
  const int64_t row_tiles = (T + kBM - 1) / kBM;
  hipLaunchKernelGGL((tiles_pipe_kernel<DP>), dim3(unsigned(row_tiles * H)), dim3(kPThreads), 0,
                     stream, static_cast<const u16*>(q), static_cast<const u16*>(k),
                     static_cast<const u16*>(v), static_cast<u16*>(h_out), n_out,
                     static_cast<const u16*>(ep.ogate), static_cast<u16*>(ep.htilde), ep.b,
                     int(T), int(row_tiles), int(H), fg);
  return hipGetLastError();
}

}  // namespace

bool tiles_pipe_supports(int64_t T, int64_t d) {
  return d % 64 == 0 && d >= 64 && d <= 384 && T >= 1 && T <= kPMaxT && T % 4 == 0;
}

bool tiles_pipe_preferred(int64_t T, int64_t d) { return tiles_pipe_supports(T, d) && d <= 192; }

hipError_t launch_tiles_pipe(const void* q, const void* k, const void* v, const float* igate,
                             const float* fgate, void* h_out, float* m_out, float* n_out,
                             const Epilogue& ep, bool exp_forget, int64_t H, int64_t T,
                             int64_t d, hipStream_t stream) {
  if (!tiles_pipe_supports(T, d)) return hipErrorInvalidValue;
  FusedGates fg;
  fg.igate = igate;
  fg.fgate = fgate;
  fg.m_out = m_out;
  fg.half_ln_d = 0.5 * log(double(d));
  fg.exp_forget = int(exp_forget);
  switch (d / 64) {
    case 1: return launch_p<64>(q, k, v, h_out, n_out, ep, H, T, fg, stream);
    case 2: return launch_p<128>(q, k, v, h_out, n_out, ep, H, T, fg, stream);
    case 3: return launch_p<192>(q, k, v, h_out, n_out, ep, H, T, fg, stream);
    case 4: return launch_p<256>(q, k, v, h_out, n_out, ep, H, T, fg, stream);
    case 5: return launch_p<320>(q, k, v, h_out, n_out, ep, H, T, fg, stream);
    case 6: return launch_p<384>(q, k, v, h_out, n_out, ep, H, T, fg, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mlstm
