// Backward pass of the stabilized parallel mLSTM (xLSTM appendix A.3,
// "Parallel mLSTM Backward Pass", Eqs. 87-105) on gfx950 matrix cores, for
// bf16 inputs: the three tile passes of the float32 backward (backward.hip)
// with every contraction on v_mfma_f32_32x32x16_bf16 (float32 accumulation).
//
// Each pass is a variant of the one-wave forward tile kernel.  A workgroup of
// 4 waves (one per SIMD) owns 128 consecutive "own" rows of one head, 32 per
// wave, whose operands stay in registers as the B operand of the first
// products; the other axis is walked in tiles of 32 rows copied into LDS
// (double buffered, one barrier per tile).  A lane holds one own row and 16
// rows of the other axis of each 32 x 32 block (the accumulator layout):
//
//   rows pass (own = queries i, tiles of keys j):
//     S^T = K_J Q^T and G^T = V_J dH^T       (s_ij = q_i . k_j, g_ij = dh_i . v_j)
//     P_ij = E_ij (g_ij / n_i + db_i)        (E dC~', Eqs. 91-93)
//     r_i += sum_j s_ij P_ij                  (row sums of dD~ = C~' (.) dC~', Eq. 95)
//     dQ^T += K_J^T bf16(P^T)                 (Eq. 98)
//   keys pass (own = keys j, tiles of queries i):
//     S = Q_I K^T and G = dH_I V^T;  P as above
//     c_j += sum_i s_ij P_ij                  (column sums, Eqs. 97, 105)
//     dK^T += Q_I^T bf16(P)                   (Eq. 99)
//   values pass (own = keys j, tiles of queries i):
//     S = Q_I K^T;  dV^T += dH_I^T bf16(s_ij E_ij / n_i)     (Eq. 100)
//
// The values and rows passes need the S, G and E of the keys pass, so by
// default the keys pass stores the operands bf16(s_ij E_ij / n_i) (in the
// layout of the values pass's B fragments) and bf16(P) (key-major 32 x 32
// blocks, which the rows pass reads transposed), and those passes
// (kValuesStored, kRowsStored) only accumulate: dV is bitwise that of the
// recomputing pass, dQ equal up to the float32 rounding order of S and G.  A
// per-row kernel then forms 1/n_i, db_i and the row sums r_i of dD~ first
// (the keys pass reads 1/n and db); r_i from its closed form
// dh_i . h~_i + db_i b_i.  The own rows' fragments are staged through LDS (one
// copy per row) before the tile loop.  In the passes with first products, a wave's 16 row copies of
// the next tile are spread over the matrix instructions of its first
// products (a copy holds its wave at issue, and with one wave per SIMD that
// would idle the matrix core); those products therefore run on every tile,
// also where the wave's own rows take nothing from it.
//
// E_ij = D'_ij / sqrt(d) = 2^((A_i - A_j) + r_i + c_j) from the gate scan's
// terms, as in the forward pass (0 above the diagonal and past the sequence
// end).  The accumulation reads its first operand transposed from LDS with
// ds_read_b64_tr_b16, in the key order of the accumulator layout.  The sums
// r and c add float32 products of float32 values (no bf16 rounding); dQ, dK
// and dV carry the bf16 rounding of P, as the forward's h~ carries that of
// C~'.  When it recomputes S, the rows pass also forms the per-row scalars
// 1/n_i and db_i (Eqs. 88-90, from dh_i . h~_i) for its own rows and stores
// them for the two key passes.  The rows and keys passes hold two sets of own fragments and d / 2
// accumulator registers; above d = 384 that exceeds a wave's 512 registers,
// so there each of those passes is split over two workgroups per row block
// that recompute S and G and accumulate one half of the output columns each.
#include "mlstm_internal.h"
#include "tile_common.h"

namespace mlstm {
namespace {

using namespace tilecommon;

constexpr int kBThreads = 256;  // 4 waves, one per SIMD
constexpr int kBWaves = kBThreads / 64;
constexpr int kBPf = 2;         // LDS fragment prefetch distance (MFMA steps)

// kValuesStored / kRowsStored: the values / rows pass on the operand that the
// keys pass stored, bf16(C~'/n) / bf16(P) (no first products)
enum { kRowsPass = 0, kKeysPass = 1, kValuesPass = 2, kValuesStored = 3, kRowsStored = 4 };

// LDS layout of one buffer.  X1 is the tensor of the first product (K in the
// rows pass, Q otherwise), X2 that of the second product (V, dH) or, in the
// values pass, of the accumulation (dH).  A tensor read only by rows takes
// the stride 2 DP + 16 (16 consecutive rows hit 16 distinct 16-byte slots),
// one read only transposed 2 DP + 64 (the 4 rows of a quad hit 4 distinct
// 64-byte groups); X1 of the rows and keys passes is read both ways and takes
// 2 DP + 32, which costs at most a 2-way conflict for either read.
template <int DP, int MODE>
struct BCfg {
  static_assert(DP % 64 == 0 && DP >= 64 && DP <= 512, "head dim of the matrix-core backward");
  static constexpr bool VAL = MODE == kValuesPass || MODE == kValuesStored;
  static constexpr bool RST = MODE == kRowsStored;
  // output-column halves per row block (see the notes above)
  static constexpr int SPLIT = (!VAL && !RST && DP > 384) ? 2 : 1;
  static constexpr int NB = DP / 32 / SPLIT;  // 32-column accumulator blocks per wave
  static constexpr int CH = DP / 8;  // 16-byte chunks per row
  // X1 of the stored rows pass (K) is read only transposed
  static constexpr int S1 = RST ? 2 * DP + 64 : VAL ? 2 * DP + 16 : 2 * DP + 32;
  static constexpr int S2 = VAL ? 2 * DP + 64 : 2 * DP + 16;
  static constexpr int X1_OFF = 0;
  static constexpr int X2_OFF = MODE == kValuesStored ? 0 : kBN * S1;  // only dH: no X1
  static constexpr int GT = X2_OFF + kBN * S2;  // C_j (rows pass) or R_i of the tile, float64
  static constexpr int GN = GT + 256;           // 1 / n_i of the tile (keys, values passes)
  static constexpr int GD = GT + 384;           // db_i of the tile (keys pass)
  static constexpr int GEND = GT + 512;
  // the stored-operand values pass holds two consecutive dH tiles per buffer
  // (tile J at 0, tile J + 1 at GT), so it waits and synchronises once per
  // 64 queries: its 24 matrix instructions per tile do not cover a load's
  // latency
  // the stored rows pass: K rows, then bf16(P) of the workgroup's 4 query
  // tiles against the key tile (8 KiB); where four fit in LDS, two
  // consecutive tiles per buffer (tile J at 0, tile J + 1 at RT), like the
  // stored values pass
  static constexpr int P_OFF = kBN * S1;
  static constexpr int RT = P_OFF + 8192;
  static constexpr bool RPAIR = RST && 4 * RT <= 160 * 1024;
  static constexpr int BUF = MODE == kValuesStored ? 2 * GT : RPAIR ? 2 * RT : RST ? RT : GEND;
  static constexpr int SA = VAL ? S2 : S1;          // transposed operand's stride
  static constexpr int A_OFF = VAL ? X2_OFF : X1_OFF;
  static_assert(2 * BUF <= 160 * 1024, "LDS budget");
};

// The stored operand of the dV product: for each head, key block I (128
// keys) and 32-query tile J >= 4 I of the causal triangle, one 2 KiB slot per
// wave holding its bf16(C~'/n) fragments (lane L's first 16 bytes at 16 L,
// its second at 1024 + 16 L).  Slots of tiles J < 4 I + w, which wave w does
// not need, are neither written nor read.
__host__ __device__ inline int64_t store_tiles(int64_t T) {  // tiles of one head
  const int64_t nt = (T + kBN - 1) / kBN, rt = (T + kBM - 1) / kBM;
  return rt * nt - 2 * rt * (rt - 1);  // sum over I < rt of (nt - 4 I)
}

// The stored bf16(P) for the rows pass: for each head, key tile jk and query
// tile j >= jk, a 2 KiB block of the 32 keys' 64-byte rows, blocks in the
// order (jk, j) with j innermost.  Row r (key 32 jk + r) holds the tile's 32
// queries in the order of the keys pass's fragments: position p = 16 c + 8 g + i
// holds query q_of(p) = 16 c + 4 g + i + 4 (i / 4), so that each lane of the
// keys pass stores 16 contiguous bytes per fragment.
__host__ __device__ inline int64_t p_blocks(int64_t T) {  // blocks of one head
  const int64_t nt = (T + kBN - 1) / kBN;
  return nt * (nt + 1) / 2;
}
__device__ inline int64_t p_block(int64_t nt, int64_t jk, int64_t j) {
  return jk * nt - jk * (jk - 1) / 2 + (j - jk);
}
__device__ inline int q_of(int p) {
  return (p & ~15) + 4 * ((p >> 3) & 1) + (p & 7) + 4 * ((p >> 2) & 1);
}

// Per-row scalars of the stored-operand backward, one wave per row: 1/n_i;
// db_i = sign(b_i) dn_i with dn_i = -(dh_i . h~_i) / n_i where |b_i| is above
// the floor exp(-m_i), else 0 (Eqs. 88-90); and the row sum of dD~ (Eq. 95),
// r_i = sum_j C~'_ij dC~'_ij = dh_i . h~_i + db_i b_i, which follows from
// dC~'_ij = (dh_i . v_j) / n_i + db_i and sum_j C~'_ij v_j = n_i h~_i (Eqs. 83,
// 86).  (The rows pass that recomputes S forms these itself.)
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const u16* __restrict__ h, const u16* __restrict__ dh, const float* __restrict__ m,
    const float* __restrict__ n, const float* __restrict__ b, float* __restrict__ inv_n,
    float* __restrict__ db, float* __restrict__ rsum, int64_t rows, int d) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  // the row's scalars are loaded with its vectors, so that their latencies overlap
  const float nn = n[row], bb = b[row], mm = m[row];
  float acc = 0.0f;
  for (int c = 8 * lane; c < d; c += 512) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(dh + row * d + c);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(h + row * d + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += float(x[e]) * float(y[e]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) {
    const float dn = -acc / nn;
    const bool above_floor = fabsf(bb) > expf(-mm);
    const float dbv = above_floor ? (bb > 0.0f ? dn : (bb < 0.0f ? -dn : 0.0f)) : 0.0f;
    inv_n[row] = 1.0f / nn;
    db[row] = dbv;
    rsum[row] = acc + dbv * bb;
  }
}

// STORE (keys pass only): also store the values pass's operand.  Above
// d = 384 both workgroups of a row block store the same bytes (they compute
// the same S and E); a branch on the workgroup would cost the keys pass
// register spills.
template <int DP, int MODE, bool STORE>
__global__ __attribute__((amdgpu_flat_work_group_size(kBThreads, kBThreads),
                          amdgpu_waves_per_eu(1, 1))) void bwd_mfma_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dh, const u16* __restrict__ hsrc, const float* __restrict__ m_in,
    const float* __restrict__ n_in, const float* __restrict__ b_in, float* __restrict__ inv_n,
    float* __restrict__ db, const double* __restrict__ rowt, const double* __restrict__ colt,
    u16* __restrict__ out, float* __restrict__ sums, int T, int d, int Tp, int row_tiles, int H,
    u16* __restrict__ vstore, int64_t tri, u16* __restrict__ pstore, int64_t ptri) {
  using C = BCfg<DP, MODE>;
  constexpr bool kTwo = MODE == kRowsPass || MODE == kKeysPass;  // a second first product (G)
  constexpr bool kFirst = MODE != kValuesStored && MODE != kRowsStored;  // first products at all
  constexpr bool kRows = MODE == kRowsPass || MODE == kRowsStored;   // own rows are queries
  constexpr int NS = DP / 16;                 // MFMA steps of a first-stage product
  constexpr int NV = 2 * C::NB;               // MFMA steps of the accumulation
  const int cb0 = C::NB * int(blockIdx.y);    // first 32-column block of this workgroup
  // two distinct tile buffers, so that the copies into one never alias reads
  // of the other (one array would make the compiler wait for the copies
  // before reading); before the tile loop they stage the own rows, 64 each
  __shared__ __attribute__((aligned(1024))) char smem0[C::BUF];
  __shared__ __attribute__((aligned(1024))) char smem1[C::BUF];
  constexpr int RSQ = 2 * DP + 16;  // staging row stride: 16 consecutive rows hit
                                    // 16 distinct 16-byte slots
  static_assert(!kFirst || (kBM / 2) * RSQ <= C::BUF, "64 staged rows fit in a tile buffer");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int j16 = l32 & 15;
  int64_t I64, head64;
  map_tile(blockIdx.x, row_tiles, H, I64, head64);
  // heaviest blocks first: the last query blocks for the rows pass, the first
  // key blocks for the key passes
  const int I = kRows ? int(I64) : row_tiles - 1 - int(I64);
  const int head = int(head64);
  const int64_t hoff = int64_t(head) * T * d;
  const int ow = I * kBM + 32 * w;  // first own row of this wave
  const int oi = ow + l32;          // own row of this lane (< Tp)
  const int dch = d / 8;
  const int n_tiles = (T + kBN - 1) / kBN;

  const u16* own1 = MODE == kRowsPass ? q : k;
  const u16* own2 = MODE == kRowsPass ? dh : v;
  const u16* x1 = kRows ? k : q;
  const u16* x2 = MODE == kRowsPass ? v : dh;

  // own fragments (B operands): row oi, head dims 16 s + 8 g + 0..7; rows past
  // the sequence end and padded columns are zeros.  The workgroup's 128 own
  // rows of a tensor are staged in LDS with one copy per row (lanes fetch
  // consecutive 16-byte chunks), then each wave reads its 32 rows' fragments:
  // loading them straight from memory, 32 rows per instruction, was slower.
  const unsigned vchunk = lane < dch ? unsigned(16 * lane) : kOutOfRange;
  auto stage = [&](const u16* src) {
#pragma unroll 4
    for (int i = 0; i < kBM / kBWaves; ++i) {
      const int r = (kBM / kBWaves) * w + i;
      const int row = I * kBM + r;
      if (lane < C::CH)
        dma16(make_rsrc(src + hoff + int64_t(row) * d, row < T ? 2 * d : 0), vchunk,
              (r < kBM / 2 ? smem0 : smem1) + (r % (kBM / 2)) * RSQ);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  const char* const frow = (w < 2 ? smem0 : smem1) + (32 * (w & 1) + l32) * RSQ + 16 * g;
  auto read_frags = [&](bf16x8* f) {
#pragma unroll
    for (int s = 0; s < NS; ++s) f[s] = *reinterpret_cast<const bf16x8*>(frow + 32 * s);
  };
  bf16x8 f1[kFirst ? NS : 1];
  bf16x8 f2[kTwo ? NS : 1];
  if (kTwo) {
    stage(own2);
    read_frags(f2);
    __syncthreads();  // the staging space is refilled below
  }

  // own gate terms: R_i, 1/n_i, db_i (rows pass) or C_j (key passes; -inf past
  // the sequence end)
  const double own_t = !kFirst ? 0.0
                      : MODE == kRowsPass ? rowt[int64_t(head) * Tp + oi]
                                          : colt[int64_t(head) * Tp + oi];
  float own_in = 0.0f, own_db = 0.0f;
  if (MODE == kRowsPass) {
    // dn_i = -(dh_i . h~_i) / n_i (Eqs. 88-89); db_i = sign(b_i) dn_i where
    // |b_i| is above the floor exp(-m_i) (Eq. 90), else 0
    float hd = 0.0f;
    stage(hsrc);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 hv = *reinterpret_cast<const bf16x8*>(frow + 32 * s);
#pragma unroll
      for (int e = 0; e < 8; ++e) hd += float(f2[s][e]) * float(hv[e]);
    }
    __syncthreads();  // the staging space is refilled below
    hd += __shfl_xor(hd, 32, 64);
    if (oi < T) {
      const int64_t at = int64_t(head) * T + oi;
      const float nn = n_in[at], bb = b_in[at];
      const float dn = -hd / nn;
      const bool above_floor = fabsf(bb) > expf(-m_in[at]);
      own_in = 1.0f / nn;
      own_db = above_floor ? (bb > 0.0f ? dn : (bb < 0.0f ? -dn : 0.0f)) : 0.0f;
      if (g == 0 && blockIdx.y == 0) {  // for the key passes
        inv_n[at] = own_in;
        db[at] = own_db;
      }
    }
  }
  // the h~ fragments are dead before the Q fragments are loaded
  __builtin_amdgcn_sched_barrier(0);
  if (kFirst) {
    stage(own1);
    read_frags(f1);
    __syncthreads();  // the tile buffers are filled below
  }

  f32x16 acc[C::NB];
#pragma unroll
  for (int b = 0; b < C::NB; ++b) acc[b] = f32x16{};
  float dsum = 0.0f;

  // tiles of the other axis: keys 0 .. the diagonal (rows pass) or queries
  // from the diagonal to the end (key passes); per wave, the tiles that hold
  // some causal pair with its own rows
  const int first = kRows ? 0 : 4 * I;
  const int last = kRows ? (4 * I + 3 < n_tiles - 1 ? 4 * I + 3 : n_tiles - 1) : n_tiles - 1;
  auto wave_needs = [&](int J) { return kRows ? J <= 4 * I + w : J >= 4 * I + w; };

  auto load_tile = [&](int J, char* buf) {
    const int x0 = J * kBN;
    const int rows = T - x0 < kBN ? T - x0 : kBN;
    const int64_t nrec = int64_t(rows) * d * 2;
    const auto r1 = make_rsrc(x1 + hoff + int64_t(x0) * d, nrec);
    const auto r2 = make_rsrc(x2 + hoff + int64_t(x0) * d, nrec);
#pragma unroll
    for (int i = 0; i < kBN / kBWaves; ++i) {
      const int r = w * (kBN / kBWaves) + i;
      if (lane < C::CH) {
        const unsigned off = lane < dch ? unsigned(r * d * 2 + 16 * lane) : kOutOfRange;
        if (kFirst || MODE == kRowsStored) dma16(r1, off, buf + C::X1_OFF + r * C::S1);
        if (MODE != kRowsStored) dma16(r2, off, buf + C::X2_OFF + r * C::S2);
      }
    }
    if constexpr (MODE == kRowsStored) {
      // bf16(P) of key tile J against the query tiles 4 I .. 4 I + 3 (8 KiB,
      // contiguous; blocks the waves do not need, and blocks past the head's
      // last one, arrive as whatever precedes them, resp. zeros)
      const auto rp = make_rsrc(pstore + int64_t(head) * ptri * 1024, ptri * 2048);
      const unsigned base = unsigned(p_block(n_tiles, J, 4 * I) * 2048);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma16(rp, base + unsigned(1024 * (2 * w + i) + 16 * lane),
              buf + C::P_OFF + 1024 * (2 * w + i));
    }
    if (!kFirst) return;
    const double* tsrc = MODE == kRowsPass ? colt : rowt;
    if (w == 0 && lane < kBN / 2)
      dma16(make_rsrc(tsrc + int64_t(head) * Tp + x0, kBN * 8), unsigned(16 * lane), buf + C::GT);
    if (MODE != kRowsPass) {
      // per-row scalars of [H][T] arrays: 4 bytes per lane (rows need not be
      // 16-byte aligned); rows past the sequence end read as zeros
      if (w == 1 && lane < kBN)
        dma4(make_rsrc(inv_n + int64_t(head) * T + x0, int64_t(rows) * 4), unsigned(4 * lane),
             buf + C::GN);
      if (MODE == kKeysPass && w == 2 && lane < kBN)
        dma4(make_rsrc(db + int64_t(head) * T + x0, int64_t(rows) * 4), unsigned(4 * lane),
             buf + C::GD);
    }
  };

  // The rows and keys passes (and the recomputing values pass) copy a tile's
  // rows one at a time during the previous tile's first products: row copy
  // i (0 <= i < 16) is row i of this wave's 8 rows of X1 (i < 8) or of X2.
  struct TileSrc {
    i32x4 x1, x2;
  };
  auto tile_src = [&](int J) {
    const int r0 = J * kBN + w * (kBN / kBWaves);
    const int left = T - r0;
    const int64_t nrec =
        int64_t(left < 0 ? 0 : left < kBN / kBWaves ? left : kBN / kBWaves) * 2 * d;
    return TileSrc{rsrc_words(x1 + hoff + int64_t(r0) * d, nrec),
                   rsrc_words(x2 + hoff + int64_t(r0) * d, nrec)};
  };
  auto row_copy = [&](const TileSrc& ts, char* buf, auto ic) {
    constexpr int i = decltype(ic)::value;
    if (lane < C::CH) {
      if constexpr (i < 8)
        copy16_row<i & 7, (i & 7) * C::S1>(ts.x1, vchunk, 2 * d,
                                            lds_addr(buf + C::X1_OFF + w * (kBN / kBWaves) * C::S1));
      else
        copy16_row<i & 7, (i & 7) * C::S2>(ts.x2, vchunk, 2 * d,
                                            lds_addr(buf + C::X2_OFF + w * (kBN / kBWaves) * C::S2));
    }
  };
  // the tile's gate terms and per-row scalars (as in load_tile)
  auto small_copies = [&](int J, char* buf) {
    const int x0 = J * kBN;
    const int rows = T - x0 < kBN ? T - x0 : kBN;
    const double* tsrc = MODE == kRowsPass ? colt : rowt;
    if (w == 0 && lane < kBN / 2)
      copy16(rsrc_words(tsrc + int64_t(head) * Tp + x0, kBN * 8), unsigned(16 * lane),
             lds_addr(buf + C::GT));
    if (MODE != kRowsPass) {
      if (w == 1 && lane < kBN)
        copy4(rsrc_words(inv_n + int64_t(head) * T + x0, int64_t(rows) * 4), unsigned(4 * lane),
              lds_addr(buf + C::GN));
      if (MODE == kKeysPass && w == 2 && lane < kBN)
        copy4(rsrc_words(db + int64_t(head) * T + x0, int64_t(rows) * 4), unsigned(4 * lane),
              lds_addr(buf + C::GD));
    }
  };

  // per-lane LDS offsets: rows of X1 / X2 for the first products, the
  // transposed gather of the accumulation operand
  const int off1 = C::X1_OFF + l32 * C::S1 + 16 * g;
  const int off2 = C::X2_OFF + l32 * C::S2 + 16 * g;
  const int offt = C::A_OFF + (4 * g + (j16 >> 2)) * C::SA + 32 * (l32 >> 4) + 8 * (j16 & 3);

  // byte offset of this wave's slot of the stored dV operand for tile J
  auto slot = [&](int J) {
    const int64_t t = int64_t(I) * n_tiles - 2 * int64_t(I) * (I - 1) + (J - 4 * I);
    return ((int64_t(head) * tri + t) * kBWaves + w) * 2048;
  };

  // tile J from `buf`; during its first products the row copies of tile
  // J + 1 (sources `ts`) go into `nxt` when `more`; the rest only when `needs`
  auto compute = [&](const char* buf, int J, const bf16x8 (&pin)[2], char* nxt, bool more,
                     const TileSrc& ts, bool needs) {
    constexpr int NT = kTwo ? 2 * NS : NS;  // matrix instructions that carry the copies
    bf16x8 pb[2];
    if constexpr (MODE == kValuesStored) {
      pb[0] = pin[0];
      pb[1] = pin[1];
    } else if constexpr (MODE == kRowsStored) {
      // the B fragments P^T[keys][query q_of(l32)] from this wave's block of
      // the stored tile, read transposed like the accumulation's A operand
      // (the lane's accumulator column is query q_of(l32) of the wave)
      const char* pp = buf + C::P_OFF + 2048 * w + (4 * g + (j16 >> 2)) * 64 + 32 * (l32 >> 4) +
                       8 * (j16 & 3);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const i16x4 lo = tr_read(pp + 16 * c * 64);
        const i16x4 hi = tr_read(pp + 16 * c * 64 + 8 * 64);
        pb[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    } else {
    // first products: Y1 = X1_J Own1^T (and Y2 = X2_J Own2^T)
    f32x16 y1 = f32x16{}, y2 = f32x16{};
    {
      const char* p = buf + off1;
      bf16x8 kf[kBPf + 1];
#pragma unroll
      for (int t = 0; t < kBPf; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(p + 32 * t);
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        if (t + kBPf < NS)
          kf[(t + kBPf) % (kBPf + 1)] = *reinterpret_cast<const bf16x8*>(p + 32 * (t + kBPf));
        y1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % (kBPf + 1)], f1[t], y1, 0, 0, 0);
        static_for<16>([&](auto ic) {
          if ((decltype(ic)::value * NT) / 16 == t && more) row_copy(ts, nxt, ic);
        });
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (kTwo) {
      const char* p = buf + off2;
      bf16x8 kf[kBPf + 1];
#pragma unroll
      for (int t = 0; t < kBPf; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(p + 32 * t);
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        if (t + kBPf < NS)
          kf[(t + kBPf) % (kBPf + 1)] = *reinterpret_cast<const bf16x8*>(p + 32 * (t + kBPf));
        y2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % (kBPf + 1)], f2[t], y2, 0, 0, 0);
        static_for<16>([&](auto ic) {
          if ((decltype(ic)::value * NT) / 16 == NS + t && more) row_copy(ts, nxt, ic);
        });
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // a wave whose rows need none of the tile stops after the first products
    // (which carry the copies of the next tile)
    if (!needs) return;
    // lane (g, l32), register r: own row l32, other row 8(r/4) + 4g + r%4 of the tile
    const bool diag = J * kBN == ow;
    const double* gt = reinterpret_cast<const double*>(buf + C::GT);
    const float* gn = reinterpret_cast<const float*>(buf + C::GN);
    const float* gd = reinterpret_cast<const float*>(buf + C::GD);
    float pv[16];
    // with STORE, vb receives the values pass's operand bf16(s E / n_i), in
    // the layout of its B fragments and computed as there (so dV is bitwise
    // that of the recomputing values pass)
    bf16x8 vb[2];
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const double2 t01 = *reinterpret_cast<const double2*>(gt + 8 * rq + 4 * g);
      const double2 t23 = *reinterpret_cast<const double2*>(gt + 8 * rq + 4 * g + 2);
      const double tt[4] = {t01.x, t01.y, t23.x, t23.y};
      float nn[4] = {0.0f, 0.0f, 0.0f, 0.0f}, dd[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (MODE != kRowsPass) {
        const float4 n4 = *reinterpret_cast<const float4*>(gn + 8 * rq + 4 * g);
        nn[0] = n4.x; nn[1] = n4.y; nn[2] = n4.z; nn[3] = n4.w;
      }
      if (MODE == kKeysPass) {
        const float4 d4 = *reinterpret_cast<const float4*>(gd + 8 * rq + 4 * g);
        dd[0] = d4.x; dd[1] = d4.y; dd[2] = d4.z; dd[3] = d4.w;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ol = 8 * rq + 4 * g + e;  // other row within the tile
        // causal pairs j <= i only (Eq. 71), and real rows only
        bool valid;
        if (MODE == kRowsPass) valid = oi < T && !(diag && ol > l32);
        else valid = J * kBN + ol < T && !(diag && l32 > ol);
        // E = 2^(R_i + C_j), summed in float64 and rounded once
        const float E = valid ? __builtin_amdgcn_exp2f(float(own_t + tt[e])) : 0.0f;
        const float s = y1[4 * rq + e];
        if (MODE == kValuesPass) {
          pv[4 * rq + e] = s * E * nn[e];
        } else {
          const float in_i = MODE == kRowsPass ? own_in : nn[e];
          const float db_i = MODE == kRowsPass ? own_db : dd[e];
          const float P = E * (y2[4 * rq + e] * in_i + db_i);
          dsum += s * P;
          pv[4 * rq + e] = P;
          if (STORE) vb[rq >> 1][4 * (rq & 1) + e] = (__bf16)(s * E * nn[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb[0][e] = (__bf16)pv[e];
      pb[1][e] = (__bf16)pv[8 + e];
    }
    if constexpr (STORE) {
      char* dst = reinterpret_cast<char*>(vstore) + slot(J);
      *reinterpret_cast<bf16x8*>(dst + 16 * lane) = vb[0];
      *reinterpret_cast<bf16x8*>(dst + 1024 + 16 * lane) = vb[1];
      // bf16(P) into block (key tile 4 I + w, query tile J): row l32 (own
      // key), fragment c at positions 16 c + 8 g .. + 7
      char* pd = reinterpret_cast<char*>(pstore) +
                 (int64_t(head) * ptri + p_block(n_tiles, 4 * I + w, J)) * 2048 + 64 * l32 + 16 * g;
      *reinterpret_cast<bf16x8*>(pd) = pb[0];
      *reinterpret_cast<bf16x8*>(pd + 32) = pb[1];
    }
    }
    // accumulation: step t = (column block b, half c of the tile's rows); the
    // A operand holds X[16c + 4g + 0..3][32b + l32] and X[16c + 8 + 4g + 0..3][32b + l32]
    {
      const char* p = buf + offt;
      i16x4 lo[kBPf + 1], hi[kBPf + 1];
      auto addr = [&](int t) { return p + 16 * (t & 1) * C::SA + 64 * (cb0 + (t >> 1)); };
#pragma unroll
      for (int t = 0; t < kBPf; ++t) {
        lo[t] = tr_read(addr(t));
        hi[t] = tr_read(addr(t) + 8 * C::SA);
      }
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const int tn = t + kBPf;
        if (tn < NV) {
          lo[tn % (kBPf + 1)] = tr_read(addr(tn));
          hi[tn % (kBPf + 1)] = tr_read(addr(tn) + 8 * C::SA);
        }
        const i16x8 a16 = __builtin_shufflevector(lo[t % (kBPf + 1)], hi[t % (kBPf + 1)], 0, 1, 2,
                                                  3, 4, 5, 6, 7);
        acc[t >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16),
                                                              pb[t & 1], acc[t >> 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // the stored operand of the values pass: tile J + 1's is loaded while tile
  // J is computed, and has landed by the closing wait of tile J
  bf16x8 pin[2] = {bf16x8{}, bf16x8{}}, pnext[2] = {bf16x8{}, bf16x8{}};
  auto load_pin = [&](int J, bf16x8 (&dst)[2]) {
    if constexpr (MODE == kValuesStored) {
      if (J <= last && wave_needs(J)) {
        const char* src = reinterpret_cast<const char*>(vstore) + slot(J);
        dst[0] = *reinterpret_cast<const bf16x8*>(src + 16 * lane);
        dst[1] = *reinterpret_cast<const bf16x8*>(src + 1024 + 16 * lane);
      }
    }
  };
  auto next_pin = [&]() {
    if constexpr (MODE == kValuesStored) {
      pin[0] = pnext[0];
      pin[1] = pnext[1];
    }
  };

  if constexpr (MODE == kValuesStored) {
    // pairs of tiles: (J, J + 1) from one buffer while (J + 2, J + 3) land in
    // the other
    bf16x8 pin1[2] = {bf16x8{}, bf16x8{}}, pnext1[2] = {bf16x8{}, bf16x8{}};
    auto load_pair = [&](int J, char* buf) {
      load_tile(J, buf);
      if (J + 1 <= last) load_tile(J + 1, buf + C::GT);
    };
    auto compute_pair = [&](const char* buf, int J) {
      if (wave_needs(J)) compute(buf, J, pin, nullptr, false, TileSrc{}, true);
      if (J + 1 <= last && wave_needs(J + 1))
        compute(buf + C::GT, J + 1, pin1, nullptr, false, TileSrc{}, true);
    };
    auto next_pins = [&](int J) {
      pin[0] = pnext[0];
      pin[1] = pnext[1];
      pin1[0] = pnext1[0];
      pin1[1] = pnext1[1];
      load_pin(J, pnext);
      load_pin(J + 1, pnext1);
    };
    load_pair(first, smem0);
    load_pin(first, pin);
    load_pin(first + 1, pin1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int J = first; J <= last; J += 4) {
      load_pin(J + 2, pnext);
      load_pin(J + 3, pnext1);
      if (J + 2 <= last) load_pair(J + 2, smem1);
      compute_pair(smem0, J);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (J + 2 > last) break;
      next_pins(J + 4);
      if (J + 4 <= last) load_pair(J + 4, smem0);
      compute_pair(smem1, J + 2);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      pin[0] = pnext[0];
      pin[1] = pnext[1];
      pin1[0] = pnext1[0];
      pin1[1] = pnext1[1];
    }
  } else if constexpr (MODE == kRowsStored && C::RPAIR) {
    // pairs of tiles: (J, J + 1) from one buffer while (J + 2, J + 3) land in
    // the other
    auto load_pair = [&](int J, char* buf) {
      load_tile(J, buf);
      if (J + 1 <= last) load_tile(J + 1, buf + C::RT);
    };
    auto compute_pair = [&](const char* buf, int J) {
      if (wave_needs(J)) compute(buf, J, pin, nullptr, false, TileSrc{}, true);
      if (J + 1 <= last && wave_needs(J + 1))
        compute(buf + C::RT, J + 1, pin, nullptr, false, TileSrc{}, true);
    };
    load_pair(first, smem0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int J = first; J <= last; J += 4) {
      if (J + 2 <= last) load_pair(J + 2, smem1);
      compute_pair(smem0, J);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (J + 2 > last) break;
      if (J + 4 <= last) load_pair(J + 4, smem0);
      compute_pair(smem1, J + 2);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else if constexpr (MODE == kRowsStored) {
    // one tile per buffer (the widest heads): K rows and the stored P blocks
    // of tile J + 1 land while tile J is accumulated
    load_tile(first, smem0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int J = first; J <= last; J += 2) {
      if (J + 1 <= last) load_tile(J + 1, smem1);
      if (wave_needs(J)) compute(smem0, J, pin, nullptr, false, TileSrc{}, true);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (J + 1 > last) break;
      if (J + 2 <= last) load_tile(J + 2, smem0);
      if (wave_needs(J + 1)) compute(smem1, J + 1, pin, nullptr, false, TileSrc{}, true);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
  load_tile(first, smem0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto step = [&](const char* buf, int J, char* nxt) {
    const bool more = J + 1 <= last;
    const TileSrc ts = tile_src(J + 1);
    if (more) small_copies(J + 1, nxt);
    compute(buf, J, pin, nxt, more, ts, wave_needs(J));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int J = first; J <= last; J += 2) {
    step(smem0, J, smem1);  // even tile from smem0, the next into smem1
    if (J + 1 > last) break;
    step(smem1, J + 1, smem0);  // odd tile from smem1, the next into smem0
  }
  }

  // ---- epilogue: the row or column sums of dD~, and dQ / dK / dV in bf16
  if (MODE == kRowsPass || MODE == kKeysPass) {
    dsum += __shfl_xor(dsum, 32, 64);
    if (oi < T && g == 0 && blockIdx.y == 0) sums[int64_t(head) * T + oi] = dsum;
  }
  // the output row of the lane's accumulator column (the stored rows pass
  // holds the wave's queries in the stored blocks' order)
  const int orow = MODE == kRowsStored ? ow + q_of(l32) : oi;
  if (orow < T) {
    const int64_t row = hoff + int64_t(orow) * d;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = 32 * (cb0 + b) + 8 * rq + 4 * g;
        if (col < d) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[b][4 * rq + e];
          *reinterpret_cast<bf16x4*>(out + row + col) = o;
        }
      }
    }
  }
}

template <int DP, int MODE, bool STORE = false>
void launch_pass(const void* q, const void* k, const void* v, const void* dh, const void* h,
                 const float* m, const float* n, const float* b, float* inv_n, float* db,
                 const Workspace& ws, void* out, float* sums, void* store, int64_t H, int64_t T,
                 int64_t d, hipStream_t stream) {
  const int64_t row_tiles = (T + kBM - 1) / kBM;
  static_assert(!STORE || MODE == kKeysPass, "only the keys pass stores operands");
  // the store holds the values pass's operand, then the rows pass's
  u16* vstore = static_cast<u16*>(store);
  u16* pstore = store ? vstore + H * store_tiles(T) * kBWaves * 1024 : nullptr;
  hipLaunchKernelGGL((bwd_mfma_kernel<DP, MODE, STORE>),
                     dim3(unsigned(row_tiles * H), unsigned(BCfg<DP, MODE>::SPLIT)), dim3(kBThreads),
                     0, stream, static_cast<const u16*>(q), static_cast<const u16*>(k),
                     static_cast<const u16*>(v), static_cast<const u16*>(dh),
                     static_cast<const u16*>(h), m, n, b, inv_n, db, ws.rowt, ws.colt,
                     static_cast<u16*>(out), sums, int(T), int(d), int(ws.Tp), int(row_tiles),
                     int(H), vstore, store_tiles(T), pstore, p_blocks(T));
}

template <int DP>
void launch_all(const void* q, const void* k, const void* v, const void* dh, const void* h,
                const float* m, const float* n, const float* b, float* inv_n, float* db,
                const Workspace& ws, void* dq, void* dk, void* dv, float* rsum, float* csum,
                void* store, int64_t H, int64_t T, int64_t d, hipStream_t stream) {
  if (store != nullptr) {
    // the per-row scalars first; the keys pass forms S and G once and stores
    // the operands of the values and rows passes, which only accumulate
    const int64_t rows = H * T;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, stream,
                       static_cast<const u16*>(h), static_cast<const u16*>(dh), m, n, b, inv_n, db,
                       rsum, rows, int(d));
    launch_pass<DP, kKeysPass, true>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dk, csum, store, H,
                                     T, d, stream);
    launch_pass<DP, kValuesStored>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dv, nullptr, store, H,
                                   T, d, stream);
    launch_pass<DP, kRowsStored>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, nullptr, store, H,
                                 T, d, stream);
  } else {
    launch_pass<DP, kRowsPass>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, rsum, nullptr, H, T, d,
                               stream);
    launch_pass<DP, kKeysPass>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dk, csum, nullptr, H, T, d,
                               stream);
    launch_pass<DP, kValuesPass>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dv, nullptr, nullptr, H,
                                 T, d, stream);
  }
}

}  // namespace

bool backward_mfma_supports(int64_t d) { return d % 16 == 0 && d >= 16 && d <= 512; }

size_t backward_mfma_store_bytes(int64_t H, int64_t T) {
  return size_t(H) * (size_t(store_tiles(T)) * kBWaves + size_t(p_blocks(T))) * 2048;
}

hipError_t launch_backward_mfma_tiles(const void* q, const void* k, const void* v,
                                      const void* dh, const void* h, const float* m,
                                      const float* n, const float* b, float* inv_n, float* db,
                                      const Workspace& ws, void* dq, void* dk, void* dv,
                                      float* rsum, float* csum, void* vstore, int64_t H,
                                      int64_t T, int64_t d, hipStream_t stream) {
  if (!backward_mfma_supports(d)) return hipErrorInvalidValue;
  // head dims are padded up to a multiple of 64 (zero columns add nothing)
  switch ((d + 63) / 64) {
    case 1: launch_all<64>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, dk, dv, rsum, csum, vstore, H, T, d, stream); break;
    case 2: launch_all<128>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, dk, dv, rsum, csum, vstore, H, T, d, stream); break;
    case 3: launch_all<192>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, dk, dv, rsum, csum, vstore, H, T, d, stream); break;
    case 4: launch_all<256>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, dk, dv, rsum, csum, vstore, H, T, d, stream); break;
    case 5: launch_all<320>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, dk, dv, rsum, csum, vstore, H, T, d, stream); break;
    case 6: launch_all<384>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, dk, dv, rsum, csum, vstore, H, T, d, stream); break;
    case 7: launch_all<448>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, dk, dv, rsum, csum, vstore, H, T, d, stream); break;
    case 8: launch_all<512>(q, k, v, dh, h, m, n, b, inv_n, db, ws, dq, dk, dv, rsum, csum, vstore, H, T, d, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mlstm
