// Backward pass of the stabilized parallel mLSTM (xLSTM appendix A.3,
// "Parallel mLSTM Backward Pass", Eqs. 87-105) for float32 inputs, with the
// row and column passes on the gfx950 float32 matrix instruction
// v_mfma_f32_32x32x2_f32 (float32 products and sums, nothing rounded to a
// narrower type).  The per-entry formulas and exponent terms are those of
// the float32 vector passes (backward.hip):
//
//   E_ij = 2^fl32(R_i + C_j)  (0 above the diagonal and past the sequence end)
//   dC~'_ij = g_ij / n_i + db_i,  P_ij = E_ij dC~'_ij,  C~'_ij = s_ij E_ij
//
// in three passes of one kernel template:
//   rows   (own: 32 queries i; tiles of 32 keys j <= i)
//            S^T = K_J Q^T, G^T = V_J dH^T
//            r_i += sum_j C~'_ij dC~'_ij,  dQ^T += K_J^T P^T        (Eqs. 95, 98)
//   keys   (own: 32 keys j; tiles of 32 queries i >= j)
//            S = Q_I K^T, G = dH_I V^T
//            c_j += sum_i C~'_ij dC~'_ij,  dK^T += Q_I^T P          (Eqs. 97, 99, 105)
//   values (own: 32 keys j; tiles of 32 queries i >= j)
//            S = Q_I K^T,  dV^T += dH_I^T (C~' / n)                  (Eq. 100)
//
// Work decomposition.  A workgroup of 4 waves (one per SIMD) owns 32 rows of
// one head.  The first products reduce over the head dimension, which the
// waves split in quarters: wave u holds its own rows' operands for head dims
// [u d/4, (u+1) d/4) in registers (the B operand) and forms a partial 32 x 32
// result.  The four partials meet in LDS, and every wave sums all four in
// the fixed order 0, 1, 2, 3, so all of them hold the same S (and G) and
// form the tile's exponentials and P themselves (16 per lane, cheap next to
// the products).  The second product's 32-column output blocks are dealt to
// the waves round-robin (block b to wave b % 4); its reduction index is the
// tile's row, paired with the accumulator layout of the first product
// (step s: row 8 (s / 4) + 4 g + s % 4 for lane half g), so P feeds the B
// operand from registers and the tile is read one float per lane per step.
//
// Data movement.  The tiles come into LDS by global -> LDS copies (rows past
// the sequence end read as zeros), spread over the matrix instructions.  In
// the rows and keys passes the tile read by both products is double
// buffered and the next one is copied during the first products; the tile
// read only by the first products is copied during the second.  Where three
// tiles and the 32 KiB of partials do not fit in LDS (d = 352, 384), the
// partials go to the buffer of the tile that only the first products read,
// once every wave has read it (one more barrier per tile).  The values pass
// reads Q in the first product and dH in the second, one buffer each.
#include "mlstm_internal.h"
#include "tile_common.h"

namespace mlstm {
namespace {

using namespace tilecommon;

constexpr int kRowsPass = 0, kKeysPass = 1, kValuesPass = 2;
constexpr int kBThreads = 256;
constexpr int kBPf = 2;  // LDS operand prefetch distance of the first products (groups)
constexpr int kBPf2 = 4;  // and of the second product (steps)

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DP, int MODE>
struct BCfg {
  static_assert(DP % 32 == 0 && DP >= 32 && DP <= 384, "head dim of the float32 backward");
  static constexpr bool TWO = MODE != kValuesPass;  // S and G, or S only
  static constexpr int QD = DP / 4;                 // head dims of a wave's partial products
  static constexpr int NU = QD / 8;                 // 16-byte operand groups per row
  static constexpr int RB = 4 * DP;                 // bytes of a row in memory
  static constexpr int CH = DP / 4;                 // 16-byte chunks per row
  static constexpr int NCP = (CH + 63) / 64;        // copy instructions per row
  // LDS rows at 4 d + 16 bytes: the row reads (16 bytes of 32 rows) hit an
  // odd number of 16-byte slots apart, every 16 lanes distinct slots
  static constexpr int RS = RB + 16;
  static constexpr int TILE = kBN * RS;
  static constexpr int NBLK = DP / 32;         // 32-column output blocks
  static constexpr int NBW = (NBLK + 3) / 4;   // output blocks of a wave (at most)
  static constexpr int XCH = (TWO ? 2 : 1) * 4 * 4 * 1024;  // partials of the 4 waves
  static constexpr bool ALIAS = TWO && 3 * TILE + XCH > 160 * 1024;
  // rows / keys: X1 (read by both products) in buffers 0 and 1, X2 (first
  // products only), the partials (in the X2 buffer when ALIAS); values:
  // X1 = Q, X3 = dH, the partials
  static constexpr int X2_OFF = 2 * TILE;
  static constexpr int X3_OFF = TILE;
  static constexpr int XCH_OFF = TWO ? 3 * TILE : 2 * TILE;
  static constexpr int BYTES = TWO ? (ALIAS ? 3 * TILE : 3 * TILE + XCH) : 2 * TILE + XCH;
  static constexpr int kCopies = 8 * NCP;  // copy instructions per wave and tile tensor
  static_assert(!ALIAS || XCH <= TILE, "the partials fit in a tile buffer");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int DP, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(kBThreads, kBThreads),
                          amdgpu_waves_per_eu(1, 1))) void bwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dh, const float* __restrict__ inv_n, const float* __restrict__ db,
    const double* __restrict__ rowt, const double* __restrict__ colt, float* __restrict__ out,
    float* __restrict__ sums, int T, int Tp, int NT, int H) {
  using C = BCfg<DP, MODE>;
  constexpr bool ROWS = MODE == kRowsPass;
  __shared__ __attribute__((aligned(1024))) char lds[C::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  int64_t I64, head64;
  map_tile(blockIdx.x, NT, H, I64, head64);  // heaviest own block first
  const int head = int(head64);
  const int O = ROWS ? int(I64) : NT - 1 - int(I64);  // own 32-row block
  const int t_first = ROWS ? 0 : O;
  const int t_last = ROWS ? O : NT - 1;
  const int64_t hoff = int64_t(head) * T * DP;
  const int own = 32 * O + l32;  // this lane's own row (query or key)
  const bool own_in = own < T;
  const int D0 = w * C::QD;      // this wave's head dims in the first products

  // tensors: own rows (first products' B operands) and tiles
  const float* own1 = ROWS ? q : k;
  const float* own2 = ROWS ? dh : v;
  const float* x1 = ROWS ? k : q;                       // first product (and second, rows/keys)
  const float* x2 = ROWS ? v : dh;                      // G's tile (rows/keys); dH (values)

  // ---- own operands: 16 bytes of head dims D0 + 8 u + 4 g of the own row
  f32x4 o1[C::NU], o2[C::TWO ? C::NU : 1];
#pragma unroll
  for (int u = 0; u < C::NU; ++u) {
    const int64_t off = hoff + int64_t(own) * DP + D0 + 8 * u + 4 * g;
    o1[u] = own_in ? *reinterpret_cast<const f32x4*>(own1 + off) : f32x4{};
    if constexpr (C::TWO) o2[u] = own_in ? *reinterpret_cast<const f32x4*>(own2 + off) : f32x4{};
  }
  // per-lane terms of the own row
  double own_t;  // R_i (rows) or C_j (keys, values)
  float own_in_n = 0.0f, own_db = 0.0f;
  if constexpr (ROWS) {
    own_t = rowt[int64_t(head) * Tp + own];
    if (own_in) {
      own_in_n = inv_n[int64_t(head) * T + own];
      own_db = db[int64_t(head) * T + own];
    }
  } else {
    own_t = colt[int64_t(head) * Tp + own];  // -inf past the sequence end
  }

  // ---- copies: the wave's 8 rows of a 32-row tile, NCP pieces per row
  const unsigned vchunk = unsigned(16 * lane);
  auto rows_src = [&](const float* base, int tile) {
    const int r0 = 32 * tile + 8 * w;
    const int left = T - r0;
    const int n = left <= 0 ? 0 : (left < 8 ? left : 8);
    return rsrc_words(base + hoff + int64_t(r0) * DP, int64_t(n) * C::RB);
  };
  auto copy = [&](auto cc, const i32x4& rs, unsigned lds_base) {
    constexpr int c = decltype(cc)::value;
    constexpr int r = c / C::NCP, p = c % C::NCP;
    if (lane < C::CH - 64 * p)
      copy16_row<r, r * C::RS + 1024 * p>(rs, vchunk + 1024u * p, C::RB, lds_base);
  };
  auto tile_base = [&](int off) { return lds_addr(lds + off + 8 * w * C::RS); };
  auto x1_off = [&](int tile) { return C::TWO ? (tile & 1) * C::TILE : 0; };

  // the first tile(s)
  {
    const i32x4 rs1 = rows_src(x1, t_first);
    static_for<C::kCopies>([&](auto cc) { copy(cc, rs1, tile_base(x1_off(t_first))); });
    if constexpr (C::TWO) {
      const i32x4 rs2 = rows_src(x2, t_first);
      static_for<C::kCopies>([&](auto cc) { copy(cc, rs2, tile_base(C::X2_OFF)); });
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  f32x16 acc[C::NBW];
#pragma unroll
  for (int b = 0; b < C::NBW; ++b) acc[b] = f32x16{};
  float rsum = 0.0f;  // r_i (rows) or c_j (keys) of this lane's half of the tile rows

  // the wave's last output block may not exist (d / 32 not a multiple of 4)
  const bool last_block = w + 4 * (C::NBW - 1) < C::NBLK;
  constexpr int NS2 = 16 * C::NBW;  // steps of the second product

  for (int J = t_first; J <= t_last; ++J) {
    const bool more = J < t_last;
    const int cur = x1_off(J);
    char* const xch = lds + (C::ALIAS ? C::X2_OFF : C::XCH_OFF);

    // terms of the tile's rows 32 J + 8 rq + 4 g + e (register 4 rq + e)
    double tt[16];
    float tin[16], tdb[16];
    {
      const double* src = (ROWS ? colt : rowt) + int64_t(head) * Tp + 32 * J + 4 * g;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const double2 a = *reinterpret_cast<const double2*>(src + 8 * rq);
        const double2 b = *reinterpret_cast<const double2*>(src + 8 * rq + 2);
        tt[4 * rq] = a.x;
        tt[4 * rq + 1] = a.y;
        tt[4 * rq + 2] = b.x;
        tt[4 * rq + 3] = b.y;
      }
      if constexpr (!ROWS) {
        const int64_t base = int64_t(head) * T + 32 * J + 4 * g;
        if ((T & 3) == 0 && 32 * J + 32 <= T) {  // whole tile inside, rows 16-byte aligned
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(inv_n + base + 8 * rq);
            f32x4 b = f32x4{};
            if constexpr (MODE == kKeysPass) b = *reinterpret_cast<const f32x4*>(db + base + 8 * rq);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              tin[4 * rq + e] = a[e];
              tdb[4 * rq + e] = b[e];
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = 32 * J + 8 * (r >> 2) + 4 * g + (r & 3);
            tin[r] = i < T ? inv_n[int64_t(head) * T + i] : 0.0f;
            if constexpr (MODE == kKeysPass) tdb[r] = i < T ? db[int64_t(head) * T + i] : 0.0f;
          }
        }
      }
    }

    // ===== phase 1: partial first products over the wave's head dims =====
    {
      const char* const r1 = lds + cur + l32 * C::RS + 16 * g + 4 * D0;
      const char* const r2 = lds + C::X2_OFF + l32 * C::RS + 16 * g + 4 * D0;
      // copies during phase 1: the next X1 tile (rows / keys, unaliased) or
      // the current dH tile (values)
      constexpr bool kCopy1 = true;
      const int ctile = C::TWO ? J + 1 : J;
      const bool cdo = C::TWO ? more : true;
      const i32x4 rs_c = rows_src(C::TWO ? x1 : x2, ctile);
      const unsigned cdst = tile_base(C::TWO ? x1_off(J + 1) : C::X3_OFF);
      f32x16 st = f32x16{}, gt = f32x16{};
      f32x4 a1[kBPf + 1], a2[kBPf + 1];
#pragma unroll
      for (int u = 0; u < kBPf && u < C::NU; ++u) {
        a1[u] = *reinterpret_cast<const f32x4*>(r1 + 32 * u);
        if constexpr (C::TWO) a2[u] = *reinterpret_cast<const f32x4*>(r2 + 32 * u);
      }
      static_for<C::NU>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (u + kBPf < C::NU) {
          a1[(u + kBPf) % (kBPf + 1)] = *reinterpret_cast<const f32x4*>(r1 + 32 * (u + kBPf));
          if constexpr (C::TWO)
            a2[(u + kBPf) % (kBPf + 1)] = *reinterpret_cast<const f32x4*>(r2 + 32 * (u + kBPf));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          st = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[u % (kBPf + 1)][e], o1[u][e], st, 0, 0, 0);
          if constexpr (C::TWO)
            gt = __builtin_amdgcn_mfma_f32_32x32x2f32(a2[u % (kBPf + 1)][e], o2[u][e], gt, 0, 0,
                                                      0);
        }
        if constexpr (kCopy1) {
          if (cdo) {
            static_for<C::kCopies>([&](auto cc) {
              constexpr int c = decltype(cc)::value;
              if constexpr ((c * C::NU) / C::kCopies == u) copy(cc, rs_c, cdst);
            });
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      // partials to LDS: tensor t, wave w, register group rq: 16 bytes per lane
      // (aliased: into the X2 tile, once every wave has read it)
      if constexpr (C::ALIAS) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      char* const xw = xch + 4096 * w + 16 * lane;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        *reinterpret_cast<f32x4*>(xw + 1024 * rq) =
            f32x4{st[4 * rq], st[4 * rq + 1], st[4 * rq + 2], st[4 * rq + 3]};
        if constexpr (C::TWO)
          *reinterpret_cast<f32x4*>(xw + 16384 + 1024 * rq) =
              f32x4{gt[4 * rq], gt[4 * rq + 1], gt[4 * rq + 2], gt[4 * rq + 3]};
      }
      if constexpr (!C::TWO) __builtin_amdgcn_s_waitcnt(0);  // the dH tile has landed
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // ===== phase 2: the whole S (and G), P, the second product =====
    float s[16], gg[16];
    {
      const char* const xr = xch + 16 * lane;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 sa = *reinterpret_cast<const f32x4*>(xr + 1024 * rq);
        f32x4 ga = f32x4{};
        if constexpr (C::TWO) ga = *reinterpret_cast<const f32x4*>(xr + 16384 + 1024 * rq);
#pragma unroll
        for (int u = 1; u < 4; ++u) {
          sa += *reinterpret_cast<const f32x4*>(xr + 4096 * u + 1024 * rq);
          if constexpr (C::TWO) ga += *reinterpret_cast<const f32x4*>(xr + 16384 + 4096 * u + 1024 * rq);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[4 * rq + e] = sa[e];
          gg[4 * rq + e] = ga[e];
        }
      }
    }
    if constexpr (C::ALIAS) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // P (rows, keys) or C~' / n (values), register r: tile row 32 J + 8 (r / 4) + 4 g + r % 4
    float wgt[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int other = 32 * J + 8 * (r >> 2) + 4 * g + (r & 3);
      // causal mask (Eq. 71): key <= query, both inside the sequence
      const bool valid = ROWS ? (own_in && other <= own) : (other < T && own <= other);
      const double rc = ROWS ? own_t + tt[r] : tt[r] + own_t;
      const float e = valid ? exp2f(float(rc)) : 0.0f;
      if constexpr (MODE == kValuesPass) {
        wgt[r] = (s[r] * e) * tin[r];
      } else {
        const float in_i = ROWS ? own_in_n : tin[r];
        const float db_i = ROWS ? own_db : tdb[r];
        const float dct = gg[r] * in_i + db_i;  // dC~' (Eqs. 91-93)
        rsum += (s[r] * e) * dct;               // dD~ = C~' dC~' (Eqs. 94-95)
        wgt[r] = e * dct;
      }
    }

    {
      // second product: A = the tile read one float per lane, B = wgt
      const int toff = C::TWO ? cur : C::X3_OFF;
      const char* const cp = lds + toff + 4 * g * C::RS + 4 * l32 + 4 * 32 * w;
      auto caddr = [&](int t) {
        const int bt = t >> 4, st2 = t & 15;
        return cp + (8 * (st2 >> 2) + (st2 & 3)) * C::RS + 4 * 32 * 4 * bt;
      };
      // copies during phase 2: X2 of the next tile; the next Q (values)
      const i32x4 rs_a = rows_src(C::TWO ? x2 : x1, J + 1);
      const unsigned dst_a = tile_base(C::TWO ? C::X2_OFF : 0);
      float af[kBPf2 + 1];
#pragma unroll
      for (int t = 0; t < kBPf2; ++t) af[t] = *reinterpret_cast<const float*>(caddr(t));
      static_for<NS2>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr (t + kBPf2 < NS2)
          af[(t + kBPf2) % (kBPf2 + 1)] = *reinterpret_cast<const float*>(caddr(t + kBPf2));
        if (t < 16 * (C::NBW - 1) || last_block)
          acc[t >> 4] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[t % (kBPf2 + 1)], wgt[t & 15],
                                                            acc[t >> 4], 0, 0, 0);
        if (more) {
          static_for<C::kCopies>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            if constexpr ((c * NS2) / C::kCopies == t) copy(cc, rs_a, dst_a);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: the sums over the two lane halves, the accumulators
  rsum += __shfl_xor(rsum, 32, 64);
  if (own_in) {
    if (MODE != kValuesPass && w == 0 && g == 0) sums[int64_t(head) * T + own] = rsum;
    const int64_t row = hoff + int64_t(own) * DP;
#pragma unroll
    for (int bt = 0; bt < C::NBW; ++bt) {
      const int b = w + 4 * bt;
      if (b < C::NBLK) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          // register 4 rq + e of block b: head dim 32 b + 8 rq + 4 g + e
          const f32x4 o = f32x4{acc[bt][4 * rq], acc[bt][4 * rq + 1], acc[bt][4 * rq + 2],
                                acc[bt][4 * rq + 3]};
          *reinterpret_cast<f32x4*>(out + row + 32 * b + 8 * rq + 4 * g) = o;
        }
      }
    }
  }
}

template <int DP, int MODE>
void launch_pass(const float* q, const float* k, const float* v, const float* dh,
                 const float* inv_n, const float* db, const Workspace& ws, float* out,
                 float* sums, int64_t H, int64_t T, hipStream_t stream) {
  const int64_t nt = (T + kBN - 1) / kBN;
  hipLaunchKernelGGL((bwd_f32_kernel<DP, MODE>), dim3(unsigned(nt * H)), dim3(kBThreads), 0,
                     stream, q, k, v, dh, inv_n, db, ws.rowt, ws.colt, out, sums, int(T),
                     int(ws.Tp), int(nt), int(H));
}

template <int DP>
hipError_t launch_all(const float* q, const float* k, const float* v, const float* dh,
                      const float* inv_n, const float* db, const Workspace& ws, float* dq,
                      float* dk, float* dv, float* rsum, float* csum, int64_t H, int64_t T,
                      hipStream_t stream) {
  launch_pass<DP, kRowsPass>(q, k, v, dh, inv_n, db, ws, dq, rsum, H, T, stream);
  launch_pass<DP, kKeysPass>(q, k, v, dh, inv_n, db, ws, dk, csum, H, T, stream);
  launch_pass<DP, kValuesPass>(q, k, v, dh, inv_n, db, ws, dv, nullptr, H, T, stream);
  return hipGetLastError();
}

}  // namespace

bool backward_f32_supports(int64_t d) { return d % 32 == 0 && d >= 32 && d <= 384; }

hipError_t launch_backward_f32_tiles(const float* q, const float* k, const float* v,
                                     const float* dh, const float* inv_n, const float* db,
                                     const Workspace& ws, float* dq, float* dk, float* dv,
                                     float* rsum, float* csum, int64_t H, int64_t T, int64_t d,
                                     hipStream_t stream) {
  if (!backward_f32_supports(d)) return hipErrorInvalidValue;
#define MLSTM_DP(n) \
  launch_all<32 * n>(q, k, v, dh, inv_n, db, ws, dq, dk, dv, rsum, csum, H, T, stream)
  switch (d / 32) {
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
    default: return hipErrorInvalidValue;
  }
#undef MLSTM_DP
}

}  // namespace mlstm
