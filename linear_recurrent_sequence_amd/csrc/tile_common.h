// Pieces of the bf16 matrix-core tile kernels kept apart from their bodies:
// operand types, tile sizes, the workgroup-to-tile mapping, and the
// global -> LDS copy and LDS transpose-read helpers shared by the bf16
// tile kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace mlstm {
namespace tilecommon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 32;   // keys per tile
constexpr int kRsrcFlags = 0x00020000;         // buffer resource word 3: 32-bit data format
constexpr unsigned kOutOfRange = 0x40000000u;  // a buffer offset that reads zeros

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

// Gate inputs of a tile kernel that scans its head's gates in its prologue:
// the pre-activations, the forget activation, ln(d)/2, and the m output of
// the workgroup's rows.
struct FusedGates {
  const float* igate;
  const float* fgate;
  float* m_out;
  double half_ln_d;
  int exp_forget;
};
// s_waitcnt operand: vmcnt(N) for N < 64 (bits 3:0 and 15:14), no wait on
// expcnt (bits 6:4) or lgkmcnt (bits 11:8)
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// a buffer resource: offsets at or past `num_records` bytes read as zeros
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t num_records) {
  const int n = num_records > 0x7FFFFFFF ? 0x7FFFFFFF : int(num_records);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcFlags);
}
// 16 bytes per lane, global -> LDS at (wave-uniform) dst + 16 * lane
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rsrc, unsigned voffset, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, voffset, 0, 0, 0);
}
// 4 bytes per lane, to dst + 4 * lane
__device__ inline void dma4(__amdgpu_buffer_rsrc_t rsrc, unsigned voffset, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 4, voffset, 0, 0, 0);
}

// The same copies issued through inline assembly, so that the compiler does
// not wait for them before unrelated LDS reads; the kernel waits for them
// (vmcnt) itself before each barrier.  They write M0 themselves, which the
// compiler may not expect to change: a kernel that also uses the builtin
// copies above (for which the compiler sets M0) issues all of those before
// the first of these.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// buffer resource words: offsets at or past num_records bytes read as zeros
__device__ inline i32x4 rsrc_words(const void* base, int64_t num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int n = num_records > 0x7FFFFFFF ? 0x7FFFFFFF : int(num_records);
  return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xFFFFu), n, kRsrcFlags};
}
__device__ inline unsigned lds_addr(const char* p) {
  return unsigned(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}
// 16 bytes per active lane, global -> LDS at (wave-uniform) dst + 16 * lane.
// M0 holds the LDS destination; one wait state separates its write from the copy.
// Wave-uniform operands of the copies, forced into scalar registers: the "s"
// constraint alone does not stop the compiler from placing a uniform value
// that it computed in vector registers there.
__device__ inline unsigned sreg(unsigned x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline i32x4 sreg(i32x4 x) {
  return i32x4{__builtin_amdgcn_readfirstlane(x[0]), __builtin_amdgcn_readfirstlane(x[1]),
               __builtin_amdgcn_readfirstlane(x[2]), __builtin_amdgcn_readfirstlane(x[3])};
}
__device__ inline void copy16(i32x4 rsrc, unsigned voffset, unsigned dst) {
  rsrc = sreg(rsrc);
  dst = sreg(dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(dst), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
// 4 bytes per active lane to dst + 4 * lane
__device__ inline void copy4(i32x4 rsrc, unsigned voffset, unsigned dst) {
  rsrc = sreg(rsrc);
  dst = sreg(dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(dst), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// Row I of a run of rows, 16 bytes per active lane: global offset
// vchunk + I * row_bytes in the range rsrc, LDS destination
// lds_base + LDS_OFF + 16 * lane.  The row's offsets are formed inside the
// instruction sequence, so that only the bases stay in registers: with the
// offsets of every row of a tile formed up front, the compiler keeps them all
// live and spills once the copies are spread over a loop of products.
template <int I, int LDS_OFF>
__device__ inline void copy16_row(i32x4 rsrc, unsigned vchunk, int row_bytes, unsigned lds_base) {
  rsrc = sreg(rsrc);
  lds_base = sreg(lds_base);
  row_bytes = int(sreg(unsigned(row_bytes)));
  unsigned vtmp;
  int stmp;
  asm volatile(
      "s_mul_i32 %1, %3, %5\n\t"
      "v_add_u32 %0, %1, %2\n\t"
      "s_add_u32 m0, %4, %6\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %7, 0 offen lds"
      : "=&v"(vtmp), "=&s"(stmp)
      : "v"(vchunk), "s"(row_bytes), "s"(lds_base), "n"(I), "n"(LDS_OFF), "s"(rsrc)
      : "memory", "m0", "scc");
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order
template <typename F, int... Is>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ inline i16x4 tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

}  // namespace tilecommon
}  // namespace mlstm
