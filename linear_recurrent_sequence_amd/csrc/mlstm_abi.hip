// C ABI of libmlstm (declared in include/mlstm.h): argument validation,
// workspace handling, and the kernel launches of the stabilized parallel
// mLSTM forward pass (xLSTM appendix A.3, Eqs. 79-86: one launch of a tile
// kernel that scans its own gates, or the gate scan and then a tile kernel),
// of its backward pass and of the recurrent step.
#include "mlstm.h"
#include "mlstm_internal.h"

#include <stdint.h>

#include <initializer_list>
#include <mutex>

namespace mlstm {

// Workspace of mlstm_parallel_fwd_noalloc: one fixed array per GPU, which
// holds it until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address on each GPU comes from
// hipGetSymbolAddress, and only that address is ever handed to a kernel.
__device__ __attribute__((aligned(256))) char scratch[MLSTM_NOALLOC_SCRATCH_BYTES];

}  // namespace mlstm

namespace {

using mlstm::Workspace;

constexpr int64_t kMaxT = int64_t(1) << 30;
constexpr int64_t kMaxElems = int64_t(1) << 46;
constexpr int64_t kMaxHeadDim = 1024;

int check_shape(int64_t B, int64_t NH, int64_t T, int64_t d) {
  if (B < 1 || NH < 1 || T < 1 || d < 1) return MLSTM_ERR_SHAPE;
  if (T > kMaxT || B > (int64_t(1) << 31) || NH > (int64_t(1) << 31)) return MLSTM_ERR_SHAPE;
  const int64_t H = B * NH;
  if (H > (int64_t(1) << 31) - 1) return MLSTM_ERR_SHAPE;
  const int64_t Tp = mlstm::padded_len(T);
  if (H > kMaxElems / Tp) return MLSTM_ERR_SHAPE;
  // launch grids are one-dimensional: (T / 16) x H workgroups at most
  if (((Tp / 16) * H) > int64_t(0xFFFFFFFF)) return MLSTM_ERR_SHAPE;
  if (d % 16 != 0 || d > kMaxHeadDim) return MLSTM_ERR_HEAD_DIM;
  if (H * Tp > kMaxElems / d) return MLSTM_ERR_SHAPE;
  return MLSTM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MLSTM_OK : MLSTM_ERR_HIP; }

// a caller buffer's byte range; a null pointer or an empty range is skipped
struct Span {
  const void* p;
  size_t n;
};

// MLSTM_ERR_ALIAS if an output overlaps an input or another output (inputs
// may overlap each other: they are only read).  Runs after every other
// argument check, on shapes that check_shape has bounded.
int check_alias(std::initializer_list<Span> ins, std::initializer_list<Span> outs) {
  for (const Span* o = outs.begin(); o != outs.end(); ++o) {
    if (!o->p || o->n == 0) continue;
    for (const Span& i : ins)
      if (i.p && i.n && overlaps(o->p, o->n, i.p, i.n)) return MLSTM_ERR_ALIAS;
    for (const Span* o2 = outs.begin(); o2 != o; ++o2)
      if (o2->p && o2->n && overlaps(o->p, o->n, o2->p, o2->n)) return MLSTM_ERR_ALIAS;
  }
  return MLSTM_OK;
}

// bytes of a [B][NH][T][d] tensor of `dtype` and of a [B][NH][T] float32 array
size_t tensor_bytes(int64_t B, int64_t NH, int64_t T, int64_t d, int dtype) {
  return size_t(B * NH) * size_t(T) * size_t(d) * (dtype == MLSTM_BF16 ? 2 : 4);
}
size_t rows_bytes(int64_t B, int64_t NH, int64_t T) { return size_t(B * NH) * size_t(T) * 4; }

// the forward's inputs against its outputs (optional ones may be NULL)
int check_forward_alias(const void* q, const void* k, const void* v, const float* igate,
                        const float* fgate, const void* ogate, const void* h_out,
                        const void* htilde_out, const float* m_out, const float* n_out,
                        const float* b_out, int64_t B, int64_t NH, int64_t T, int64_t d,
                        int dtype) {
  const size_t tb = tensor_bytes(B, NH, T, d, dtype), rb = rows_bytes(B, NH, T);
  return check_alias({{q, tb}, {k, tb}, {v, tb}, {igate, rb}, {fgate, rb}, {ogate, tb}},
                     {{h_out, tb}, {htilde_out, tb}, {m_out, rb}, {n_out, rb}, {b_out, rb}});
}

int check_scan_args(const float* igate, const float* fgate, const float* m_out, const void* ws) {
  if (!igate || !fgate || !m_out || !ws) return MLSTM_ERR_NULL;
  if (!aligned16(igate) || !aligned16(fgate) || !aligned16(m_out)) return MLSTM_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return MLSTM_ERR_ALIGN;
  return MLSTM_OK;
}

int check_tile_args(const void* q, const void* k, const void* v, const float* m, const void* ws,
                    const void* h_out, const float* n_out, int dtype, int kernel) {
  if (!q || !k || !v || !m || !ws || !h_out || !n_out) return MLSTM_ERR_NULL;
  if (dtype != MLSTM_FP32 && dtype != MLSTM_BF16) return MLSTM_ERR_DTYPE;
  if (kernel != MLSTM_KERNEL_AUTO && kernel != MLSTM_KERNEL_MFMA &&
      kernel != MLSTM_KERNEL_VECTOR && kernel != MLSTM_KERNEL_MFMA_ALL_TILES &&
      kernel != MLSTM_KERNEL_MFMA_SINGLE && kernel != MLSTM_KERNEL_MFMA_WIDE)
    return MLSTM_ERR_KERNEL;
  if ((kernel == MLSTM_KERNEL_MFMA || kernel == MLSTM_KERNEL_MFMA_ALL_TILES ||
       kernel == MLSTM_KERNEL_MFMA_SINGLE || kernel == MLSTM_KERNEL_MFMA_WIDE) &&
      dtype != MLSTM_BF16)
    return MLSTM_ERR_KERNEL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(m) || !aligned16(h_out) ||
      !aligned16(n_out))
    return MLSTM_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return MLSTM_ERR_ALIGN;
  return MLSTM_OK;
}

int run_tiles(const void* q, const void* k, const void* v, const float* m, const Workspace& w,
              void* h_out, float* n_out, const mlstm::Epilogue& ep, int64_t H, int64_t T,
              int64_t d, int dtype, int kernel, hipStream_t stream) {
  const bool use_mfma = kernel == MLSTM_KERNEL_MFMA || kernel == MLSTM_KERNEL_MFMA_ALL_TILES ||
                        kernel == MLSTM_KERNEL_MFMA_SINGLE || kernel == MLSTM_KERNEL_MFMA_WIDE ||
                        (kernel == MLSTM_KERNEL_AUTO && dtype == MLSTM_BF16);
  const bool skip = kernel != MLSTM_KERNEL_MFMA_ALL_TILES;
  if (!use_mfma) {
    // float32 inputs: the float32 matrix-core kernel where it applies, unless
    // the vector kernel is asked for
    if (kernel == MLSTM_KERNEL_AUTO && dtype == MLSTM_FP32 && mlstm::tiles_f32_supports(d))
      return hip_status(mlstm::launch_tiles_f32(q, k, v, m, w, h_out, n_out, ep, true, H, T, d,
                                                stream));
    return hip_status(mlstm::launch_tiles_vector(q, k, v, m, w, h_out, n_out, ep, H, T, d,
                                                 dtype == MLSTM_BF16, stream));
  }
  if (kernel == MLSTM_KERNEL_MFMA_SINGLE) {
    if (d > 512) return MLSTM_ERR_HEAD_DIM;
    return hip_status(mlstm::launch_tiles_mfma(q, k, v, m, w, h_out, n_out, ep, skip, H, T, d,
                                               stream));
  }
  if (kernel == MLSTM_KERNEL_MFMA_WIDE || d > 512)
    return hip_status(mlstm::launch_tiles_wide(q, k, v, m, w, h_out, n_out, ep, skip, H, T, d,
                                               stream));
  if (mlstm::tiles_pairs_supports(d))
    return hip_status(mlstm::launch_tiles_pairs(q, k, v, m, w, h_out, n_out, ep, skip, H, T, d,
                                                stream));
  return hip_status(mlstm::launch_tiles_mfma(q, k, v, m, w, h_out, n_out, ep, skip, H, T, d,
                                             stream));
}

// float32 inputs whose head dim the float32 matrix-core kernel does not take,
// on sequences the vector kernel's own gate scan covers
bool vector_fused_path(int64_t T, int64_t d, int dtype) {
  return dtype == MLSTM_FP32 && !mlstm::tiles_f32_supports(d) &&
         mlstm::tiles_vector_fused_supports(T, d);
}

// float32 inputs on the float32 matrix-core kernel, same sequence bound
bool f32_fused_path(int64_t T, int64_t d, int dtype) {
  return dtype == MLSTM_FP32 && mlstm::tiles_f32_fused_supports(T, d);
}

// Whether the whole pass runs as one launch of the tile kernel that scans its
// gates itself (no workspace).
bool fused_path(int64_t T, int64_t d, int dtype) {
  return (dtype == MLSTM_BF16 &&
          (mlstm::tiles_pipe_preferred(T, d) || mlstm::tiles_pairs_fused_supports(T, d) ||
           mlstm::tiles_mfma_fused_supports(T, d))) ||
         vector_fused_path(T, d, dtype) || f32_fused_path(T, d, dtype);
}

// Both stages on a given workspace (mlstm::workspace_bytes(B * NH, T) bytes,
// 256-byte aligned; unused on the fused path).  Arguments are checked by the
// caller.
int forward_on(void* ws, const void* q, const void* k, const void* v, const float* igate,
               const float* fgate, const mlstm::Epilogue& ep, void* h_out, float* m_out,
               float* n_out, int64_t B, int64_t NH, int64_t T, int64_t d, int dtype,
               hipStream_t s, bool exp_forget) {
  const int64_t H = B * NH;
  if (f32_fused_path(T, d, dtype))
    return hip_status(mlstm::launch_tiles_f32_fused(q, k, v, igate, fgate, h_out, m_out, n_out,
                                                    ep, exp_forget, H, T, d, s));
  if (vector_fused_path(T, d, dtype))
    return hip_status(mlstm::launch_tiles_vector_fused(q, k, v, igate, fgate, h_out, m_out, n_out,
                                                       ep, exp_forget, H, T, d, false, s));
  if (fused_path(T, d, dtype) && mlstm::tiles_pipe_preferred(T, d))
    return hip_status(mlstm::launch_tiles_pipe(q, k, v, igate, fgate, h_out, m_out, n_out, ep,
                                               exp_forget, H, T, d, s));
  if (fused_path(T, d, dtype))
    return hip_status(
        mlstm::tiles_pairs_fused_supports(T, d)
            ? mlstm::launch_tiles_pairs_fused(q, k, v, igate, fgate, h_out, m_out, n_out, ep,
                                              exp_forget, H, T, d, s)
            : mlstm::launch_tiles_mfma_fused(q, k, v, igate, fgate, h_out, m_out, n_out, ep,
                                             exp_forget, H, T, d, s));
  const Workspace w = mlstm::carve(ws, H, T);
  int st = hip_status(mlstm::launch_gate_scan(igate, fgate, m_out, w, H, T, d, exp_forget, s));
  if (st == MLSTM_OK)
    st = run_tiles(q, k, v, m_out, w, h_out, n_out, ep, H, T, d, dtype, MLSTM_KERNEL_AUTO, s);
  return st;
}

// Both stages with a stream-ordered workspace (safe under concurrent calls on
// different streams).  Arguments are checked by the caller.
int forward(const void* q, const void* k, const void* v, const float* igate, const float* fgate,
            const mlstm::Epilogue& ep, void* h_out, float* m_out, float* n_out, int64_t B,
            int64_t NH, int64_t T, int64_t d, int dtype, hipStream_t s,
            bool exp_forget = false) {
  if (fused_path(T, d, dtype))
    return forward_on(nullptr, q, k, v, igate, fgate, ep, h_out, m_out, n_out, B, NH, T, d,
                      dtype, s, exp_forget);
  const size_t bytes = mlstm::workspace_bytes(B * NH, T);
  void* ws = nullptr;
  if (hipMallocAsync(&ws, bytes, s) != hipSuccess) {
    (void)hipGetLastError();
    return MLSTM_ERR_HIP;
  }
  int st = forward_on(ws, q, k, v, igate, fgate, ep, h_out, m_out, n_out, B, NH, T, d, dtype, s,
                      exp_forget);
  if (hipFreeAsync(ws, s) != hipSuccess && st == MLSTM_OK) st = MLSTM_ERR_HIP;
  return st;
}

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return MLSTM_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return MLSTM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(mlstm::scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return MLSTM_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLSTM_OK;
}

int check_forward_args(const void* q, const void* k, const void* v, const float* igate,
                       const float* fgate, const void* h_out, const float* m_out,
                       const float* n_out, int64_t B, int64_t NH, int64_t T, int64_t d,
                       int dtype) {
  if (dtype != MLSTM_FP32 && dtype != MLSTM_BF16) return MLSTM_ERR_DTYPE;
  int st = check_shape(B, NH, T, d);
  if (st != MLSTM_OK) return st;
  if (!q || !k || !v || !igate || !fgate || !h_out || !m_out || !n_out) return MLSTM_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(igate) ||
      !aligned16(fgate) || !aligned16(h_out) || !aligned16(m_out) || !aligned16(n_out))
    return MLSTM_ERR_ALIGN;
  return MLSTM_OK;
}

}  // namespace

extern "C" {

size_t mlstm_workspace_bytes(int64_t B, int64_t NH, int64_t T) {
  if (check_shape(B, NH, T, 16) != MLSTM_OK) return 0;
  return mlstm::workspace_bytes(B * NH, T);
}

int mlstm_gate_scan(const float* igate, const float* fgate, float* m_out, void* workspace,
                    size_t workspace_bytes, int64_t B, int64_t NH, int64_t T, int64_t d,
                    int forget_activation, void* stream) {
  if (forget_activation != MLSTM_FORGET_SIGMOID && forget_activation != MLSTM_FORGET_EXP)
    return MLSTM_ERR_ACTIVATION;
  int st = check_scan_args(igate, fgate, m_out, workspace);
  if (st != MLSTM_OK) return st;
  if ((st = check_shape(B, NH, T, d)) != MLSTM_OK) return st;
  const int64_t H = B * NH;
  if (workspace_bytes < mlstm::workspace_bytes(H, T)) return MLSTM_ERR_WORKSPACE;
  const size_t rb = rows_bytes(B, NH, T);
  if ((st = check_alias({{igate, rb}, {fgate, rb}},
                        {{m_out, rb}, {workspace, mlstm::workspace_bytes(H, T)}})) != MLSTM_OK)
    return st;
  const Workspace w = mlstm::carve(workspace, H, T);
  return hip_status(mlstm::launch_gate_scan(igate, fgate, m_out, w, H, T, d,
                                            forget_activation == MLSTM_FORGET_EXP,
                                            static_cast<hipStream_t>(stream)));
}

int mlstm_causal_tiles(const void* q, const void* k, const void* v, const float* m,
                       const void* workspace, size_t workspace_bytes, void* h_out, float* n_out,
                       int64_t B, int64_t NH, int64_t T, int64_t d, int dtype, int kernel,
                       void* stream) {
  int st = check_tile_args(q, k, v, m, workspace, h_out, n_out, dtype, kernel);
  if (st != MLSTM_OK) return st;
  if ((st = check_shape(B, NH, T, d)) != MLSTM_OK) return st;
  const int64_t H = B * NH;
  if (workspace_bytes < mlstm::workspace_bytes(H, T)) return MLSTM_ERR_WORKSPACE;
  const size_t tb = tensor_bytes(B, NH, T, d, dtype), rb = rows_bytes(B, NH, T);
  if ((st = check_alias({{q, tb}, {k, tb}, {v, tb}, {m, rb},
                         {workspace, mlstm::workspace_bytes(H, T)}},
                        {{h_out, tb}, {n_out, rb}})) != MLSTM_OK)
    return st;
  const Workspace w = mlstm::carve(const_cast<void*>(workspace), H, T);
  return run_tiles(q, k, v, m, w, h_out, n_out, mlstm::Epilogue{}, H, T, d, dtype, kernel,
                   static_cast<hipStream_t>(stream));
}

int mlstm_parallel_fwd_stream(const void* q, const void* k, const void* v, const float* igate,
                              const float* fgate, void* h_out, float* m_out, float* n_out,
                              int64_t B, int64_t NH, int64_t T, int64_t d, int dtype,
                              void* stream) {
  int st = check_forward_args(q, k, v, igate, fgate, h_out, m_out, n_out, B, NH, T, d, dtype);
  if (st != MLSTM_OK) return st;
  st = check_forward_alias(q, k, v, igate, fgate, nullptr, h_out, nullptr, m_out, n_out, nullptr,
                           B, NH, T, d, dtype);
  if (st != MLSTM_OK) return st;
  return forward(q, k, v, igate, fgate, mlstm::Epilogue{}, h_out, m_out, n_out, B, NH, T, d,
                 dtype, static_cast<hipStream_t>(stream));
}

int mlstm_parallel_fwd_gated(const void* q, const void* k, const void* v, const float* igate,
                             const float* fgate, const void* ogate, void* h_out,
                             void* htilde_out, float* m_out, float* n_out, int64_t B,
                             int64_t NH, int64_t T, int64_t d, int dtype, void* stream) {
  int st = check_forward_args(q, k, v, igate, fgate, h_out, m_out, n_out, B, NH, T, d, dtype);
  if (st != MLSTM_OK) return st;
  if (!ogate) return MLSTM_ERR_NULL;
  if (!aligned16(ogate) || (htilde_out && !aligned16(htilde_out))) return MLSTM_ERR_ALIGN;
  st = check_forward_alias(q, k, v, igate, fgate, ogate, h_out, htilde_out, m_out, n_out, nullptr,
                           B, NH, T, d, dtype);
  if (st != MLSTM_OK) return st;
  mlstm::Epilogue ep;
  ep.ogate = ogate;
  ep.htilde = htilde_out;
  return forward(q, k, v, igate, fgate, ep, h_out, m_out, n_out, B, NH, T, d, dtype,
                 static_cast<hipStream_t>(stream));
}

int mlstm_parallel_fwd_noalloc(const void* q, const void* k, const void* v, const float* igate,
                               const float* fgate, void* h_out, float* m_out, float* n_out,
                               int64_t B, int64_t NH, int64_t T, int64_t d, int dtype,
                               void* stream) {
  int st = check_forward_args(q, k, v, igate, fgate, h_out, m_out, n_out, B, NH, T, d, dtype);
  if (st != MLSTM_OK) return st;
  // the single-launch path needs no workspace, whatever the size
  if (!fused_path(T, d, dtype) &&
      mlstm::workspace_bytes(B * NH, T) > size_t(MLSTM_NOALLOC_SCRATCH_BYTES))
    return MLSTM_ERR_SCRATCH;
  st = check_forward_alias(q, k, v, igate, fgate, nullptr, h_out, nullptr, m_out, n_out, nullptr,
                           B, NH, T, d, dtype);
  if (st != MLSTM_OK) return st;
  void* ws = nullptr;
  if (!fused_path(T, d, dtype) && (st = scratch_on_current_device(&ws)) != MLSTM_OK) return st;
  // every byte of the workspace that a kernel reads is written earlier in the
  // same call (the scan writes all its terms up to the padded length), so
  // nothing left by an earlier call needs clearing
  return forward_on(ws, q, k, v, igate, fgate, mlstm::Epilogue{}, h_out, m_out, n_out, B, NH, T,
                    d, dtype, static_cast<hipStream_t>(stream), false);
}

int mlstm_parallel_fwd(const void* q, const void* k, const void* v, const float* igate,
                       const float* fgate, void* h_out, float* m_out, float* n_out, int64_t B,
                       int64_t NH, int64_t T, int64_t d, int dtype) {
  return mlstm_parallel_fwd_stream(q, k, v, igate, fgate, h_out, m_out, n_out, B, NH, T, d,
                                   dtype, nullptr);
}

int mlstm_parallel_fwd_train(const void* q, const void* k, const void* v, const float* igate,
                             const float* fgate, void* h_out, float* m_out, float* n_out,
                             float* b_out, int64_t B, int64_t NH, int64_t T, int64_t d,
                             int dtype, int forget_activation, void* stream) {
  int st = check_forward_args(q, k, v, igate, fgate, h_out, m_out, n_out, B, NH, T, d, dtype);
  if (st != MLSTM_OK) return st;
  if (forget_activation != MLSTM_FORGET_SIGMOID && forget_activation != MLSTM_FORGET_EXP)
    return MLSTM_ERR_ACTIVATION;
  if (!b_out) return MLSTM_ERR_NULL;
  if (!aligned16(b_out)) return MLSTM_ERR_ALIGN;
  st = check_forward_alias(q, k, v, igate, fgate, nullptr, h_out, nullptr, m_out, n_out, b_out, B,
                           NH, T, d, dtype);
  if (st != MLSTM_OK) return st;
  mlstm::Epilogue ep;
  ep.b = b_out;
  return forward(q, k, v, igate, fgate, ep, h_out, m_out, n_out, B, NH, T, d, dtype,
                 static_cast<hipStream_t>(stream), forget_activation == MLSTM_FORGET_EXP);
}

int mlstm_parallel_bwd(const void* q, const void* k, const void* v, const float* igate,
                       const float* fgate, const void* h, const float* m, const float* n,
                       const float* b, const void* dh, void* dq, void* dk, void* dv,
                       float* digate, float* dfgate, int64_t B, int64_t NH, int64_t T,
                       int64_t d, int dtype, int forget_activation, void* stream) {
  if (dtype != MLSTM_FP32 && dtype != MLSTM_BF16) return MLSTM_ERR_DTYPE;
  if (forget_activation != MLSTM_FORGET_SIGMOID && forget_activation != MLSTM_FORGET_EXP)
    return MLSTM_ERR_ACTIVATION;
  const bool exp_forget = forget_activation == MLSTM_FORGET_EXP;
  int st = check_shape(B, NH, T, d);
  if (st != MLSTM_OK) return st;
  if (d > mlstm::kBackwardMaxHeadDim) return MLSTM_ERR_HEAD_DIM;
  const void* ins[] = {q, k, v, igate, fgate, h, m, n, b, dh};
  const void* outs[] = {dq, dk, dv, digate, dfgate};
  for (const void* p : ins)
    if (!p) return MLSTM_ERR_NULL;
  for (const void* p : outs)
    if (!p) return MLSTM_ERR_NULL;
  for (const void* p : ins)
    if (!aligned16(p)) return MLSTM_ERR_ALIGN;
  for (const void* p : outs)
    if (!aligned16(p)) return MLSTM_ERR_ALIGN;
  {
    const size_t tb = tensor_bytes(B, NH, T, d, dtype), rb = rows_bytes(B, NH, T);
    st = check_alias({{q, tb}, {k, tb}, {v, tb}, {h, tb}, {dh, tb}, {igate, rb}, {fgate, rb},
                      {m, rb}, {n, rb}, {b, rb}},
                     {{dq, tb}, {dk, tb}, {dv, tb}, {digate, rb}, {dfgate, rb}});
    if (st != MLSTM_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t H = B * NH;
  const size_t wsb = mlstm::workspace_bytes(H, T);
  const size_t mb = mlstm::align256(size_t(H) * size_t(T) * sizeof(float));
  // read once: the scratch size and the launch must see the same store size
  const size_t store = mlstm::backward_store_bytes(H, T, d, dtype == MLSTM_BF16);
  const size_t scb = mlstm::backward_scratch_bytes(H, T, store);
  void* ws = nullptr;
  if (hipMallocAsync(&ws, wsb + mb + scb, s) != hipSuccess) {
    (void)hipGetLastError();
    return MLSTM_ERR_HIP;
  }
  const Workspace w = mlstm::carve(ws, H, T);
  float* m_scan = reinterpret_cast<float*>(static_cast<char*>(ws) + wsb);
  void* scratch = static_cast<char*>(ws) + wsb + mb;
  // the exponent terms of D' are recomputed from the gates (the scan's m is
  // bitwise the forward's)
  st = hip_status(mlstm::launch_gate_scan(igate, fgate, m_scan, w, H, T, d, exp_forget, s));
  if (st == MLSTM_OK)
    st = hip_status(mlstm::launch_backward(q, k, v, fgate, h, m, n, b, dh, w, scratch, store, dq,
                                           dk, dv, digate, dfgate, H, T, d, dtype == MLSTM_BF16,
                                           exp_forget, s));
  if (hipFreeAsync(ws, s) != hipSuccess && st == MLSTM_OK) st = MLSTM_ERR_HIP;
  return st;
}

int mlstm_recurrent_step(const void* q, const void* k, const void* v, const float* igate,
                         const float* fgate, const float* C_in, const float* n_in,
                         const float* m_in, float* C_out, float* n_out, float* m_out,
                         void* h_out, float* den_out, int64_t B, int64_t NH, int64_t d,
                         int dtype, int forget_activation, void* stream) {
  if (dtype != MLSTM_FP32 && dtype != MLSTM_BF16) return MLSTM_ERR_DTYPE;
  if (forget_activation != MLSTM_FORGET_SIGMOID && forget_activation != MLSTM_FORGET_EXP)
    return MLSTM_ERR_ACTIVATION;
  int st = check_shape(B, NH, 1, d);
  if (st != MLSTM_OK) return st;
  if (!q || !k || !v || !igate || !fgate || !C_in || !n_in || !m_in || !C_out || !n_out ||
      !m_out || !h_out)
    return MLSTM_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(C_in) || !aligned16(n_in) ||
      !aligned16(C_out) || !aligned16(n_out) || !aligned16(h_out) ||
      (reinterpret_cast<uintptr_t>(igate) & 3) || (reinterpret_cast<uintptr_t>(fgate) & 3) ||
      (reinterpret_cast<uintptr_t>(m_in) & 3) || (reinterpret_cast<uintptr_t>(m_out) & 3) ||
      (reinterpret_cast<uintptr_t>(den_out) & 3))
    return MLSTM_ERR_ALIGN;
  const int64_t H = B * NH;
  // C may be updated in place, but not through a shifted window; n and m are
  // read by every workgroup while the first of each head writes them
  const size_t cb = size_t(H) * size_t(d) * size_t(d) * sizeof(float);
  const size_t nb = size_t(H) * size_t(d) * sizeof(float);
  const size_t mb = size_t(H) * sizeof(float);
  if ((C_out != C_in && overlaps(C_in, cb, C_out, cb)) || overlaps(n_in, nb, n_out, nb) ||
      overlaps(m_in, mb, m_out, mb))
    return MLSTM_ERR_ALIAS;
  return hip_status(mlstm::launch_recurrent_step(q, k, v, igate, fgate, C_in, n_in, m_in, C_out,
                                                 n_out, m_out, h_out, den_out, H, d,
                                                 dtype == MLSTM_BF16,
                                                 forget_activation == MLSTM_FORGET_EXP,
                                                 static_cast<hipStream_t>(stream)));
}

const char* mlstm_strerror(int status) {
  switch (status) {
    case MLSTM_OK: return "success";
    case MLSTM_ERR_NULL: return "a required pointer is NULL";
    case MLSTM_ERR_SHAPE: return "invalid shape: B, NH, T, d must be >= 1 and sizes must not overflow";
    case MLSTM_ERR_DTYPE: return "invalid dtype: expected MLSTM_FP32 or MLSTM_BF16";
    case MLSTM_ERR_HEAD_DIM: return "unsupported head dimension: d must be a multiple of 16 in [16, 1024] (and <= 512 for the one-wave MFMA kernel)";
    case MLSTM_ERR_ALIGN: return "misaligned pointer: tensors need 16-byte, workspaces 256-byte alignment";
    case MLSTM_ERR_HIP: return "HIP allocation or kernel launch failed";
    case MLSTM_ERR_WORKSPACE: return "workspace smaller than mlstm_workspace_bytes()";
    case MLSTM_ERR_KERNEL: return "unknown kernel selector, or the MFMA kernel asked for float32";
    case MLSTM_ERR_ALIAS: return "an output overlaps an input it must not alias";
    case MLSTM_ERR_ACTIVATION: return "unknown forget-gate activation";
    case MLSTM_ERR_SCRATCH: return "the problem needs more workspace than the allocation-free entry point's fixed buffer holds (MLSTM_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
