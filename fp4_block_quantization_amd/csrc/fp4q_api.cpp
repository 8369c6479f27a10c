// fp4q_api.cpp -- the C ABI declared in include/fp4q.h: host-side argument
// validation, then the kernel launches of the call on the caller's stream.
// Validation touches no HIP API, so a rejected call returns its status
// even on a machine without a GPU.
#include "fp4q.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "fp4q_launch.h"

namespace {

// Largest sizes accepted: element indices fit comfortably in 64 bits and
// row lengths in an int; calls above 2^31 work-items are split into several
// launches by the launchers.
constexpr int64_t kMaxRows = (int64_t)1 << 32;
constexpr int64_t kMaxHidden = (int64_t)1 << 30;
constexpr int64_t kMaxElements = (int64_t)1 << 40;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

fp4q_status check_shape(int64_t rows, int64_t hidden, int64_t block) {
  if (rows < 0 || hidden <= 0 || hidden % block != 0) return FP4Q_ERROR_INVALID_SHAPE;
  if (rows > kMaxRows || hidden > kMaxHidden || rows * hidden > kMaxElements)
    return FP4Q_ERROR_INVALID_SHAPE;
  return FP4Q_SUCCESS;
}

fp4q_status launched(hipError_t e) { return e == hipSuccess ? FP4Q_SUCCESS : FP4Q_ERROR_LAUNCH; }

// Scratch of nvfp4_quantize_global_noalloc: the partial maxima its tensor-max
// pass hands to its quantize pass, in place of the caller's workspace.  One
// copy per device, held until the process ends; every call on a device
// shares it, so calls that overlap on one device race.  Nothing in it needs
// to start at zero: the max pass writes every slot the quantize pass reads.
static __device__ __align__(256) uint8_t scratch[FP4Q_GLOBAL_WORKSPACE_BYTES];

// Its device address per device, looked up once per device with that
// device current (in host code the array's name is not a device address).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The array on the device the call's kernels run on: the stream's device
// (the current device for the NULL stream), which need not be the calling
// thread's current device.  The first lookup on a device makes that device
// current for the hipGetSymbolAddress call and then restores the caller's.
hipError_t scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = -1;
      e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
      if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      if (back != hipSuccess) return back;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

fp4q_status nvfp4_quantize(const void* x, int64_t rows, int64_t hidden,
                           const int64_t* group_offsets, int64_t num_groups, int four_over_six,
                           uint8_t* codes, uint8_t* block_scales, float* token_scales,
                           void* dequant, void* stream) {
  fp4q_status st = check_shape(rows, hidden, 16);
  if (st != FP4Q_SUCCESS) return st;
  if (four_over_six < 0 || four_over_six > 2) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (num_groups < 0 || (num_groups == 0 && group_offsets != nullptr))
    return FP4Q_ERROR_INVALID_SHAPE;
  if (num_groups > 0 && group_offsets == nullptr) return FP4Q_ERROR_NULL_POINTER;
  if (rows == 0) return FP4Q_SUCCESS;
  if (!x || !codes || !block_scales || !token_scales) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(token_scales, 4) ||
      (dequant && !aligned(dequant, 16)) || (group_offsets && !aligned(group_offsets, 8)))
    return FP4Q_ERROR_MISALIGNED;
  fp4q::NvQuantArgs a{x,     rows,         hidden,       group_offsets, num_groups,
                      four_over_six, codes, block_scales, token_scales, dequant};
  return launched(fp4q::nvfp4_quantize_launch(a, (hipStream_t)stream));
}

fp4q_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* block_scales,
                             const float* token_scales, int64_t rows, int64_t hidden, void* out,
                             void* stream) {
  fp4q_status st = check_shape(rows, hidden, 16);
  if (st != FP4Q_SUCCESS) return st;
  if (rows == 0) return FP4Q_SUCCESS;
  if (!codes || !block_scales || !token_scales || !out) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(codes, 8) || !aligned(token_scales, 4) || !aligned(out, 16))
    return FP4Q_ERROR_MISALIGNED;
  return launched(fp4q::nvfp4_dequantize_launch(codes, block_scales, token_scales, rows, hidden,
                                                out, (hipStream_t)stream));
}

fp4q_status mxfp4_resq_quantize(const void* x, int64_t rows, int64_t hidden, uint8_t* codes,
                                uint8_t* scales, uint8_t* res_codes, uint8_t* res_meta,
                                uint8_t* res_scales, void* stream) {
  fp4q_status st = check_shape(rows, hidden, 32);
  if (st != FP4Q_SUCCESS) return st;
  if (rows == 0) return FP4Q_SUCCESS;
  if (!x || !codes || !scales || !res_codes || !res_meta || !res_scales)
    return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(res_codes, 8) || !aligned(res_meta, 4))
    return FP4Q_ERROR_MISALIGNED;
  return launched(fp4q::mxfp4_resq_launch(x, rows, hidden, codes, scales, res_codes, res_meta,
                                          res_scales, (hipStream_t)stream));
}

fp4q_status mxfp4_resq_dense_quantize(const void* x, int64_t rows, int64_t hidden,
                                      uint8_t* codes, uint8_t* scales, uint8_t* res_codes,
                                      uint8_t* res_scales, void* stream) {
  fp4q_status st = check_shape(rows, hidden, 32);
  if (st != FP4Q_SUCCESS) return st;
  if (rows == 0) return FP4Q_SUCCESS;
  if (!x || !codes || !scales || !res_codes || !res_scales) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(res_codes, 16))
    return FP4Q_ERROR_MISALIGNED;
  return launched(fp4q::mxfp4_resq_dense_launch(x, rows, hidden, codes, scales, res_codes,
                                                res_scales, (hipStream_t)stream));
}

fp4q_status mxfp4_resq_reconstruct(const uint8_t* codes, const uint8_t* scales,
                                   const uint8_t* res_codes, const uint8_t* res_meta,
                                   const uint8_t* res_scales, int64_t rows, int64_t hidden,
                                   int residual, float* out, void* stream) {
  fp4q_status st = check_shape(rows, hidden, 32);
  if (st != FP4Q_SUCCESS) return st;
  if (residual < 0 || residual > 2) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (rows == 0) return FP4Q_SUCCESS;
  if (!codes || !scales || !out) return FP4Q_ERROR_NULL_POINTER;
  if (residual != 0 && (!res_codes || !res_scales)) return FP4Q_ERROR_NULL_POINTER;
  if (residual == 1 && !res_meta) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(codes, 16) || !aligned(out, 16) ||
      (residual == 1 && !aligned(res_codes, 8)) || (residual == 2 && !aligned(res_codes, 16)))
    return FP4Q_ERROR_MISALIGNED;
  return launched(fp4q::mxfp4_reconstruct_launch(codes, scales, res_codes, res_meta, res_scales,
                                                 rows, hidden, residual, out,
                                                 (hipStream_t)stream));
}

fp4q_status nvfp4_quantize_guided(const void* x, int64_t rows, int64_t hidden,
                                  const uint8_t* guide_codes, const uint8_t* block_scales,
                                  const float* token_scales, uint8_t* codes, void* dequant,
                                  void* stream) {
  fp4q_status st = check_shape(rows, hidden, 16);
  if (st != FP4Q_SUCCESS) return st;
  if (rows == 0) return FP4Q_SUCCESS;
  if (!x || !block_scales || !token_scales || !codes) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(guide_codes, 4) || !aligned(codes, 4) ||
      !aligned(token_scales, 4) || (dequant && !aligned(dequant, 16)))
    return FP4Q_ERROR_MISALIGNED;
  return launched(fp4q::nvfp4_guided_launch(x, guide_codes, block_scales, token_scales, rows,
                                            hidden, codes, dequant, (hipStream_t)stream));
}

fp4q_status nvfp4_quantize_global(const void* x, int64_t rows, int64_t hidden,
                                  int four_over_six, uint8_t* codes, uint8_t* block_scales,
                                  float* tensor_scale, void* dequant, void* workspace,
                                  void* stream) {
  fp4q_status st = check_shape(rows, hidden, 16);
  if (st != FP4Q_SUCCESS) return st;
  if (four_over_six < 0 || four_over_six > 2) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (rows == 0) return FP4Q_SUCCESS;
  if (!x || !codes || !block_scales || !tensor_scale || !workspace)
    return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4) ||
      !aligned(workspace, 16) || (dequant && !aligned(dequant, 16)))
    return FP4Q_ERROR_MISALIGNED;
  fp4q::NvQuantArgs a{x,     rows,         hidden,  nullptr, 0,
                      four_over_six, codes, block_scales, nullptr, dequant};
  return launched(
      fp4q::nvfp4_quantize_global_launch(a, tensor_scale, workspace, (hipStream_t)stream));
}

fp4q_status nvfp4_quantize_global_noalloc(const void* x, int64_t rows, int64_t hidden,
                                          int four_over_six, uint8_t* codes,
                                          uint8_t* block_scales, float* tensor_scale,
                                          void* dequant, void* stream) {
  fp4q_status st = check_shape(rows, hidden, 16);
  if (st != FP4Q_SUCCESS) return st;
  if (four_over_six < 0 || four_over_six > 2) return FP4Q_ERROR_INVALID_ARGUMENT;
  if (rows == 0) return FP4Q_SUCCESS;
  if (!x || !codes || !block_scales || !tensor_scale) return FP4Q_ERROR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4) ||
      (dequant && !aligned(dequant, 16)))
    return FP4Q_ERROR_MISALIGNED;
  // the scratch need is fixed (at most 512 two-byte partial maxima, padded
  // to 16-byte units), whatever the tensor's size
  if (fp4q::global_workspace_bytes(rows, hidden) > (int64_t)sizeof(scratch))
    return FP4Q_ERROR_INVALID_SHAPE;
  void* ws = nullptr;
  if (scratch_for_stream((hipStream_t)stream, &ws) != hipSuccess) return FP4Q_ERROR_LAUNCH;
  fp4q::NvQuantArgs a{x,     rows,         hidden,  nullptr, 0,
                      four_over_six, codes, block_scales, nullptr, dequant};
  return launched(fp4q::nvfp4_quantize_global_launch(a, tensor_scale, ws, (hipStream_t)stream));
}

const char* fp4q_status_string(fp4q_status status) {
  switch (status) {
    case FP4Q_SUCCESS: return "success";
    case FP4Q_ERROR_NULL_POINTER: return "a required pointer is NULL";
    case FP4Q_ERROR_INVALID_SHAPE: return "invalid shape or group count";
    case FP4Q_ERROR_MISALIGNED: return "a pointer lacks its required alignment";
    case FP4Q_ERROR_LAUNCH: return "HIP kernel launch failed";
    case FP4Q_ERROR_INVALID_ARGUMENT: return "an option is outside its documented values";
  }
  return "unknown status";
}

}  // extern "C"
