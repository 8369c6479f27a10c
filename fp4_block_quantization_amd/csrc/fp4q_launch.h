// fp4q_launch.h -- internal launchers behind the C ABI (include/fp4q.h).
// Arguments reaching these have already been validated on the host.
#pragma once

// The memory-pattern stand-in build (-DFP4Q_STANDIN=1) and the
// exact-error decision build (-DFP4Q_NV_CERTIFY=0) put everything in a
// namespace of their own, so that their kernels carry names of their own in
// profiles and cannot be mistaken for the quantizer's.
#if defined(FP4Q_STANDIN) && FP4Q_STANDIN && !defined(fp4q)
#define fp4q fp4q_standin
#elif defined(FP4Q_NV_CERTIFY) && !FP4Q_NV_CERTIFY && !defined(fp4q)
#define fp4q fp4q_exactdecision
#endif

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q.h"

// Work-items per kernel launch at most; larger calls are split into several
// launches over consecutive rows (or blocks).  The dispatch packet counts
// work-items in 32 bits.
#ifndef FP4Q_MAX_LAUNCH_ITEMS
#define FP4Q_MAX_LAUNCH_ITEMS ((int64_t)1 << 31)
#endif

namespace fp4q {

struct NvQuantArgs {
  const void* x;
  int64_t rows;
  int64_t hidden;
  const int64_t* offsets;
  int64_t num_groups;
  int four_over_six;
  uint8_t* codes;
  uint8_t* block_scales;
  float* token_scales;
  void* dequant;
  // one scale for the whole tensor: the tensor-max pass's per-workgroup
  // maxima (16-bit BF16 magnitude patterns, zero-padded; num_partials
  // 16-byte units of them), from which every wave derives s, and where the
  // first wave stores it
  const uint4* global_partials = nullptr;
  int num_partials = 0;
  float* tensor_scale_out = nullptr;
};

hipError_t nvfp4_quantize_launch(const NvQuantArgs& a, hipStream_t stream);
hipError_t nvfp4_quantize_global_launch(const NvQuantArgs& a, float* tensor_scale,
                                        void* workspace, hipStream_t stream);
// Bytes of workspace that call uses for a tensor of rows x hidden.
int64_t global_workspace_bytes(int64_t rows, int64_t hidden);
hipError_t nvfp4_dequantize_launch(const uint8_t* codes, const uint8_t* scales,
                                   const float* token_scales, int64_t rows, int64_t hidden,
                                   void* out, hipStream_t stream);
hipError_t mxfp4_resq_launch(const void* x, int64_t rows, int64_t hidden, uint8_t* codes,
                             uint8_t* scales, uint8_t* res_codes, uint8_t* res_meta,
                             uint8_t* res_scales, hipStream_t stream);

hipError_t mxfp4_resq_dense_launch(const void* x, int64_t rows, int64_t hidden, uint8_t* codes,
                                   uint8_t* scales, uint8_t* res_codes, uint8_t* res_scales,
                                   hipStream_t stream);
hipError_t mxfp4_reconstruct_launch(const uint8_t* codes, const uint8_t* scales,
                                    const uint8_t* res_codes, const uint8_t* res_meta,
                                    const uint8_t* res_scales, int64_t rows, int64_t hidden,
                                    int residual, float* out, hipStream_t stream);

hipError_t nvfp4_guided_launch(const void* x, const uint8_t* guide, const uint8_t* scales,
                              const float* tscale, int64_t rows, int64_t hidden, uint8_t* codes,
                              void* dequant, hipStream_t stream);

}  // namespace fp4q
