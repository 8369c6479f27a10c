// fp4q_launch.h -- internal launchers behind the C ABI (include/fp4q.h).
// Arguments reaching these have already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  const float* global_scale = nullptr;  // set: the token scale s of every row (one for the tensor)
};

hipError_t nvfp4_quantize_launch(const NvQuantArgs& a, hipStream_t stream);
hipError_t nvfp4_quantize_global_launch(const NvQuantArgs& a, float* tensor_scale,
                                        hipStream_t stream);
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
