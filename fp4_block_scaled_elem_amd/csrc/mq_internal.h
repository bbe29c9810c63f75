// mq_internal.h - host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mq.h"

namespace mq {

struct DeviceInfo {
  int device = -1;
  int num_cu = 0;
  int ok = 0;  // gfx950
};

// With MQ_LOG=1 in the environment (read once per process) every launch
// prints its kernel, grid, block, dynamic LDS and shape to stderr; otherwise
// the call returns at once.
void log_launch(const char* kernel, unsigned grid, unsigned block, size_t lds, const char* fmt, ...)
    __attribute__((format(printf, 5, 6)));

hipError_t launch_amax(const void* x_bf16, int64_t nelem, mq_scale_rec* rec, const DeviceInfo& dev,
                       hipStream_t stream);
hipError_t launch_quantize(const void* x_bf16, int64_t nelem, uint8_t* codes, uint8_t* scales,
                           mq_scale_rec* rec, bool given, const DeviceInfo& dev, hipStream_t stream);
// A operand of a GEMM launch: packed (codes, scales) or, fused, bf16 values
// quantized in the kernel (rec then receives or, when given, supplies s_t).
struct GemmOperandA {
  const uint8_t* codes;
  const uint8_t* scales;
  const void* bf16;
  mq_scale_rec* rec;
  bool given;
  // fused (bf16 given): buffers that receive A's NVFP4, which switches the
  // launch to the quantize-once form; NULL: re-quantize per tile
  uint8_t* out_codes;
  uint8_t* out_scales;
};

// One weight of a (grouped) GEMM launch and its output C [M][n].
struct GemmWeight {
  const uint8_t* codes;
  const uint8_t* scales;
  const mq_scale_rec* rec;
  void* c;
  int64_t n;
};

hipError_t launch_gemm(const GemmOperandA& a, const GemmWeight* w, int ngroup, int64_t M, int64_t K, bool out_f32,
                       const DeviceInfo& dev, hipStream_t stream);
hipError_t launch_gemv(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                       const DeviceInfo& dev, hipStream_t stream);
// One weight of a grouped decode GEMV: W [n][K] bf16 and its output Y [M][n].
struct GemvWeight {
  const void* w;
  void* y;
  int64_t n;
};
hipError_t launch_gemv_grouped(const void* x, const GemvWeight* w, int ngroup, int64_t M, int64_t K,
                               const DeviceInfo& dev, hipStream_t stream);

// NVFP4 x NVFP4 decode GEMV operands: X [M][K] and W [N][K], output bf16
// Y [M][N].
struct GemvNvfp4Args {
  const uint8_t* x_codes;
  const uint8_t* x_scales;
  const mq_scale_rec* x_rec;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const mq_scale_rec* w_rec;
  void* y;
  int64_t M, N, K;
};

hipError_t launch_gemv_nvfp4(const GemvNvfp4Args& a, hipStream_t stream);

hipError_t launch_rmsnorm_amax(const void* x, const void* g, void* y, int64_t rows, int64_t cols, float eps,
                               mq_scale_rec* rec, const DeviceInfo& dev, hipStream_t stream);
hipError_t launch_swiglu_amax(const void* a, const void* b, void* y, int64_t n, mq_scale_rec* rec,
                              const DeviceInfo& dev, hipStream_t stream);

}  // namespace mq
