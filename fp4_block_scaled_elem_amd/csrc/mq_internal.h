// mq_internal.h - host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mq.h"

namespace mq {

// Inputs of at most this many elements take their absolute maximum inside
// the kernel that needs it (the quantizer, or the fused GEMM's per-tile
// form) instead of a separate amax pass: one launch fewer.
constexpr int64_t kInlineAmaxElems = (int64_t)1 << 17;

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
// inline_amax (dynamic scale, nelem <= kInlineAmaxElems): no amax pass
// before it; every workgroup takes max|x| itself.
hipError_t launch_quantize(const void* x_bf16, int64_t nelem, uint8_t* codes, uint8_t* scales,
                           mq_scale_rec* rec, bool given, const DeviceInfo& dev, hipStream_t stream,
                           bool inline_amax = false);
// The single-launch quantizer addresses its input through buffer
// resources: under 4 GiB of bf16.
constexpr int64_t kResidentMaxElems = (int64_t)1 << 31;
// Dynamic scale in one launch: the input read once into registers, the
// workgroups meeting at its maximum through rec (whose flags count the
// calls: the record must be zeroed when allocated).  For the input lengths
// where quantize_resident_pays; others take the amax pass and the encode.
bool quantize_resident_pays(int64_t nelem, const DeviceInfo& dev);
hipError_t launch_quantize_resident(const void* x_bf16, int64_t nelem, uint8_t* codes, uint8_t* scales,
                                    mq_scale_rec* rec, const DeviceInfo& dev, hipStream_t stream);
// Test support: the single-launch quantizer's poll limit (0: every
// workgroup takes the give-up path) and the count of workgroups that gave up
// since the last read.  Both return ~0u on a HIP error.
uint32_t set_rq_spin_limit(uint32_t polls);
uint32_t take_rq_gave_up();
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
  // fused per-tile form with a dynamic scale and A of at most
  // kInlineAmaxElems elements: no amax pass, every workgroup takes max|A|
  bool inline_amax;
};


// One weight of a (grouped) GEMM launch and its output C [M][n].
struct GemmWeight {
  const uint8_t* codes;
  const uint8_t* scales;
  const mq_scale_rec* rec;
  void* c;
  int64_t n;
};

// Test support: the column tiles each sharer of a 256-row panel must get for
// the fused quantize-once launch to take the panel form (default 4; 1 forces
// it wherever K allows); returns the previous value.
int set_panel_min_tiles(int tiles);
// Row counts (M) that the small-problem GEMM kernel takes, in every A form:
// 16 or 32 A rows and 16 W rows per workgroup, K split over its waves.
bool gemm_small_rows(int64_t M);
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
// RMSNorm fused with NVFP4 quantization: y's partial maxima into rec (y not
// stored), then y recomputed and encoded into codes and scales, s_t into rec.
hipError_t launch_rmsnorm_quantize(const void* x, const void* g, int64_t rows, int64_t cols, float eps,
                                   uint8_t* codes, uint8_t* scales, mq_scale_rec* rec, const DeviceInfo& dev,
                                   hipStream_t stream);
hipError_t launch_swiglu_amax(const void* a, const void* b, void* y, int64_t n, mq_scale_rec* rec,
                              const DeviceInfo& dev, hipStream_t stream);

}  // namespace mq
