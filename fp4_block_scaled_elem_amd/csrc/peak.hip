// peak.hip - the fp16 MFMA rate this chip sustains, alone and with the
// dequantization's VALU work beside it (measurement support for the
// benchmark; exported, not part of the public ABI in include/mq.h).
//
// The prefill GEMM issues v_mfma_f32_32x32x16_f16 on operands it has just
// dequantized in registers, one wave per SIMD, 4 x 4 accumulator fragments of
// 32 x 32 per wave (the whole accumulation register file), and about 4 VALU
// instructions per MFMA (per fragment and K16 step: four fp4 -> f16
// conversions and four packed multiplies).  This kernel runs that same
// register-resident inner loop with no memory traffic at all, so its rate
// is the ceiling of the GEMM's main loop on this chip:
//   V = 0: MFMAs only (operands fixed);
//   V = 4: each step's operands dequantized as the GEMM does (dequant8);
//   V = 6: the same plus two more packed multiplies per fragment.
// Every block's first wave also records the shader clock counter
// (s_memtime) and the constant-rate counter (s_memrealtime) at its start
// and end, from which the caller derives the clock the SIMDs ran at.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int kPeakThreads = 256;  // four waves: one per SIMD

// Makes the compiler assume v changed (no instruction): keeps the per-step
// dequantization inside the loop.
template <typename T>
__device__ __forceinline__ void opaque(T& v) {
  asm volatile("" : "+v"(v));
}

template <int V>
struct PeakPipe {
  uint32_t ca[4], cw[4];
  half2_t sa[4], sw[4];
  half8_t one;
  half8_t oa[2][4], ow[2][4];

  template <int B>
  __device__ __forceinline__ void produce() {
    if constexpr (V >= 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        opaque(ca[i]);
        opaque(cw[i]);
        oa[B][i] = dequant8(ca[i], sa[i][0]);
        ow[B][i] = dequant8(cw[i], sw[i][0]);
      }
    }
    if constexpr (V >= 6) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        oa[B][i] = oa[B][i] * one;
        ow[B][i] = ow[B][i] * one;
      }
    }
  }
  template <int B>
  __device__ __forceinline__ void mfma(f32x16_t (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ow[B][j], oa[B][i], acc[i][j], 0, 0, 0);
  }
};

template <int NVALU>
__device__ __forceinline__ void peak_interleave() {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if constexpr (NVALU > 0) __builtin_amdgcn_sched_group_barrier(0x002, NVALU / 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int V>
__global__ __launch_bounds__(kPeakThreads, 1) void mfma_peak_kernel(int iters, float* __restrict__ sink,
                                                                    uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  PeakPipe<V> p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p.ca[i] = 0x3A2B1C0Du * (lane + 1) + i;
    p.cw[i] = 0x1C2D3A0Bu * (lane + 3) + i;
    p.sa[i] = half2_t{(_Float16)0.5f, (_Float16)0.5f};
    p.sw[i] = half2_t{(_Float16)0.25f, (_Float16)0.25f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p.oa[0][i][k] = p.oa[1][i][k] = (_Float16)(0.001f * (lane + k));
      p.ow[0][i][k] = p.ow[1][i][k] = (_Float16)(0.002f * (k - lane));
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) p.one[k] = (_Float16)1.0f;
  opaque(p.one);
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  constexpr int kValu = V == 0 ? 0 : (V == 4 ? 64 : 96);  // VALU instructions per step of 16 MFMAs

  __syncthreads();
  uint64_t m0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    m0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  p.template produce<0>();
  for (int it = 0; it < iters; ++it) {
    p.template produce<1>();
    p.template mfma<0>(acc);
    peak_interleave<kValu>();
    p.template produce<0>();
    p.template mfma<1>(acc);
    peak_interleave<kValu>();
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  sink[blockIdx.x * kPeakThreads + threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t m1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    uint64_t* c = clocks + 4 * blockIdx.x;
    c[0] = m0;
    c[1] = r0;
    c[2] = m1;
    c[3] = r1;
  }
}

template <int V>
hipError_t launch_peak(int iters, int blocks, float* sink, uint64_t* clocks, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel<V>, dim3(blocks), dim3(kPeakThreads), 0, s, iters, sink, clocks);
  return hipGetLastError();
}

}  // namespace
}  // namespace mq

extern "C" {

// One launch of the rate kernel with V VALU instructions per MFMA (0, 4 or
// 6): `blocks` workgroups of four waves, each wave `iters` x 32 MFMAs
// (32x32x16 f16, 32768 flops each).  sink: DEVICE float [blocks * 256];
// clocks: DEVICE uint64 [blocks][4] = s_memtime and s_memrealtime at the
// first wave's start, then at its end.  Returns 0, 1 (bad arguments) or 5
// (launch error).
int32_t mq_check_mfma_rate(int32_t valu_per_mfma, int32_t iters, int32_t blocks, float* sink, uint64_t* clocks,
                           void* hip_stream) {
  if (iters < 1 || blocks < 1 || !sink || !clocks) return MQ_ERR_INVALID;
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e;
  switch (valu_per_mfma) {
    case 0: e = mq::launch_peak<0>(iters, blocks, sink, clocks, s); break;
    case 4: e = mq::launch_peak<4>(iters, blocks, sink, clocks, s); break;
    case 6: e = mq::launch_peak<6>(iters, blocks, sink, clocks, s); break;
    default: return MQ_ERR_INVALID;
  }
  return e == hipSuccess ? MQ_OK : MQ_ERR_LAUNCH;
}

// Rate of the s_memrealtime counter on the current device, in kHz.
int32_t mq_check_wall_clock_khz(int32_t* khz) {
  int d = 0;
  if (!khz || hipGetDevice(&d) != hipSuccess) return MQ_ERR_DEVICE;
  return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, d) == hipSuccess ? MQ_OK : MQ_ERR_DEVICE;
}

}  // extern "C"
