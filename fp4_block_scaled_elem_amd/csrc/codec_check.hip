// codec_check.hip - exhaustive views of the conversions the NVFP4 kernels
// are built on, for the test suite (exported, but not part of the public ABI
// declared in include/mq.h).
//
// The quantizer and the fused prologue take every element code and group
// scale byte from gfx950's conversion instructions (mq_device.h: encode8,
// e4m3_from_f32), and the GEMM and NVFP4 GEMV take every operand from the
// dequantization sigma_pair + dequant8.  These entry points run exactly those
// device functions over their whole input domains so that a test can hold
// them to the plain definitions of the formats (E2M1 and E4M3 rounding to
// nearest with ties to even and saturation, the value of an E2M1 code times
// the value of an E4M3 byte; gist.science English explainer of "Mix-Quant:
// Quantized Prefilling, Precise Decoding for Agentic LLMs", Technical
// Summary s.2, Hybrid Precision Strategy):
//
//   mq_check_codec_steps   a conversion as a step function of the binary32
//                          bit pattern: every pattern where its result
//                          differs from the previous pattern's (a handful
//                          of steps instead of 2^32 results)
//   mq_check_dequant_table every (scale byte, code) operand value as
//                          binary16 bits
//
// two knobs of the single-launch quantizer's bounded wait, so that a test
// can force its give-up path (mq_check_set_quant_spin_limit,
// mq_check_quant_gave_up), and the fused GEMM's panel-form threshold
// (mq_check_set_panel_min_tiles).
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {
namespace {

constexpr int kCheckThreads = 256;
constexpr int kPatternsPerThread = 1024;

// which = 0: the 4-bit element code encode8 gives for y = binary32 pattern
// p: y = x * e with x = +1 or -1 (bf16, the sign of p) and e = |y|, exact,
// so every non-NaN binary32 y is reachable.  which = 1: the E4M3 byte
// e4m3_from_f32 gives for rho = binary32 pattern p.
__device__ __forceinline__ uint32_t codec_value(int which, uint32_t p) {
  if (which == 0) {
    const uint32_t x = (p >> 31) ? 0xBF80BF80u : 0x3F803F80u;  // two bf16 -1.0 or +1.0
    const uint32_t w[4] = {x, x, x, x};
    return encode8<false>(w, __uint_as_float(p & 0x7FFFFFFFu)) & 0xFu;
  }
  return e4m3_from_f32(__uint_as_float(p));
}

// Patterns lo + i, i in [0, count): thread t walks its own 1024 of them in
// order and appends (p, value) wherever the value differs from that of
// p - 1 (and at i = 0).  out[0] counts the steps (appended through a global
// atomic, so their order is arbitrary); entries past cap are counted but not
// stored.
__global__ __launch_bounds__(kCheckThreads) void codec_steps_kernel(int which, uint32_t lo, uint64_t count,
                                                                    uint32_t* __restrict__ out, uint32_t cap) {
  const uint64_t i0 = ((uint64_t)blockIdx.x * kCheckThreads + threadIdx.x) * kPatternsPerThread;
  if (i0 >= count) return;
  const uint64_t i1 = i0 + kPatternsPerThread < count ? i0 + kPatternsPerThread : count;
  uint32_t prev = i0 == 0 ? 0xFFFFFFFFu : codec_value(which, lo + (uint32_t)(i0 - 1));
  for (uint64_t i = i0; i < i1; ++i) {
    const uint32_t p = lo + (uint32_t)i;
    const uint32_t v = codec_value(which, p);
    if (v != prev) {
      const uint32_t slot = atomicAdd(out, 1u);
      if (slot < cap) {
        out[1 + 2 * slot] = p;
        out[2 + 2 * slot] = v;
      }
      prev = v;
    }
  }
}

__global__ void init_counter_kernel(uint32_t* out) { out[0] = 0u; }

// Thread S (0..127): the scale byte S in all four bytes of a scale dword,
// its binary16 value through sigma_pair with both byte selectors, and the 16
// codes (two dwords: codes 0..7 and 8..15) through dequant8 with each of the
// four: out[S][sel][code], 128 x 4 x 16 binary16 bit patterns.
__global__ void dequant_table_kernel(uint16_t* __restrict__ out) {
  const uint32_t S = threadIdx.x;
  const uint32_t dword = S * 0x01010101u;
  const half2_t s01 = sigma_pair<false>(dword), s23 = sigma_pair<true>(dword);
  const _Float16 sig[4] = {s01[0], s01[1], s23[0], s23[1]};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const half8_t lo = dequant8(0x76543210u, sig[k]);
    const half8_t hi = dequant8(0xFEDCBA98u, sig[k]);
    uint16_t* o = out + (S * 4 + k) * 16;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      o[c] = __builtin_bit_cast(uint16_t, (_Float16)lo[c]);
      o[8 + c] = __builtin_bit_cast(uint16_t, (_Float16)hi[c]);
    }
  }
}

}  // namespace
}  // namespace mq

extern "C" {

// Steps of conversion `which` (0: element code, 1: E4M3 group scale byte)
// over the binary32 patterns lo..hi (inclusive, lo <= hi).  out: DEVICE
// uint32 [1 + 2 * cap]; out[0] receives the number of steps, out[1 + 2i] /
// out[2 + 2i] the pattern and value of step i (unordered).  Queued on
// hip_stream; returns 0, or 1 for bad arguments, 5 for a launch error.
int32_t mq_check_codec_steps(int32_t which, uint32_t lo, uint32_t hi, uint32_t* out, uint32_t cap,
                             void* hip_stream) {
  if ((which != 0 && which != 1) || lo > hi || out == nullptr) return MQ_ERR_INVALID;
  hipStream_t s = (hipStream_t)hip_stream;
  const uint64_t count = (uint64_t)hi - lo + 1;
  const uint64_t per_block = (uint64_t)mq::kCheckThreads * mq::kPatternsPerThread;
  const unsigned blocks = (unsigned)((count + per_block - 1) / per_block);
  hipLaunchKernelGGL(mq::init_counter_kernel, dim3(1), dim3(1), 0, s, out);
  hipLaunchKernelGGL(mq::codec_steps_kernel, dim3(blocks), dim3(mq::kCheckThreads), 0, s, (int)which, lo, count,
                     out, cap);
  return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_LAUNCH;
}

// The GEMM operand of every (scale byte S, code) pair: out DEVICE uint16
// [128][4][16] (binary16 bits; the 4 = byte position of S in the scale dword).
int32_t mq_check_dequant_table(uint16_t* out, void* hip_stream) {
  if (out == nullptr) return MQ_ERR_INVALID;
  hipLaunchKernelGGL(mq::dequant_table_kernel, dim3(1), dim3(128), 0, (hipStream_t)hip_stream, out);
  return hipGetLastError() == hipSuccess ? MQ_OK : MQ_ERR_LAUNCH;
}

// The single-launch quantizer's poll limit before a workgroup stops waiting
// for the others and takes the maximum itself (0: no wait, every workgroup
// gives up): returns the previous limit, ~0u on error.  Device-wide, for the
// current device; only for tests that run nothing else meanwhile.
uint32_t mq_check_set_quant_spin_limit(uint32_t polls) { return mq::set_rq_spin_limit(polls); }

// Workgroups of the single-launch quantizer that gave up waiting since the
// last call (the count is reset), ~0u on error.
uint32_t mq_check_quant_gave_up(void) { return mq::take_rq_gave_up(); }

// The column tiles per panel sharer from which the fused quantize-once GEMM
// takes its panel form (1: wherever K allows, so that tests reach it at
// small shapes); returns the previous value.  Process-wide.
int32_t mq_check_set_panel_min_tiles(int32_t tiles) { return mq::set_panel_min_tiles(tiles); }

}  // extern "C"
