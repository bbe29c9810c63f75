// gemv.hip - BF16 decode GEMV / skinny GEMM, Y = X . W^T (gfx950).
//
// The decode linear of "Mix-Quant: Quantized Prefilling, Precise Decoding for
// Agentic LLMs" (gist.science English explainer, Technical Summary s.2:
// Hybrid Precision Strategy, Decoding; System-Level Deployment, decode
// workers) runs on the original BF16 weights.  With M <= 32 rows of X the
// work is bound by streaming W from HBM (2 bytes per weight, M flops/byte),
// so the kernel is organised around W's bytes:
//   - a workgroup owns 16 rows of W and all of K; its NW waves split K in
//     interleaved 128-element chunks, so the whole chip streams W with many
//     16-byte loads in flight;
//   - each lane reads 64 contiguous bytes of one W row per chunk and feeds
//     them to v_mfma_f32_16x16x32_bf16 (W rows as the 16-row operand, X^T
//     as the 16-column operand; up to two column tiles for M <= 32).  The
//     MFMA is used for its fp32 accumulation of exact bf16 products, not for
//     its rate: the kernel stays HBM-bound;
//   - the K order inside a chunk is permuted identically for W and X;
//   - the per-wave partial tiles are summed through LDS in a fixed order
//     (deterministic), scaled to bf16 with round-to-nearest-even and stored.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

constexpr int kGvChunk = 128;  // K elements per wave per chunk
constexpr int kGvMaxWaves = 16;

template <int MT>
__global__ __launch_bounds__(kGvMaxWaves * 64) void gemv_bf16_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ w,
                                                                   uint16_t* __restrict__ y, int M, int N,
                                                                   int K) {
  __shared__ f32x4_t red[kGvMaxWaves][MT][64];
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16;
  int nrow = n0 + i;
  nrow = nrow < N ? nrow : N - 1;
  const uint16_t* wrow = w + (int64_t)nrow * K + 32 * h;
  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = i + 16 * t;
    xok[t] = m < M;
    xrow[t] = x + (int64_t)(xok[t] ? m : 0) * K + 32 * h;
  }
  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (K + kGvChunk - 1) / kGvChunk;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  int c = wave;
  // two chunks per iteration: 8 W loads of 16 bytes in flight per lane
  for (; c + nw < nchunks; c += 2 * nw) {
    uint4 wv[2][4], xv[2][MT][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k0 = (c + u * nw) * kGvChunk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool in = k0 + 32 * h + 8 * q < K;
        wv[u][q] = in ? ld_stream(wrow + k0 + 8 * q) : zero;
#pragma unroll
        for (int t = 0; t < MT; ++t)
          xv[u][t][q] = (in && xok[t]) ? *(const uint4*)(xrow[t] + k0 + 8 * q) : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[u][q]),
                                                          __builtin_bit_cast(bf16x8_t, xv[u][t][q]),
                                                          acc[t], 0, 0, 0);
  }
  for (; c < nchunks; c += nw) {
    const int k0 = c * kGvChunk;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool in = k0 + 32 * h + 8 * q < K;
      uint4 wq = in ? ld_stream(wrow + k0 + 8 * q) : zero;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        uint4 xq = (in && xok[t]) ? *(const uint4*)(xrow[t] + k0 + 8 * q) : zero;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wq),
                                                        __builtin_bit_cast(bf16x8_t, xq), acc[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  // wave t finishes column tile t (a single wave does both when nw == 1)
  for (int t = wave; t < MT; t += nw) {
    f32x4_t s = red[0][t][lane];
    for (int v = 1; v < nw; ++v) s += red[v][t][lane];
    const int m = (lane & 15) + 16 * t;
    if (m < M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 4 * (lane >> 4) + r;
        if (n < N) {
          uint32_t u = __float_as_uint(s[r]);
          y[(int64_t)m * N + n] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
        }
      }
    }
  }
}

hipError_t launch_gemv(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                       const DeviceInfo& dev, hipStream_t stream) {
  const int nwg = (int)((N + 15) / 16);
  const int nchunks = (int)((K + kGvChunk - 1) / kGvChunk);
  // aim for about eight waves per CU over the whole grid
  int nw = (8 * dev.num_cu + nwg - 1) / nwg;
  nw = nw < 4 ? 4 : nw;
  nw = nw > kGvMaxWaves ? kGvMaxWaves : nw;
  nw = nw > nchunks ? (nchunks < 1 ? 1 : nchunks) : nw;
  if (M <= 16) {
    hipLaunchKernelGGL(gemv_bf16_kernel<1>, dim3(nwg), dim3(nw * 64), 0, stream, (const uint16_t*)x,
                       (const uint16_t*)w, (uint16_t*)y, (int)M, (int)N, (int)K);
  } else {
    hipLaunchKernelGGL(gemv_bf16_kernel<2>, dim3(nwg), dim3(nw * 64), 0, stream, (const uint16_t*)x,
                       (const uint16_t*)w, (uint16_t*)y, (int)M, (int)N, (int)K);
  }
  return hipGetLastError();
}

}  // namespace mq
