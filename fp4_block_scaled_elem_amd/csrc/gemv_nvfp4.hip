// gemv_nvfp4.hip - NVFP4 x NVFP4 decode GEMV / skinny GEMM (gfx950): the
// uniform-NVFP4 decode that the method departs from.
//
// "Mix-Quant: Quantized Prefilling, Precise Decoding for Agentic LLMs"
// (gist.science English explainer, Technical Summary s.1 Problem Statement:
// low-bit quantization of both phases speeds the computation up but degrades
// the output, because decode errors accumulate over long trajectories; s.4
// Experimental Results: uniform NVFP4 scores below Mix-Quant) keeps decode
// in BF16.  This kernel runs the decode step the uniform way, with the
// prefill format in both operands, so that the two decode paths can be put
// side by side on bytes moved and time.  The arithmetic is the prefill
// GEMM's: exact binary16 operands g*sigma, binary32 accumulation, the sum
// scaled by s_tA*s_tW and rounded to nearest-even bf16.  With M <= 32 rows
// of X it is bound by streaming W's 0.5625 bytes per weight:
//   - a workgroup owns 16 rows of W; its eight waves take the K chunks (256
//     elements: 128 code bytes + 16 scale bytes per row) in turn;
//   - lane (i, h) of a wave loads row i's K elements 64h .. 64h+63 of a
//     chunk: 32 code bytes and the 4 scale bytes of those groups, for W and
//     for each 16-row tile of X (X is small and stays in L2); the next
//     chunk's loads are issued before this chunk is used;
//   - a lane's 64 elements feed eight v_mfma_f32_16x16x32_f16 steps, eight
//     elements per step; the K order inside a chunk is the same for W and X,
//     so the sum is the dot product;
//   - dequantization in registers (hardware fp4 -> f16, one packed multiply
//     by sigma: exact);
//   - the waves' partial tiles are summed through LDS in a fixed order
//     (deterministic), scaled, rounded and stored.
// K % 256 == 0 loads whole 16-byte pieces; other K (K % 16 == 0) load group
// by group, each bounds-checked.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

constexpr int kGnWaves = 8;      // waves per workgroup (split K)
constexpr int kGnChunk = 256;    // K elements per chunk

// One operand row's share of a chunk for one lane: 8 code dwords (K steps
// 0..7) and the 4 scale bytes (groups 0..3) as one dword.
struct GnFrag {
  uint32_t c[8];
  uint32_t s;
};

// The lane's share of chunk `chunk` of row `row` (a valid row: rows past N
// or M are clamped by the caller; they only feed outputs that are never
// stored).  Every load is unconditional, so that waiting for one chunk never
// waits for loads issued after it; groups past K (ragged K only) are loaded
// from a clamped index and zeroed by a select.
template <bool FAST>
__device__ __forceinline__ GnFrag gn_load(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                          int row, int K, int chunk, int h) {
  GnFrag f;
  const int g0 = chunk * (kGnChunk / 16) + 4 * h;  // first group of the lane
  const uint8_t* crow = codes + (int64_t)row * (K / 2);
  const uint8_t* srow = scales + (int64_t)row * (K / 16);
  if constexpr (FAST) {
    // whole chunks: 16-byte aligned codes, 4-byte aligned scales
    const u32x4_t a = *(const u32x4_t*)(crow + g0 * 8);
    const u32x4_t b = *(const u32x4_t*)(crow + g0 * 8 + 16);
    f.c[0] = a[0]; f.c[1] = a[1]; f.c[2] = a[2]; f.c[3] = a[3];
    f.c[4] = b[0]; f.c[5] = b[1]; f.c[6] = b[2]; f.c[7] = b[3];
    f.s = *(const uint32_t*)(srow + g0);
  } else {
    const int G = K / 16;
    f.s = 0u;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const bool ok = g0 + g < G;
      const int gc = ok ? g0 + g : G - 1;
      const u32x2_t v = *(const u32x2_t*)(crow + gc * 8);
      const uint32_t sb = srow[gc];
      f.c[2 * g] = ok ? v[0] : 0u;
      f.c[2 * g + 1] = ok ? v[1] : 0u;
      f.s |= (ok ? sb : 0u) << (8 * g);
    }
  }
  return f;
}

// MT column tiles of X (16 rows each) against 16 rows of W per workgroup.
template <int MT, bool FAST>
__global__ __launch_bounds__(kGnWaves * 64) void gemv_nvfp4_kernel(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, const mq_scale_rec* __restrict__ xrec,
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws, const mq_scale_rec* __restrict__ wrec,
    uint16_t* __restrict__ y, int M, int N, int K) {
  __shared__ f32x4_t red[kGnWaves][MT][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int i = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16;
  // rows past N (W) or M (X) read the last row instead: they only feed
  // outputs that are never stored
  const int wrow = min(n0 + i, N - 1);
  int xrow[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) xrow[u] = min(16 * u + i, M - 1);
  const int nchunks = (K + kGnChunk - 1) / kGnChunk;
  const int mine = nchunks > wave ? (nchunks - wave + kGnWaves - 1) / kGnWaves : 0;  // this wave's chunks

  f32x4_t acc[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // chunk t of this wave.  Past the last chunk it re-reads that chunk (the
  // loads stay unconditional, so waiting for one chunk never waits for the
  // next); compute then zeroes W's scales, and the chunk adds nothing.
  auto load = [&](int t, GnFrag& fw, GnFrag (&fx)[MT]) __attribute__((always_inline)) {
    const int c = wave + kGnWaves * min(t, mine - 1);
    fw = gn_load<FAST>(wc, ws, wrow, K, c, h);
#pragma unroll
    for (int u = 0; u < MT; ++u) fx[u] = gn_load<FAST>(xc, xs, xrow[u], K, c, h);
  };
  auto compute = [&](const GnFrag& fw, const GnFrag (&fx)[MT], bool live) __attribute__((always_inline)) {
    const uint32_t wsc = live ? fw.s : 0u;
    const half2_t sw01 = sigma_pair<false>(wsc), sw23 = sigma_pair<true>(wsc);
    half2_t sx01[MT], sx23[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      sx01[u] = sigma_pair<false>(fx[u].s);
      sx23[u] = sigma_pair<true>(fx[u].s);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int g = q >> 1;  // group of step q
      const half8_t a = dequant8(fw.c[q], g < 2 ? sw01[g] : sw23[g - 2]);
#pragma unroll
      for (int u = 0; u < MT; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            a, dequant8(fx[u].c[q], g < 2 ? sx01[u][g] : sx23[u][g - 2]), acc[u], 0, 0, 0);
    }
  };
  // Two register buffers in turn, one chunk ahead (no copies between them:
  // a copy would wait for the prefetch); an odd share ends on a zeroed chunk.
  if (mine > 0) {
    GnFrag aw, ax[MT], bw, bx[MT];
    load(0, aw, ax);
    for (int t = 0; t < mine; t += 2) {
      load(t + 1, bw, bx);
      __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before this chunk's math
      compute(aw, ax, true);
      load(t + 2, aw, ax);
      __builtin_amdgcn_sched_barrier(0);
      compute(bw, bx, t + 1 < mine);
    }
  }
#pragma unroll
  for (int u = 0; u < MT; ++u) red[wave][u][lane] = acc[u];
  __syncthreads();
  // wave u finishes column tile u: the waves' partials in wave order
  if (wave < MT) {
    const int u = wave;
    f32x4_t s = red[0][u][lane];
    for (int v = 1; v < kGnWaves; ++v) s += red[v][u][lane];
    const float scale = xrec->s_t * wrec->s_t;
    const int m = (lane & 15) + 16 * u;
    if (m < M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 4 * (lane >> 4) + r;
        if (n < N) {
          const uint32_t b = __float_as_uint(s[r] * scale);
          y[(int64_t)m * N + n] = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
        }
      }
    }
  }
}

template <int MT, bool FAST>
static hipError_t launch_gn(const GemvNvfp4Args& a, hipStream_t stream) {
  log_launch("gemv_nvfp4_kernel", (unsigned)((a.N + 15) / 16), kGnWaves * 64, 0,
             "column_tiles=%d fast=%d M=%lld N=%lld K=%lld", MT, (int)FAST, (long long)a.M, (long long)a.N,
             (long long)a.K);
  hipLaunchKernelGGL((gemv_nvfp4_kernel<MT, FAST>), dim3((unsigned)((a.N + 15) / 16)), dim3(kGnWaves * 64), 0,
                     stream, a.x_codes, a.x_scales, a.x_rec, a.w_codes, a.w_scales, a.w_rec, (uint16_t*)a.y,
                     (int)a.M, (int)a.N, (int)a.K);
  return hipGetLastError();
}

hipError_t launch_gemv_nvfp4(const GemvNvfp4Args& a, hipStream_t stream) {
  // fast loads need whole chunks and 16-byte aligned rows of codes and 4-byte
  // aligned rows of scales (K % 256 == 0 gives both, given aligned bases)
  const bool fast = a.K % kGnChunk == 0 && ((uintptr_t)a.x_codes & 15) == 0 && ((uintptr_t)a.w_codes & 15) == 0 &&
                    ((uintptr_t)a.x_scales & 3) == 0 && ((uintptr_t)a.w_scales & 3) == 0;
  if (a.M <= 16) return fast ? launch_gn<1, true>(a, stream) : launch_gn<1, false>(a, stream);
  return fast ? launch_gn<2, true>(a, stream) : launch_gn<2, false>(a, stream);
}

}  // namespace mq
