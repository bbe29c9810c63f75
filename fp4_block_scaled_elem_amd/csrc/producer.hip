// producer.hip - the ops that write the prefill linears' activations, with
// the activation quantizer's amax pass folded into them (gfx950).
//
// NVFP4's tensor-level scale of an activation comes from the absolute
// maximum of the whole tensor, taken at run time (gist.science English
// explainer of "Mix-Quant: Quantized Prefilling, Precise Decoding for
// Agentic LLMs", Technical Summary s.2 Hybrid Precision Strategy), which
// costs the quantizer one full read of the activation before it can encode.
// The op that writes the activation can take that maximum on the way out:
// each workgroup stores one partial maximum of the bf16 values it wrote,
// in the layout of the amax pass's record (binary32 bits of a bf16
// magnitude per workgroup, their count in nparts), and the encode pass then
// runs alone (MQ_SCALE_PARTIALS).  The two ops of an 8B-shaped layer that
// produce the linears' inputs:
//   rmsnorm_amax_kernel  y = bf16((x * rstd) * g), rstd = 1 / sqrt(mean(x^2)
//                        + eps) per row, a wave per row (grid-stride);
//   swiglu_amax_kernel   y = bf16(silu(a) * b), silu(a) = a / (1 + exp(-a)),
//                        elementwise, 16-byte loads.
// Both are HBM-bound: 2 bytes read and 2 written per element (RMSNorm),
// 4 read and 2 written (SwiGLU).  The RMSNorm also comes fused with the
// quantization, when y feeds only the linears (the q/k/v and gate/up
// inputs): a first pass takes the maxima without storing y, a second
// recomputes y and encodes it (rmsnorm_encode_kernel), so y never goes to
// HBM: 2 + 2.5625 bytes per element instead of 2 + 2 + 2.5625.  Their outputs are rounded binary32 results, not bit-identical
// to any other order of evaluation; the maxima they emit are those of the
// exact bf16 values they store.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

constexpr int kPThreads = 256;

template <int NT>
__device__ __forceinline__ uint32_t block_max_bits(uint32_t v, uint32_t* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r = r > sh[i] ? r : sh[i];
  return r;
}

// nearest-even bf16 bits of a finite binary32
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// One wave per row (a workgroup's eight waves take eight rows at a time,
// grid-stride over rows; eight so that 4096 rows fit in one round of the
// workgroups the record has partial slots for), no block barriers in the
// loop.  A row of up to
// 64 * 8 * kRowPieces elements stays in registers between the sum of squares
// and the output; longer rows are read twice (the second time from L2).
// 8 elements per 16-byte piece, cols % 16 == 0.
constexpr int kRowPieces = 8;  // pieces per lane held in registers: rows up to 4096 elements
constexpr int kRThreads = 512;  // eight waves per workgroup

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ uint4 rms_piece(uint4 v, uint4 gv, float rstd, uint32_t& am) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = bf16_bits_rne((bf16_lo(w[j]) * rstd) * bf16_lo(gw[j]));
    const uint32_t hi = bf16_bits_rne((bf16_hi(w[j]) * rstd) * bf16_hi(gw[j]));
    o[j] = lo | (hi << 16);
    const uint32_t m = bf16x2_absmax_bits(o[j]);
    am = am > m ? am : m;
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float sumsq_piece(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
    ss += lo * lo;
    ss += hi * hi;
  }
  return ss;
}

// STORE false: the maxima alone (the first pass of the RMSNorm fused with
// quantization, whose second pass recomputes y).
template <bool STORE>
__global__ __launch_bounds__(kRThreads) void rmsnorm_amax_kernel(const uint4* __restrict__ x,
                                                                 const uint4* __restrict__ g,
                                                                 uint4* __restrict__ y, int64_t rows, int cols,
                                                                 float eps, mq_scale_rec* __restrict__ rec) {
  __shared__ uint32_t shm[kRThreads / 64];
  constexpr int kWaves = kRThreads / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pieces = cols / 8;
  const float inv_cols = 1.0f / (float)cols;
  uint32_t am = 0;  // max bf16 magnitude bits written by this lane
  const int64_t rstride = (int64_t)gridDim.x * kWaves;
  const int64_t r0 = (int64_t)blockIdx.x * kWaves + wave;
  if (!STORE && pieces <= 64 * kRowPieces) {
    // maxima only (the fused quantization's first pass): rows one ahead
    // (the next row's loads go out before this row's math), gamma loaded
    // once per wave, and x read through the caches, where the second pass
    // finds it
    uint4 gv[kRowPieces], v[kRowPieces];
    auto load_row = [&](int64_t row, uint4 (&dst)[kRowPieces]) __attribute__((always_inline)) {
      const uint4* xr = x + row * pieces;
#pragma unroll
      for (int k = 0; k < kRowPieces; ++k) {
        const int p = lane + 64 * k;
        dst[k] = (p < pieces && row < rows) ? xr[p] : make_uint4(0, 0, 0, 0);
      }
    };
#pragma unroll
    for (int k = 0; k < kRowPieces; ++k) {
      const int p = lane + 64 * k;
      gv[k] = p < pieces ? g[p] : make_uint4(0, 0, 0, 0);
    }
    load_row(r0, v);
    for (int64_t r = r0; r < rows; r += rstride) {
      uint4 nv[kRowPieces];
      load_row(r + rstride, nv);
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < kRowPieces; ++k) ss += sumsq_piece(v[k]);
      const float rstd = 1.0f / sqrtf(wave_sum_f32(ss) * inv_cols + eps);
#pragma unroll
      for (int k = 0; k < kRowPieces; ++k) {
        const int p = lane + 64 * k;
        if (p < pieces) (void)rms_piece(v[k], gv[k], rstd, am);
      }
#pragma unroll
      for (int k = 0; k < kRowPieces; ++k) v[k] = nv[k];
    }
  } else {
    for (int64_t r = r0; r < rows; r += rstride) {
      const uint4* xr = x + r * pieces;
      uint4* yr = y + r * pieces;
      if (pieces <= 64 * kRowPieces) {
        uint4 v[kRowPieces];
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < kRowPieces; ++k) {
          const int p = lane + 64 * k;
          v[k] = p < pieces ? ld_stream(&xr[p]) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kRowPieces; ++k) ss += sumsq_piece(v[k]);
        const float rstd = 1.0f / sqrtf(wave_sum_f32(ss) * inv_cols + eps);
#pragma unroll
        for (int k = 0; k < kRowPieces; ++k) {
          const int p = lane + 64 * k;
          if (p < pieces) {
            const uint4 o = rms_piece(v[k], g[p], rstd, am);
            if constexpr (STORE) yr[p] = o;
          }
        }
      } else {
        float ss = 0.0f;
        for (int p = lane; p < pieces; p += 64) ss += sumsq_piece(xr[p]);
        const float rstd = 1.0f / sqrtf(wave_sum_f32(ss) * inv_cols + eps);
        for (int p = lane; p < pieces; p += 64) {
          const uint4 o = rms_piece(xr[p], g[p], rstd, am);
          if constexpr (STORE) yr[p] = o;
        }
      }
    }
  }
  const uint32_t m = block_max_bits<kRThreads>(am, shm);
  if (threadIdx.x == 0) {
    rec->part[blockIdx.x] = m << 16;
    if (blockIdx.x == 0) rec->nparts = gridDim.x;
  }
}

// Second pass of the RMSNorm fused with NVFP4 quantization: the tensor
// scale from the first pass's partial maxima (as the encode pass reduces
// them), then every row's y recomputed exactly as rmsnorm_amax_kernel
// computes it (the same functions in the same order, so the same bf16
// values) and encoded as the quantizer's encode pass encodes a half-group
// per lane: a row's pieces 2q and 2q + 1 (one 16-element group) sit in
// lanes 2j and 2j + 1, which swap their half maxima.  y itself is never
// stored.
template <bool OVF>
__device__ __forceinline__ void encode_piece(uint4 yv, int64_t h, const GroupScaleTab& tab,
                                             uint32_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const uint32_t w[4] = {yv.x, yv.y, yv.z, yv.w};
  uint32_t am = bf16_absmax_bits<4>(w);
  const uint32_t other = __shfl_xor(am, 1, 64);
  am = am > other ? am : other;
  float e;
  const uint32_t S = group_scale(am, tab, e);
  codes[h] = encode8<OVF>(w, e);
  if ((h & 1) == 0) scales[h >> 1] = (uint8_t)S;
}

__global__ __launch_bounds__(kRThreads) void rmsnorm_encode_kernel(const uint4* __restrict__ x,
                                                                   const uint4* __restrict__ g, int64_t rows,
                                                                   int cols, float eps,
                                                                   uint32_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ scales,
                                                                   mq_scale_rec* __restrict__ rec) {
  __shared__ uint32_t shm[kRThreads / 64];
  __shared__ float recip[128];
  constexpr int kWaves = kRThreads / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pieces = cols / 8;  // even: a group never straddles two lanes' rows
  const float inv_cols = 1.0f / (float)cols;
  const int64_t rstride = (int64_t)gridDim.x * kWaves;
  int64_t r = (int64_t)blockIdx.x * kWaves + wave;
  const bool regs = pieces <= 64 * kRowPieces;
  // rows held in registers: gamma's pieces once per wave, the wave's first
  // row in flight before the tensor scale is reduced
  uint4 gv[kRowPieces], v[kRowPieces];
  auto load_row = [&](int64_t row, uint4 (&dst)[kRowPieces]) __attribute__((always_inline)) {
    const uint4* xr = x + row * pieces;
#pragma unroll
    for (int k = 0; k < kRowPieces; ++k) {
      const int p = lane + 64 * k;
      dst[k] = (p < pieces && row < rows) ? ld_stream(&xr[p]) : make_uint4(0, 0, 0, 0);
    }
  };
  if (regs) {
#pragma unroll
    for (int k = 0; k < kRowPieces; ++k) {
      const int p = lane + 64 * k;
      gv[k] = p < pieces ? g[p] : make_uint4(0, 0, 0, 0);
    }
    load_row(r, v);
  }
  // the partial maxima (the count clamped to the record's capacity)
  const uint32_t n = min(rec->nparts, (uint32_t)MQ_AMAX_PARTS);
  uint32_t m = 0;
  for (uint32_t j = threadIdx.x; j < n; j += kRThreads) {
    const uint32_t pv = rec->part[j];
    m = m > pv ? m : pv;
  }
  const uint32_t amax = block_max_bits<kRThreads>(m, shm);
  const float s_t = tensor_scale_from_amax(amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    rec->s_t = s_t;
    rec->amax_bits = amax;
  }
  const GroupScaleTab tab = group_scale_tab<kRThreads>(s_t, recip);
  auto run = [&](auto ovf_c) __attribute__((always_inline)) {
    constexpr bool OVF = decltype(ovf_c)::value;
    uint32_t unused = 0;
    if (regs) {
      // one row ahead: the next row's loads go out before this row's math
      for (; r < rows; r += rstride) {
        uint4 nv[kRowPieces];
        load_row(r + rstride, nv);
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < kRowPieces; ++k) ss += sumsq_piece(v[k]);
        const float rstd = 1.0f / sqrtf(wave_sum_f32(ss) * inv_cols + eps);
        const int64_t h0 = r * pieces;  // the row's first half-group
#pragma unroll
        for (int k = 0; k < kRowPieces; ++k) {
          const int p = lane + 64 * k;
          if (p < pieces) encode_piece<OVF>(rms_piece(v[k], gv[k], rstd, unused), h0 + p, tab, codes, scales);
        }
#pragma unroll
        for (int k = 0; k < kRowPieces; ++k) v[k] = nv[k];
      }
    } else {
      for (; r < rows; r += rstride) {
        const uint4* xr = x + r * pieces;
        float ss = 0.0f;
        for (int p = lane; p < pieces; p += 64) ss += sumsq_piece(xr[p]);
        const float rstd = 1.0f / sqrtf(wave_sum_f32(ss) * inv_cols + eps);
        for (int p = lane; p < pieces; p += 64)
          encode_piece<OVF>(rms_piece(xr[p], g[p], rstd, unused), r * pieces + p, tab, codes, scales);
      }
    }
  };
  if (tab.ovf)
    run(BoolC<true>{});
  else
    run(BoolC<false>{});
}

// Elementwise over n8 pieces of 8 elements, grid-stride.
__global__ __launch_bounds__(kPThreads) void swiglu_amax_kernel(const uint4* __restrict__ a,
                                                                const uint4* __restrict__ b,
                                                                uint4* __restrict__ y, int64_t n8,
                                                                mq_scale_rec* __restrict__ rec) {
  __shared__ uint32_t shm[kPThreads / 64];
  uint32_t am = 0;
  const int64_t stride = (int64_t)gridDim.x * kPThreads;
  for (int64_t i = (int64_t)blockIdx.x * kPThreads + threadIdx.x; i < n8; i += stride) {
    const uint4 va = ld_stream(&a[i]), vb = ld_stream(&b[i]);
    const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = bf16_lo(wa[j]), a1 = bf16_hi(wa[j]);
      // silu(a) = a * (1 / (1 + exp(-a))); exp(-a) = inf for very negative a
      // gives a * 0 = -0
      const float s0 = a0 * __builtin_amdgcn_rcpf(1.0f + __expf(-a0));
      const float s1 = a1 * __builtin_amdgcn_rcpf(1.0f + __expf(-a1));
      const uint32_t lo = bf16_bits_rne(s0 * bf16_lo(wb[j]));
      const uint32_t hi = bf16_bits_rne(s1 * bf16_hi(wb[j]));
      o[j] = lo | (hi << 16);
      const uint32_t m = bf16x2_absmax_bits(o[j]);
      am = am > m ? am : m;
    }
    y[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  const uint32_t m = block_max_bits<kPThreads>(am, shm);
  if (threadIdx.x == 0) {
    rec->part[blockIdx.x] = m << 16;
    if (blockIdx.x == 0) rec->nparts = gridDim.x;
  }
}

static int64_t rmsnorm_blocks(int64_t rows, const DeviceInfo& dev) {
  const int64_t row_groups = (rows + kRThreads / 64 - 1) / (kRThreads / 64);  // eight rows per workgroup
  int64_t blocks = row_groups < 2 * (int64_t)dev.num_cu ? row_groups : 2 * (int64_t)dev.num_cu;
  return blocks > MQ_AMAX_PARTS ? MQ_AMAX_PARTS : blocks;
}

hipError_t launch_rmsnorm_amax(const void* x, const void* g, void* y, int64_t rows, int64_t cols, float eps,
                               mq_scale_rec* rec, const DeviceInfo& dev, hipStream_t stream) {
  const int64_t blocks = rmsnorm_blocks(rows, dev);
  log_launch("rmsnorm_amax_kernel", blocks, kRThreads, 0, "rows=%lld cols=%lld store=1", (long long)rows,
             (long long)cols);
  hipLaunchKernelGGL(rmsnorm_amax_kernel<true>, dim3((unsigned)blocks), dim3(kRThreads), 0, stream,
                     (const uint4*)x, (const uint4*)g, (uint4*)y, rows, (int)cols, eps, rec);
  return hipGetLastError();
}

// The fused passes take a workgroup per CU, so that each wave has rows to
// pipeline (two at 4096 rows).
hipError_t launch_rmsnorm_quantize(const void* x, const void* g, int64_t rows, int64_t cols, float eps,
                                   uint8_t* codes, uint8_t* scales, mq_scale_rec* rec, const DeviceInfo& dev,
                                   hipStream_t stream) {
  const int64_t row_groups = (rows + kRThreads / 64 - 1) / (kRThreads / 64);
  const int64_t blocks = row_groups < (int64_t)dev.num_cu ? row_groups : (int64_t)dev.num_cu;
  log_launch("rmsnorm_amax_kernel", blocks, kRThreads, 0, "rows=%lld cols=%lld store=0", (long long)rows,
             (long long)cols);
  hipLaunchKernelGGL(rmsnorm_amax_kernel<false>, dim3((unsigned)blocks), dim3(kRThreads), 0, stream,
                     (const uint4*)x, (const uint4*)g, nullptr, rows, (int)cols, eps, rec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  log_launch("rmsnorm_encode_kernel", blocks, kRThreads, 0, "rows=%lld cols=%lld", (long long)rows,
             (long long)cols);
  hipLaunchKernelGGL(rmsnorm_encode_kernel, dim3((unsigned)blocks), dim3(kRThreads), 0, stream, (const uint4*)x,
                     (const uint4*)g, rows, (int)cols, eps, (uint32_t*)codes, scales, rec);
  return hipGetLastError();
}

hipError_t launch_swiglu_amax(const void* a, const void* b, void* y, int64_t n, mq_scale_rec* rec,
                              const DeviceInfo& dev, hipStream_t stream) {
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + 4 * kPThreads - 1) / (4 * kPThreads);
  if (blocks > 2 * (int64_t)dev.num_cu) blocks = 2 * (int64_t)dev.num_cu;
  if (blocks > MQ_AMAX_PARTS) blocks = MQ_AMAX_PARTS;
  if (blocks < 1) blocks = 1;
  log_launch("swiglu_amax_kernel", blocks, kPThreads, 0, "elements=%lld", (long long)n);
  hipLaunchKernelGGL(swiglu_amax_kernel, dim3((unsigned)blocks), dim3(kPThreads), 0, stream, (const uint4*)a,
                     (const uint4*)b, (uint4*)y, n8, rec);
  return hipGetLastError();
}

}  // namespace mq
