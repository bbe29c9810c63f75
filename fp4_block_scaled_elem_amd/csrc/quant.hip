// quant.hip - dynamic activation quantization to NVFP4 (gfx950).
//
// Two passes, because the tensor-level scale of NVFP4 (gist.science English
// explainer of "Mix-Quant: Quantized Prefilling, Precise Decoding for Agentic
// LLMs", Technical Summary s.2, Hybrid Precision Strategy) depends on the
// absolute maximum of the whole input, which must be known before any code
// can be emitted:
//   1. amax_kernel: streaming max|x| over the bf16 input; each workgroup
//      writes one partial maximum into the scale record (no atomics, no
//      pre-zeroed memory needed).
//   2. quantize_kernel: every workgroup reduces the partials (at most a few
//      KB, L2-resident), derives s_t, then encodes 16-element groups.  One
//      lane owns 8 consecutive elements (one 16-byte load, fully coalesced);
//      the two lanes of a group exchange their half maxima with one
//      cross-lane swap; the element codes come from the hardware fp4
//      conversion of x * e, the reciprocal group scale e from a table of the
//      128 possible values built by each workgroup.
// Both passes are HBM-bound: 2 bytes read per element for the amax, 2 read
// plus 0.5625 written per element for the encode.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

constexpr int kQThreads = 256;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ uint32_t uint4_absmax(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  return bf16_absmax_bits<4>(w);
}

// Block-wide max of a per-thread value; every thread gets the result.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* sh) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint32_t r = 0;
  for (int i = 0; i < kQThreads / 64; ++i) r = r > sh[i] ? r : sh[i];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kQThreads) void amax_kernel(const uint4* __restrict__ x, int64_t n16,
                                                         mq_scale_rec* __restrict__ rec) {
  __shared__ uint32_t sh[kQThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kQThreads;
  int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  uint32_t m0 = 0, m1 = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    // ordinary (cached) loads: the encode pass reads the same bytes next,
    // and finds part of them in the caches (3% faster for both passes than
    // streaming loads here, measured)
    uint4 a = x[i];
    uint4 b = x[i + stride];
    uint4 c = x[i + 2 * stride];
    uint4 d = x[i + 3 * stride];
    uint32_t ma = uint4_absmax(a), mb = uint4_absmax(b), mc = uint4_absmax(c), md = uint4_absmax(d);
    ma = ma > mb ? ma : mb;
    mc = mc > md ? mc : md;
    m0 = m0 > ma ? m0 : ma;
    m1 = m1 > mc ? m1 : mc;
  }
  for (; i < n16; i += stride) {
    uint32_t ma = uint4_absmax(x[i]);
    m0 = m0 > ma ? m0 : ma;
  }
  uint32_t m = block_max_u32(m0 > m1 ? m0 : m1, sh);
  if (threadIdx.x == 0) {
    rec->part[blockIdx.x] = m << 16;  // binary32 bits of the bf16 magnitude
    if (blockIdx.x == 0) rec->nparts = gridDim.x;
  }
}

// Reduce the partial maxima of a record; every thread gets amax's bits.
// The count is clamped to the record's capacity: a record that no amax pass
// wrote (a caller's mistake) then gives a wrong scale, not reads past it.
__device__ __forceinline__ uint32_t reduce_parts(const mq_scale_rec* __restrict__ rec, uint32_t* sh) {
  const uint32_t n = min(rec->nparts, (uint32_t)MQ_AMAX_PARTS);
  uint32_t m = 0;
  for (uint32_t j = threadIdx.x; j < n; j += kQThreads) {
    uint32_t v = rec->part[j];
    m = m > v ? m : v;
  }
  return block_max_u32(m, sh);
}

// The scale record as the encode pass reads it: the given s_t, the number of
// partial maxima and the first two per thread (up to 2 * kQThreads partials
// without a loop), loaded before the input data, since a wait for a load
// also waits for every load issued before it.
struct RecHead {
  float s_t;
  uint32_t n, p[2];
};
__device__ __forceinline__ RecHead load_rec_head(const mq_scale_rec* __restrict__ rec) {
  RecHead r;
  r.s_t = rec->s_t;
  r.n = min(rec->nparts, (uint32_t)MQ_AMAX_PARTS);  // clamped as in reduce_parts
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = threadIdx.x + i * kQThreads;
    r.p[i] = j < MQ_AMAX_PARTS ? rec->part[j] : 0u;
  }
  return r;
}
__device__ __forceinline__ uint32_t reduce_rec_head(const RecHead& r, const mq_scale_rec* __restrict__ rec,
                                                    uint32_t* sh) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t j = threadIdx.x + i * kQThreads;
    if (j < r.n) m = m > r.p[i] ? m : r.p[i];
  }
  for (uint32_t j = threadIdx.x + 2 * kQThreads; j < r.n; j += kQThreads) {
    const uint32_t v = rec->part[j];
    m = m > v ? m : v;
  }
  return block_max_u32(m, sh);
}

// One lane owns 8 consecutive elements (one 16-byte load); the two lanes of a
// 16-element group swap their half maxima.  Each lane works on four
// half-groups per iteration, one stride apart, so four loads are in flight.
// given: 0 = s_t from the amax pass's partial maxima in rec, 1 = rec->s_t as
// set by the caller, 2 = every workgroup takes max|x| itself (small inputs).
__global__ __launch_bounds__(kQThreads) void quantize_kernel(const uint4* __restrict__ x, int64_t nhalf,
                                                             uint32_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             mq_scale_rec* __restrict__ rec, int given) {
  __shared__ uint32_t sh[kQThreads / 64];
  __shared__ float recip[128];
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * kQThreads;
  int64_t h = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  // The first iteration's loads go out before the tensor scale is known:
  // their latency overlaps the reduction of the partial maxima and the
  // table build (the barriers there wait for LDS traffic only).
  // These loads are unconditional (indices clamped into the input, which
  // holds at least two half-groups), so that the wait for the record's
  // loads can leave them in flight on every path.
  const RecHead head = load_rec_head(rec);
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = h + u * stride;
    v[u] = ld_stream(&x[i < nhalf ? i : nhalf - 1]);
  }
  float s_t;
  if (given == 1) {
    s_t = head.s_t;
  } else {
    uint32_t amax;
    if (given == 2) {
      // small input, no amax pass: every workgroup takes max|x| itself (the
      // same value), reading all of x, which stays in L2
      uint32_t m = 0;
      for (int64_t base = 0; base < nhalf; base += 8 * kQThreads) {
        uint4 t[8];  // eight loads in flight per lane
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t i = base + u * kQThreads + threadIdx.x;
          t[u] = x[i < nhalf ? i : nhalf - 1];  // a repeated element leaves the maximum unchanged
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t a = uint4_absmax(t[u]);
          m = m > a ? m : a;
        }
      }
      amax = block_max_u32(m, sh) << 16;  // binary32 bits, as the partial maxima
    } else {
      amax = reduce_rec_head(head, rec, sh);
    }
    s_t = tensor_scale_from_amax(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      rec->s_t = s_t;
      rec->amax_bits = amax;
    }
  }
  const GroupScaleTab tab = group_scale_tab<kQThreads>(s_t, recip);
  // nhalf and stride are even and a pair starts on an even index, so both
  // lanes of a group enter and leave every loop iteration together.  The
  // loops come in two copies, with and without encode8's overflow fix-up.
  auto run = [&](auto ovf_c) __attribute__((always_inline)) {
    constexpr bool OVF = decltype(ovf_c)::value;
    auto encode_iter = [&](const uint4 (&vv)[U]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t w[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        uint32_t am = uint4_absmax(vv[u]);
        const uint32_t other = __shfl_xor(am, 1, 64);
        am = am > other ? am : other;
        float e;
        const uint32_t S = group_scale(am, tab, e);
        const int64_t hu = h + u * stride;
        codes[hu] = encode8<OVF>(w, e);
        if ((hu & 1) == 0) scales[hu >> 1] = (uint8_t)S;
      }
    };
    if (h + (U - 1) * stride < nhalf) {  // first iteration: data already loaded
      encode_iter(v);
      h += U * stride;
    }
    for (; h + (U - 1) * stride < nhalf; h += U * stride) {
      uint4 nv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) nv[u] = ld_stream(&x[h + u * stride]);
      encode_iter(nv);
    }
    for (; h < nhalf; h += stride) {
      const uint4 t = ld_stream(&x[h]);
      const uint32_t w[4] = {t.x, t.y, t.z, t.w};
      uint32_t am = uint4_absmax(t);
      const uint32_t other = __shfl_xor(am, 1, 64);
      am = am > other ? am : other;
      float e;
      const uint32_t S = group_scale(am, tab, e);
      codes[h] = encode8<OVF>(w, e);
      if ((h & 1) == 0) scales[h >> 1] = (uint8_t)S;
    }
  };
  if (tab.ovf)
    run(BoolC<true>{});
  else
    run(BoolC<false>{});
}

static int grid_for(int64_t items, int threads, int max_blocks) {
  int64_t b = (items + threads - 1) / threads;
  if (b > max_blocks) b = max_blocks;
  if (b < 1) b = 1;
  return (int)b;
}

hipError_t launch_amax(const void* x_bf16, int64_t nelem, mq_scale_rec* rec, const DeviceInfo& dev,
                       hipStream_t stream) {
  const int64_t n16 = nelem / 8;
  // two workgroups per CU: enough loads in flight for HBM, and few partial
  // maxima for every quantize workgroup to reduce (measured faster than four)
  int blocks = grid_for((n16 + 3) / 4, kQThreads, dev.num_cu * 2);
  if (blocks > MQ_AMAX_PARTS) blocks = MQ_AMAX_PARTS;
  log_launch("amax_kernel", blocks, kQThreads, 0, "elements=%lld", (long long)nelem);
  hipLaunchKernelGGL(amax_kernel, dim3(blocks), dim3(kQThreads), 0, stream,
                     (const uint4*)x_bf16, n16, rec);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x_bf16, int64_t nelem, uint8_t* codes, uint8_t* scales,
                           mq_scale_rec* rec, bool given, const DeviceInfo& dev, hipStream_t stream,
                           bool inline_amax) {
  const int64_t nhalf = nelem / 8;  // 8 elements per lane, two lanes per group
  int blocks = grid_for((nhalf + 3) / 4, kQThreads, dev.num_cu * 8);
  const int mode = given ? 1 : (inline_amax ? 2 : 0);
  log_launch("quantize_kernel", blocks, kQThreads, 0, "elements=%lld mode=%d", (long long)nelem, mode);
  hipLaunchKernelGGL(quantize_kernel, dim3(blocks), dim3(kQThreads), 0, stream,
                     (const uint4*)x_bf16, nhalf, (uint32_t*)codes, scales, rec, mode);
  return hipGetLastError();
}

}  // namespace mq
