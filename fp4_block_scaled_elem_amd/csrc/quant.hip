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
// plus 0.5625 written per element for the encode.  For the input lengths
// where it pays, quantize_resident_kernel (below) does both in one launch,
// reading the input once.
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

// ------------------------------------------------- single-launch quantizer --
//
// The dynamic scale in one launch.  One workgroup of kRThreads per CU; lane
// g (of T = grid x kRThreads) owns the half-groups g, g + T, g + 2T, ...; the
// first R of them stay in registers from the maximum to the encode (the
// next ones, for inputs too long for the register file, in LDS), so the
// input is read from HBM once.  The workgroups meet at the tensor maximum
// through the record: each stores its maximum, tagged with the call's epoch
// in the low 16 bits (always zero in a binary32 pattern of a bf16 magnitude),
// in its slot of part[]; one wave per workgroup reads all slots until every
// slot carries the tag.  The epoch
// comes from rec->flags, which every workgroup of a call increments once at
// its start: with the record zeroed when allocated and a grid that is the
// same for every call on a device, all workgroups of a call read values in
// [c * grid, (c + 1) * grid) and agree on c.  Every slot is rewritten by
// every call, so a slot carries this call's tag only once this call wrote
// it.  The wait is bounded: a workgroup that runs out of polls (its partners
// not resident, say) takes the maximum over the whole input itself, which
// gives the same bits, so the result never depends on the wait.
constexpr int kRThreads = 512;
constexpr int kRMaxResident = 48;  // uint4 per lane kept in registers at most
constexpr int kRHeldLds = 16;      // and beyond them, per lane, in LDS (128 KB per workgroup)
typedef __attribute__((address_space(3))) void rq_lds_t;

__device__ uint32_t g_rq_spin_limit = 1u << 16;  // polls before a workgroup gives up (0: never wait)
__device__ uint32_t g_rq_gave_up = 0;             // workgroups that gave up, for tests

template <int NT>
__device__ __forceinline__ uint32_t block_max_n(uint32_t v, uint32_t* sh) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r = r > sh[i] ? r : sh[i];
  __syncthreads();
  return r;
}

// Operands through buffer resources: a lane's half-group j sits at lane
// offset (g + j x T) x 16, formed just before each access (so the R
// resident half-groups cost no address registers), and lane offsets past the
// input read zeros (which leave the maximum unchanged) and drop stores.  The
// whole offset is the lane's: the range check covers it, not only the part
// of a scalar offset.  Requires the input under 4 GiB (host-checked).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rq_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);  // raw, 32-bit format
}

// HOLD: the half-groups R .. R + kRHeldLds - 1 of a lane wait in LDS
// (dynamic LDS, direct-to-LDS copies, 1 KB per wave and half-group) instead
// of being read again for the encode.
template <int R, bool HOLD>
__global__ __launch_bounds__(kRThreads, 1) void quantize_resident_kernel(const uint4* __restrict__ x, uint32_t nhalf,
                                                                         int J, uint32_t* __restrict__ codes,
                                                                         uint8_t* __restrict__ scales,
                                                                         mq_scale_rec* __restrict__ rec) {
  extern __shared__ __attribute__((aligned(16))) uint8_t held[];  // [kRHeldLds][waves][64 lanes][16 B]
  __shared__ uint32_t sh[kRThreads / 64];
  __shared__ float recip[128];
  __shared__ uint32_t tag_sh;
  __shared__ uint32_t amax_sh;
  __shared__ int ok_sh;
  const uint32_t G = gridDim.x;  // <= kRThreads, host-checked
  const uint32_t T = G * kRThreads;
  const uint32_t g0 = blockIdx.x * kRThreads + threadIdx.x;
  const uint32_t limit = g_rq_spin_limit;
  const __amdgpu_buffer_rsrc_t rx = rq_rsrc(x, nhalf * 16u);
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&rec->flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tag_sh = (old / G) % 65535u + 1u;  // 1..65535: never the zero of an untagged maximum
  }
  auto load = [&](uint32_t j) __attribute__((always_inline)) {
    const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)((g0 + j * T) * 16u), 0, 2 /* nt */);
    return make_uint4(t[0], t[1], t[2], t[3]);
  };
  // every resident half-group in flight at once
  uint4 v[R];
#pragma unroll
  for (int j = 0; j < R; ++j) v[j] = load(j);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto held_at = [&](int k) __attribute__((always_inline)) {
    return held + ((k * (kRThreads / 64) + wave_u) * 64) * 16;  // the wave's 1 KB for half-group R + k
  };
  if constexpr (HOLD) {
    // past the input the copies write zeros (and are never encoded)
#pragma unroll
    for (int k = 0; k < kRHeldLds; ++k)
      if (R + k < J)  // the same for the whole grid
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (rq_lds_t*)held_at(k), 16, (int)((g0 + (R + k) * T) * 16u), 0,
                                               0, 2 /* nt */);
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint32_t a = uint4_absmax(v[j]);
    m = m > a ? m : a;
  }
  if constexpr (HOLD) {
#pragma unroll
    for (int k = 0; k < kRHeldLds; ++k) {
      if (R + k >= J) break;
      const uint32_t a = uint4_absmax(*(const uint4*)(held_at(k) + lane * 16));
      m = m > a ? m : a;
    }
  } else {
    for (int j = R; j < J; ++j) {
      const uint32_t a = uint4_absmax(load(j));
      m = m > a ? m : a;
    }
  }
  // Up to 32 resident half-groups the encode reuses their maxima from here;
  // with more, it recomputes them (keeping them live across the wait would
  // spill).
  if constexpr (R > 32) {
#pragma unroll
    for (int j = 0; j < R; ++j) asm volatile("" : "+v"(v[j].x), "+v"(v[j].y), "+v"(v[j].z), "+v"(v[j].w));
  }
  m = block_max_n<kRThreads>(m, sh);  // its barriers also publish tag_sh
  const uint32_t tag = tag_sh;
  if (threadIdx.x == 0)
    __hip_atomic_store(&rec->part[blockIdx.x], (m << 16) | tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // wave 0 reads the slots: lane l those of index l mod 64
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int ok = limit != 0;
    uint32_t mx = 0;
    for (uint32_t polls = 0; ok;) {
      bool mine = true;
      mx = 0;
#pragma unroll
      for (int k = 0; k < kRThreads / 64; ++k) {
        const uint32_t slot = (uint32_t)(lane + 64 * k);
        if (slot < G) {
          const uint32_t q = __hip_atomic_load(&rec->part[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          mine = mine && (q & 0xFFFFu) == tag;
          const uint32_t v = q & 0xFFFF0000u;
          mx = mx > v ? mx : v;
        }
      }
      if (__all(mine)) break;
      if (++polls > limit) ok = 0;
      else __builtin_amdgcn_s_sleep(1);
    }
    mx = wave_max_u32(mx);
    if (lane == 0) {
      ok_sh = ok;
      amax_sh = mx;
    }
  }
  __syncthreads();
  const int ok = ok_sh;
  uint32_t amax = amax_sh;
  if (!ok) {
    // gave up: the maximum of the whole input, read by this workgroup alone
    uint32_t w = 0;
    for (uint32_t base = 0; base < nhalf; base += 8 * kRThreads) {
      uint4 t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)((base + u * kRThreads + threadIdx.x) * 16u),
                                                                0, 0);
        t[u] = make_uint4(q[0], q[1], q[2], q[3]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t a = uint4_absmax(t[u]);
        w = w > a ? w : a;
      }
    }
    amax = block_max_n<kRThreads>(w, sh) << 16;
    if (threadIdx.x == 0) atomicAdd(&g_rq_gave_up, 1u);
  }
  const float s_t = tensor_scale_from_amax(amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    rec->s_t = s_t;
    rec->amax_bits = amax;
    rec->nparts = 0;  // part[] holds tagged maxima, not partials a consumer may reduce
  }
  const GroupScaleTab tab = group_scale_tab<kRThreads>(s_t, recip);
  const __amdgpu_buffer_rsrc_t rc = rq_rsrc(codes, nhalf * 4u);
  const __amdgpu_buffer_rsrc_t rs = rq_rsrc(scales, nhalf / 2u);
  const bool even = (g0 & 1u) == 0;  // T is even: the same for all of the lane's half-groups
  // No branches on the range: past the input the loads read zeros and the
  // stores are dropped, and both lanes of every group meet at the swap of
  // their half maxima.
  auto run = [&](auto ovf_c) __attribute__((always_inline)) {
    constexpr bool OVF = decltype(ovf_c)::value;
    auto encode = [&](const uint4& t, uint32_t j) __attribute__((always_inline)) {
      const uint32_t w[4] = {t.x, t.y, t.z, t.w};
      uint32_t am = uint4_absmax(t);
      const uint32_t other = __shfl_xor(am, 1, 64);
      am = am > other ? am : other;
      float e;
      const uint32_t S = group_scale(am, tab, e);
      const uint32_t h = g0 + j * T;
      __builtin_amdgcn_raw_buffer_store_b32(encode8<OVF>(w, e), rc, (int)(h * 4u), 0, 0);
      if (even) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)S, rs, (int)(h / 2u), 0, 0);
    };
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j < J) encode(v[j], j);
    if constexpr (HOLD) {
#pragma unroll
      for (int k = 0; k < kRHeldLds; ++k)
        if (R + k < J) encode(*(const uint4*)(held_at(k) + lane * 16), R + k);
    } else {
      for (int j = R; j < J; ++j) encode(load(j), j);
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

// Lanes' shares of the input, in half-groups, for which the single launch
// pays (measured on MI355X against the amax pass + encode): from 17, where
// reading the input once outweighs the wait at the maximum (about 2.5 us),
// to the 48 kept in registers plus the 16 held in LDS.
constexpr int64_t kResidentMinJ = 17, kResidentMaxJ = 64;
static_assert(kResidentMaxJ <= kRMaxResident + kRHeldLds, "the longest share is held in registers and LDS");

static int resident_grid(const DeviceInfo& dev) { return dev.num_cu < kRThreads ? dev.num_cu : kRThreads; }

static int64_t resident_share(int64_t nelem, const DeviceInfo& dev) {
  const int64_t T = (int64_t)resident_grid(dev) * kRThreads;
  return (nelem / 8 + T - 1) / T;
}

bool quantize_resident_pays(int64_t nelem, const DeviceInfo& dev) {
  const int64_t J = resident_share(nelem, dev);
  return nelem < kResidentMaxElems && J >= kResidentMinJ && J <= kResidentMaxJ;
}

// One workgroup per CU (at most kRThreads of them, a grid that is the same
// for every call on the device) and R = 32 or 48 registers' worth of
// half-groups per lane, beyond 48 the rest (up to kResidentMaxJ) in LDS.
hipError_t launch_quantize_resident(const void* x_bf16, int64_t nelem, uint8_t* codes, uint8_t* scales,
                                    mq_scale_rec* rec, const DeviceInfo& dev, hipStream_t stream) {
  if (!quantize_resident_pays(nelem, dev)) return hipErrorInvalidValue;  // the caller checks first
  const int G = resident_grid(dev);
  const int64_t J = resident_share(nelem, dev);
  const int R = J <= 32 ? 32 : kRMaxResident;
  log_launch("quantize_resident_kernel", G, kRThreads, 0, "elements=%lld R=%d J=%lld", (long long)nelem, R,
             (long long)J);
  auto go = [&](auto kern, int lds) {
    hipLaunchKernelGGL(kern, dim3(G), dim3(kRThreads), lds, stream, (const uint4*)x_bf16, (uint32_t)(nelem / 8),
                       (int)J, (uint32_t*)codes, scales, rec);
  };
  if (R == 32) {
    go(quantize_resident_kernel<32, false>, 0);
  } else if (J <= kRMaxResident) {
    go(quantize_resident_kernel<kRMaxResident, false>, 0);
  } else {
    auto kern = quantize_resident_kernel<kRMaxResident, true>;
    constexpr int lds = kRHeldLds * kRThreads * 16;
    static bool attr_done[64] = {};  // benign race: the call is idempotent
    if (dev.device < 0 || dev.device >= 64 || !attr_done[dev.device]) {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      if (dev.device >= 0 && dev.device < 64) attr_done[dev.device] = true;
    }
    go(kern, lds);
  }
  return hipGetLastError();
}

uint32_t set_rq_spin_limit(uint32_t polls) {
  uint32_t old = 0;
  if (hipMemcpyFromSymbol(&old, HIP_SYMBOL(g_rq_spin_limit), sizeof(old)) != hipSuccess) return ~0u;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_rq_spin_limit), &polls, sizeof(polls)) != hipSuccess) return ~0u;
  return old;
}

uint32_t take_rq_gave_up() {
  uint32_t n = 0, zero = 0;
  if (hipMemcpyFromSymbol(&n, HIP_SYMBOL(g_rq_gave_up), sizeof(n)) != hipSuccess) return ~0u;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_rq_gave_up), &zero, sizeof(zero)) != hipSuccess) return ~0u;
  return n;
}

}  // namespace mq

