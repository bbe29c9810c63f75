// gemv.hip - BF16 decode GEMV / skinny GEMM, Y = X . W^T (gfx950).
//
// The decode linear of "Mix-Quant: Quantized Prefilling, Precise Decoding for
// Agentic LLMs" (gist.science English explainer, Technical Summary s.2:
// Hybrid Precision Strategy, Decoding; System-Level Deployment, decode
// workers) runs on the original BF16 weights.  With M <= 32 rows of X the
// work is bound by streaming W from HBM (2 bytes per weight, M flops/byte),
// so the kernel is organised around W's bytes:
//   - a workgroup owns 16 rows of W (32 at M > 16 when the grid still has
//     a workgroup per CU) and all of K; its four waves take the K chunks
//     (128 elements = 256 bytes per row) in turn;
//   - each wave has two LDS buffers, one chunk each: the chunk's W rows
//     and the matching X pieces (16 rows per column tile) arrive by
//     buffer_load ... lds, every instruction copying four rows of 256 bytes
//     (whole cache lines), one chunk ahead of use (W's copies non-temporal
//     when the grid fills the CUs, so that X stays in L2); rows past N or M read
//     zeros through the buffer resources (K is a multiple of the chunk; other
//     K take a register-path kernel);
//   - the wave reads the chunk back in MFMA layout (16-byte piece L of row r
//     sits at position L ^ (r & 15), so 16 rows hit distinct banks) and
//     feeds v_mfma_f32_16x16x32_bf16 with W rows as the 16-row operand and
//     X^T as the 16-column operand (up to two column tiles for M <= 32); all
//     reads of a chunk go out together and are waited for once; the MFMA is
//     used for its fp32 accumulation of exact bf16 products, not its rate;
//   - the K order inside a chunk is the same for W and X;
//   - the per-wave partial tiles are summed through LDS in a fixed order
//     (deterministic), rounded to bf16 (nearest-even) and stored;
//   - at M > 16 with rows shorter than 8192 a second kernel takes eight
//     waves and 64-element chunks (gemv_bf16_m32_kernel); rows of 8192 or
//     more start each workgroup's chunk walk at a chunk rotated by its row
//     group (both measured, see the kernels).
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

constexpr int kGvChunk = 128;                    // K elements per chunk
constexpr int64_t kGvRotateK = 8192;             // rows this long rotate their chunk walks
constexpr int kGvRowBytes = 2 * kGvChunk;        // bytes per row and chunk
constexpr int kGvWaves = 4;                      // waves per workgroup (split K)
constexpr int kGvTile = 16 * kGvRowBytes;        // 4 KB: 16 rows of one chunk
constexpr int kGvBufferWord3 = 0x00020000;       // raw buffer, 32-bit data format
typedef __attribute__((address_space(3))) void gv_lds_t;

// All pieces of one chunk that a lane needs, in one asm block that also waits
// for them: for q = 0..3 the W piece at a[q] and the MT X pieces one tile
// (4 KB) apart after it.  The outputs are early-clobber, so no read can land
// on an address still to be used.  Ordinary loads would not do: after the
// direct-to-LDS copies the compiler puts a vmcnt(0) before any LDS load,
// which would drain the prefetch at every chunk; the copies a chunk needs
// are waited for explicitly.
template <int MT>
__device__ __forceinline__ void lds_read_chunk(const uint32_t (&a)[4], uint4 (&wv)[4], uint4 (&xv)[4][MT]) {
  u32x4_t w0, w1, w2, w3, x0, x1, x2, x3;
  if constexpr (MT == 1) {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %4, %8 offset:4096\n\t"
        "ds_read_b128 %1, %9\n\tds_read_b128 %5, %9 offset:4096\n\t"
        "ds_read_b128 %2, %10\n\tds_read_b128 %6, %10 offset:4096\n\t"
        "ds_read_b128 %3, %11\n\tds_read_b128 %7, %11 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
    xv[0][0] = __builtin_bit_cast(uint4, x0);
    xv[1][0] = __builtin_bit_cast(uint4, x1);
    xv[2][0] = __builtin_bit_cast(uint4, x2);
    xv[3][0] = __builtin_bit_cast(uint4, x3);
  } else {
    u32x4_t y0, y1, y2, y3;
    asm volatile(
        "ds_read_b128 %0, %12\n\tds_read_b128 %4, %12 offset:4096\n\tds_read_b128 %8, %12 offset:8192\n\t"
        "ds_read_b128 %1, %13\n\tds_read_b128 %5, %13 offset:4096\n\tds_read_b128 %9, %13 offset:8192\n\t"
        "ds_read_b128 %2, %14\n\tds_read_b128 %6, %14 offset:4096\n\tds_read_b128 %10, %14 offset:8192\n\t"
        "ds_read_b128 %3, %15\n\tds_read_b128 %7, %15 offset:4096\n\tds_read_b128 %11, %15 offset:8192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(y0),
          "=&v"(y1), "=&v"(y2), "=&v"(y3)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
    xv[0][0] = __builtin_bit_cast(uint4, x0);
    xv[1][0] = __builtin_bit_cast(uint4, x1);
    xv[2][0] = __builtin_bit_cast(uint4, x2);
    xv[3][0] = __builtin_bit_cast(uint4, x3);
    xv[0][MT - 1] = __builtin_bit_cast(uint4, y0);
    xv[1][MT - 1] = __builtin_bit_cast(uint4, y1);
    xv[2][MT - 1] = __builtin_bit_cast(uint4, y2);
    xv[3][MT - 1] = __builtin_bit_cast(uint4, y3);
  }
  wv[0] = __builtin_bit_cast(uint4, w0);
  wv[1] = __builtin_bit_cast(uint4, w1);
  wv[2] = __builtin_bit_cast(uint4, w2);
  wv[3] = __builtin_bit_cast(uint4, w3);
}

// Two W tiles and two X tiles (32 W rows against 32 X rows): the pieces of
// W tile t at a[q] + 4096 t, of X tile u at a[q] + 4096 (2 + u).  One asm
// block with its wait, as above.
__device__ __forceinline__ void lds_read_chunk_w2(const uint32_t (&a)[4], uint4 (&wv)[2][4], uint4 (&xv)[4][2]) {
  u32x4_t w0, w1, w2, w3, v0, v1, v2, v3, x0, x1, x2, x3, y0, y1, y2, y3;
  asm volatile(
      "ds_read_b128 %0, %16\n\tds_read_b128 %4, %16 offset:4096\n\t"
      "ds_read_b128 %8, %16 offset:8192\n\tds_read_b128 %12, %16 offset:12288\n\t"
      "ds_read_b128 %1, %17\n\tds_read_b128 %5, %17 offset:4096\n\t"
      "ds_read_b128 %9, %17 offset:8192\n\tds_read_b128 %13, %17 offset:12288\n\t"
      "ds_read_b128 %2, %18\n\tds_read_b128 %6, %18 offset:4096\n\t"
      "ds_read_b128 %10, %18 offset:8192\n\tds_read_b128 %14, %18 offset:12288\n\t"
      "ds_read_b128 %3, %19\n\tds_read_b128 %7, %19 offset:4096\n\t"
      "ds_read_b128 %11, %19 offset:8192\n\tds_read_b128 %15, %19 offset:12288\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(x0),
        "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(y0), "=&v"(y1), "=&v"(y2), "=&v"(y3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
  wv[0][0] = __builtin_bit_cast(uint4, w0);
  wv[0][1] = __builtin_bit_cast(uint4, w1);
  wv[0][2] = __builtin_bit_cast(uint4, w2);
  wv[0][3] = __builtin_bit_cast(uint4, w3);
  wv[1][0] = __builtin_bit_cast(uint4, v0);
  wv[1][1] = __builtin_bit_cast(uint4, v1);
  wv[1][2] = __builtin_bit_cast(uint4, v2);
  wv[1][3] = __builtin_bit_cast(uint4, v3);
  xv[0][0] = __builtin_bit_cast(uint4, x0);
  xv[1][0] = __builtin_bit_cast(uint4, x1);
  xv[2][0] = __builtin_bit_cast(uint4, x2);
  xv[3][0] = __builtin_bit_cast(uint4, x3);
  xv[0][1] = __builtin_bit_cast(uint4, y0);
  xv[1][1] = __builtin_bit_cast(uint4, y1);
  xv[2][1] = __builtin_bit_cast(uint4, y2);
  xv[3][1] = __builtin_bit_cast(uint4, y3);
}

template <int MT, int WT>
constexpr int gv_lds_bytes() { return kGvWaves * 2 * (WT + MT) * kGvTile; }

// Up to MQ_MAX_GROUP weights that read the same X, in one launch: weight g
// owns the row tiles [tile_end[g-1], tile_end[g]) of the grid.
struct GvGroups {
  const uint16_t* w[MQ_MAX_GROUP];
  uint16_t* y[MQ_MAX_GROUP];
  int n[MQ_MAX_GROUP];
  int tile_end[MQ_MAX_GROUP];
  int ngroup;
};

// The weight of row tile `tile`, its output, row count and first tile,
// selected with constant indices (the arrays stay in the argument segment).
struct GvView {
  const uint16_t* w;
  uint16_t* y;
  int N, t0;
};
__device__ __forceinline__ GvView gv_group_of(const GvGroups& g, int tile) {
  GvView v{g.w[0], g.y[0], g.n[0], 0};
#pragma unroll
  for (int k = 1; k < MQ_MAX_GROUP; ++k)
    if (k < g.ngroup && tile >= g.tile_end[k - 1]) v = GvView{g.w[k], g.y[k], g.n[k], g.tile_end[k - 1]};
  return v;
}

// The row tile's weight: looked up (GROUPED), or the only one (a single
// call, which then reads no other group's fields).
template <bool GROUPED>
__device__ __forceinline__ GvView gv_view(const GvGroups& g, int tile) {
  if constexpr (GROUPED) return gv_group_of(g, tile);
  return GvView{g.w[0], g.y[0], g.n[0], 0};
}

// MT column tiles of X (16 rows each) against WT row tiles of W (16 rows
// each) per workgroup (WT = 2 only with MT = 2: at M > 16 two X tiles would
// otherwise take two thirds of the ring, and with it of the bytes in flight).
// NT: W's copies are non-temporal (W is read once; X stays in L2).
template <int MT, bool GROUPED, bool NT, int WT>
__global__ __launch_bounds__(kGvWaves * 64) void gemv_bf16_kernel(const uint16_t* __restrict__ x, GvGroups grp,
                                                                int M, int K, int rotate) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const GvView gv = gv_view<GROUPED>(grp, blockIdx.x);
  const uint16_t* __restrict__ w = gv.w;
  uint16_t* __restrict__ y = gv.y;
  const int N = gv.N;
  static_assert(WT == 1 || (WT == 2 && MT == 2), "tile combination");
  constexpr int kBufBytes = (WT + MT) * kGvTile;  // WT W tiles, then MT X tiles
  constexpr int kCopies = 4 * (WT + MT);          // copy instructions per chunk
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int i = lane & 15, h = lane >> 4;
  const int n0 = (blockIdx.x - gv.t0) * 16 * WT;
  // the host guarantees 32 * K * 2 < 2^31
  const uint16_t* wtile = w + (int64_t)n0 * K;
  const int wbytes = min(16 * WT, N - n0) * K * 2, xbytes = M * K * 2;
  // copy j of a chunk covers rows 4(j%4) .. +3 of tile j/4 (W, then the X
  // column tiles); lane l: row
  // r = 4(j%4) + l/16, LDS piece l%16 holds logical piece (l%16) ^ r, i.e.
  // K elements k0 + 8((l%16) ^ r) .. +7.  K is a multiple of the chunk, so no
  // piece lies past K.
  uint32_t off[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int r = 4 * (j % 4) + (lane >> 4), tile = j / 4;
    const int row = tile < WT ? 16 * tile + r : 16 * (tile - WT) + r;  // row of W or of X
    off[j] = (uint32_t)(row * K + 8 * ((lane & 15) ^ r)) * 2u;
  }
  uint8_t* ring = lds + wave * 2 * kBufBytes;
  const int nchunks = (K + kGvChunk - 1) / kGvChunk;
  const int mine = nchunks > wave ? (nchunks - wave + kGvWaves - 1) / kGvWaves : 0;  // this wave's chunks
  // This wave's t-th chunk into buffer dst.  Past the share the resources
  // cover no bytes (zeros, no memory traffic).
  // With `rotate` (long rows, K >= 8192) workgroups start their chunk walks
  // at different chunks, rotated by the 32-row group of W (so grouped and
  // single calls, and 16- and 32-row workgroups, sum every output in the
  // same order): measured 4-9% faster for 4096 x 14336, while for K = 4096
  // rows walking in step is 15-40% faster.
  const int rot = rotate && mine > 0 ? (n0 >> 5) % mine : 0;
  auto copy = [&](int t, uint8_t* dst) __attribute__((always_inline)) {
    const bool live = t < mine;
    int tr = t + rot;
    tr = tr < mine ? tr : tr - mine;
    const int k0 = (wave + kGvWaves * tr) * kGvChunk;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)wtile, 0, live ? wbytes : 0, kGvBufferWord3);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, live ? xbytes : 0, kGvBufferWord3);
    constexpr int kAuxW = NT ? 2 : 0;  // cache policy of W's copies: nt
#pragma unroll
    for (int j = 0; j < 4 * WT; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (gv_lds_t*)(dst + 1024 * j), 16, (int)off[j],
                                               live ? k0 * 2 : 0, 0, kAuxW);
#pragma unroll
    for (int j = 4 * WT; j < kCopies; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (gv_lds_t*)(dst + 1024 * j), 16, (int)off[j],
                                               live ? k0 * 2 : 0, 0, 0);
  };

  f32x4_t acc[WT][MT];
#pragma unroll
  for (int t = 0; t < WT; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Copies run one chunk ahead through two buffers that alternate; before
  // chunk t is read, every copy but the next chunk's must have landed (vmcnt
  // counts in issue order).  The buffer refilled at step t was read at step
  // t - 1, and those reads completed inside their asm block.  Chunks past
  // this wave's share compute on zeros.
  uint8_t* cur = ring;
  uint8_t* nxt = ring + kBufBytes;
  copy(0, cur);
  constexpr int kWait = kCopies;
  static_assert(kWait < 64, "vmcnt range");
  for (int t = 0; t < mine; ++t) {
    copy(t + 1, nxt);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (kWait & 15) | ((kWait >> 4) << 14));  // vmcnt(kWait)
    uint32_t ad[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ad[q] = (uint32_t)(uintptr_t)(cur + i * kGvRowBytes + (((4 * q + h) ^ i) << 4));
    uint4 wv[WT][4], xv[4][MT];
    if constexpr (WT == 1)
      lds_read_chunk<MT>(ad, wv[0], xv);
    else
      lds_read_chunk_w2(ad, wv, xv);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < WT; ++t)
#pragma unroll
        for (int u = 0; u < MT; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[t][q]),
                                                             __builtin_bit_cast(bf16x8_t, xv[q][u]), acc[t][u], 0,
                                                             0, 0);
    uint8_t* done = cur;
    cur = nxt;
    nxt = done;
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): no copy still writes the ring
  __syncthreads();
  constexpr int kPairs = WT * MT;
  f32x4_t* red = (f32x4_t*)lds;  // [wave][WT * MT][64]
#pragma unroll
  for (int t = 0; t < WT; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) red[(wave * kPairs + t * MT + u) * 64 + lane] = acc[t][u];
  __syncthreads();
  // wave p finishes W tile p / MT against X tile p % MT
  if (wave < kPairs) {
    const int t = wave / MT, u = wave % MT;
    f32x4_t s = red[wave * 64 + lane];
    for (int v = 1; v < kGvWaves; ++v) s += red[(v * kPairs + wave) * 64 + lane];
    const int m = (lane & 15) + 16 * u;
    if (m < M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 16 * t + 4 * (lane >> 4) + r;
        if (n < N) {
          uint32_t b = __float_as_uint(s[r]);
          y[(int64_t)m * N + n] = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
        }
      }
    }
  }
}

// M > 16 with rows shorter than kGvRotateK: eight waves per workgroup and
// 64-element chunks (one 128-byte line per row and chunk) instead of four
// waves and 128-element chunks, so that the two X column tiles do not halve
// the waves a CU holds: the same bytes in flight per CU, spread over twice
// the waves (measured 3-10% faster for 4096 x 4096 and 14336 x 4096 at M =
// 17..32; 2-3% slower for 4096 x 14336, which keeps the other kernel).  A chunk's pieces are
// two K steps of 32 for each W and X tile, read back in one asm block with
// its wait (see lds_read_chunk).  Piece p of row r sits at 16-byte position
// p ^ ((r >> 1) & 7): 16 rows of 128 bytes then hit distinct banks.
constexpr int kGv2Chunk = 64;
constexpr int kGv2RowBytes = 2 * kGv2Chunk;     // 128
constexpr int kGv2Tile = 16 * kGv2RowBytes;     // 2 KB
constexpr int kGv2Waves = 8;

template <int NTILE>
__device__ __forceinline__ void lds_read_chunk64(const uint32_t (&a)[2], u32x4_t (&v)[2][NTILE]) {
  static_assert(NTILE == 3 || NTILE == 4 || NTILE == 6, "tiles per chunk");
  if constexpr (NTILE == 3) {
    u32x4_t a0, a1, a2, b0, b1, b2;
    asm volatile(
        "ds_read_b128 %0, %6\n\tds_read_b128 %1, %6 offset:2048\n\tds_read_b128 %2, %6 offset:4096\n\t"
        "ds_read_b128 %3, %7\n\tds_read_b128 %4, %7 offset:2048\n\tds_read_b128 %5, %7 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(b0), "=&v"(b1), "=&v"(b2)
        : "v"(a[0]), "v"(a[1])
        : "memory");
    v[0][0] = a0; v[0][1] = a1; v[0][2] = a2;
    v[1][0] = b0; v[1][1] = b1; v[1][2] = b2;
  } else if constexpr (NTILE == 4) {
    u32x4_t a0, a1, a2, a3, b0, b1, b2, b3;
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:2048\n\t"
        "ds_read_b128 %2, %8 offset:4096\n\tds_read_b128 %3, %8 offset:6144\n\t"
        "ds_read_b128 %4, %9\n\tds_read_b128 %5, %9 offset:2048\n\t"
        "ds_read_b128 %6, %9 offset:4096\n\tds_read_b128 %7, %9 offset:6144\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
        : "v"(a[0]), "v"(a[1])
        : "memory");
    v[0][0] = a0; v[0][1] = a1; v[0][2] = a2; v[0][3] = a3;
    v[1][0] = b0; v[1][1] = b1; v[1][2] = b2; v[1][3] = b3;
  } else {
    u32x4_t a0, a1, a2, a3, a4, a5, b0, b1, b2, b3, b4, b5;
    asm volatile(
        "ds_read_b128 %0, %12\n\tds_read_b128 %1, %12 offset:2048\n\tds_read_b128 %2, %12 offset:4096\n\t"
        "ds_read_b128 %3, %12 offset:6144\n\tds_read_b128 %4, %12 offset:8192\n\tds_read_b128 %5, %12 offset:10240\n\t"
        "ds_read_b128 %6, %13\n\tds_read_b128 %7, %13 offset:2048\n\tds_read_b128 %8, %13 offset:4096\n\t"
        "ds_read_b128 %9, %13 offset:6144\n\tds_read_b128 %10, %13 offset:8192\n\tds_read_b128 %11, %13 offset:10240\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(a4), "=&v"(a5), "=&v"(b0), "=&v"(b1), "=&v"(b2),
          "=&v"(b3), "=&v"(b4), "=&v"(b5)
        : "v"(a[0]), "v"(a[1])
        : "memory");
    v[0][0] = a0; v[0][1] = a1; v[0][2] = a2; v[0][3] = a3; v[0][4] = a4; v[0][5] = a5;
    v[1][0] = b0; v[1][1] = b1; v[1][2] = b2; v[1][3] = b3; v[1][4] = b4; v[1][5] = b5;
  }
}

template <int WT, int NW>
constexpr int gv2_lds_bytes() { return NW * 2 * (WT + 2) * kGv2Tile; }

template <bool GROUPED, bool NT, int WT, int NW = kGv2Waves>
__global__ __launch_bounds__(NW * 64) void gemv_bf16_m32_kernel(const uint16_t* __restrict__ x,
                                                                     GvGroups grp, int M, int K, int rotate) {
  constexpr int MT = 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const GvView gv = gv_view<GROUPED>(grp, blockIdx.x);
  const uint16_t* __restrict__ w = gv.w;
  uint16_t* __restrict__ y = gv.y;
  const int N = gv.N;
  constexpr int NTILE = WT + MT;
  constexpr int kBufBytes = NTILE * kGv2Tile;   // WT W tiles, then MT X tiles
  constexpr int kCopies = 2 * NTILE;            // copy instructions per chunk (8 rows each)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int i = lane & 15, h = lane >> 4;
  const int n0 = (blockIdx.x - gv.t0) * 16 * WT;
  // the host guarantees 32 * K * 2 < 2^31
  const uint16_t* wtile = w + (int64_t)n0 * K;
  const int wbytes = min(16 * WT, N - n0) * K * 2, xbytes = M * K * 2;
  // copy j of a chunk covers rows 8(j%2) .. +7 of tile j/2 (W, then the X
  // column tiles); lane l: row r = 8(j%2) + l/8, LDS position l%8 holds
  // logical piece (l%8) ^ ((r >> 1) & 7), i.e. K elements k0 + 8 * that .. +7
  uint32_t off[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int r = 8 * (j % 2) + (lane >> 3), tile = j / 2;
    const int row = tile < WT ? 16 * tile + r : 16 * (tile - WT) + r;  // row of W or of X
    off[j] = (uint32_t)(row * K + 8 * ((lane & 7) ^ ((r >> 1) & 7))) * 2u;
  }
  uint8_t* ring = lds + wave * 2 * kBufBytes;
  const int nchunks = K / kGv2Chunk;
  const int mine = nchunks > wave ? (nchunks - wave + NW - 1) / NW : 0;
  // NW < kGv2Waves: each wave stands for VW of the kGv2Waves waves of the
  // other form (its chunks alternate between them, each with its own
  // accumulators), and the partial sums are added in that form's order, so
  // every output is bit-identical to it (no chunk rotation in this form)
  constexpr int VW = kGv2Waves / NW;
  static_assert(VW * NW == kGv2Waves, "waves");
  const int rot = VW == 1 && rotate && mine > 0 ? (n0 >> 5) % mine : 0;  // as in gemv_bf16_kernel
  auto copy = [&](int t, uint8_t* dst) __attribute__((always_inline)) {
    const bool live = t < mine;
    int tr = t + rot;
    tr = tr < mine ? tr : tr - mine;
    const int k0 = (wave + NW * tr) * kGv2Chunk;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)wtile, 0, live ? wbytes : 0, kGvBufferWord3);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, live ? xbytes : 0, kGvBufferWord3);
    constexpr int kAuxW = NT ? 2 : 0;  // cache policy of W's copies: nt
#pragma unroll
    for (int j = 0; j < 2 * WT; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (gv_lds_t*)(dst + 1024 * j), 16, (int)off[j],
                                               live ? k0 * 2 : 0, 0, kAuxW);
#pragma unroll
    for (int j = 2 * WT; j < kCopies; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (gv_lds_t*)(dst + 1024 * j), 16, (int)off[j],
                                               live ? k0 * 2 : 0, 0, 0);
  };

  f32x4_t acc[VW][WT][MT];
#pragma unroll
  for (int s = 0; s < VW; ++s)
#pragma unroll
    for (int t = 0; t < WT; ++t)
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[s][t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one chunk ahead through two alternating buffers, as gemv_bf16_kernel
  uint8_t* cur = ring;
  uint8_t* nxt = ring + kBufBytes;
  copy(0, cur);
  constexpr int kWait = kCopies;
  static_assert(kWait < 64, "vmcnt range");
  for (int t0 = 0; t0 < mine; t0 += VW) {
#pragma unroll
    for (int s = 0; s < VW; ++s) {
      const int t = t0 + s;
      if (VW > 1 && t >= mine) break;  // the same for the whole wave
      copy(t + 1, nxt);
      __builtin_amdgcn_s_waitcnt(0x0F70 | (kWait & 15) | ((kWait >> 4) << 14));  // vmcnt(kWait)
      uint32_t ad[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
        ad[q] = (uint32_t)(uintptr_t)(cur + i * kGv2RowBytes + (((4 * q + h) ^ ((i >> 1) & 7)) << 4));
      u32x4_t v[2][NTILE];
      lds_read_chunk64<NTILE>(ad, v);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int tt = 0; tt < WT; ++tt)
#pragma unroll
          for (int u = 0; u < MT; ++u)
            acc[s][tt][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v[q][tt]),
                                                                   __builtin_bit_cast(bf16x8_t, v[q][WT + u]),
                                                                   acc[s][tt][u], 0, 0, 0);
      uint8_t* done = cur;
      cur = nxt;
      nxt = done;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): no copy still writes the ring
  __syncthreads();
  constexpr int kPairs = WT * MT;
  f32x4_t* red = (f32x4_t*)lds;  // [wave of the eight-wave form][WT * MT][64]
  static_assert(kGv2Waves * kPairs * 64 * 16 <= gv2_lds_bytes<WT, NW>(), "reduction fits the ring");
#pragma unroll
  for (int s = 0; s < VW; ++s)
#pragma unroll
    for (int t = 0; t < WT; ++t)
#pragma unroll
      for (int u = 0; u < MT; ++u) red[((wave + NW * s) * kPairs + t * MT + u) * 64 + lane] = acc[s][t][u];
  __syncthreads();
  // wave p finishes W tile p / MT against X tile p % MT (p = wave, wave + NW, ...)
  for (int p = wave; p < kPairs; p += NW) {
    const int t = p / MT, u = p % MT;
    f32x4_t sum = red[p * 64 + lane];
    for (int v2 = 1; v2 < kGv2Waves; ++v2) sum += red[(v2 * kPairs + p) * 64 + lane];
    const int m = (lane & 15) + 16 * u;
    if (m < M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 16 * t + 4 * (lane >> 4) + r;
        if (n < N) {
          uint32_t b = __float_as_uint(sum[r]);
          y[(int64_t)m * N + n] = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
        }
      }
    }
  }
}

// Ragged K (K % 128 != 0): 16 W rows per workgroup, up to kGvMaxWaves waves
// splitting K, loads straight into registers (the four lanes of a row read 64
// contiguous bytes per instruction), every piece bounds-checked.
constexpr int kGvMaxWaves = 16;

template <int MT, bool GROUPED>
__global__ __launch_bounds__(kGvMaxWaves * 64) void gemv_bf16_ragged_kernel(const uint16_t* __restrict__ x,
                                                                   GvGroups grp, int M, int K) {
  __shared__ f32x4_t red[kGvMaxWaves][MT][64];
  const GvView gv = gv_view<GROUPED>(grp, blockIdx.x);
  const uint16_t* __restrict__ w = gv.w;
  uint16_t* __restrict__ y = gv.y;
  const int N = gv.N;
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, h = lane >> 4;
  const int n0 = (blockIdx.x - gv.t0) * 16;
  int nrow = n0 + i;
  nrow = nrow < N ? nrow : N - 1;
  const uint16_t* wrow = w + (int64_t)nrow * K + 8 * h;
  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = i + 16 * t;
    xok[t] = m < M;
    xrow[t] = x + (int64_t)(xok[t] ? m : 0) * K + 8 * h;
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
        const bool in = k0 + 8 * h + 32 * q < K;
        wv[u][q] = in ? ld_stream(wrow + k0 + 32 * q) : zero;
#pragma unroll
        for (int t = 0; t < MT; ++t)
          xv[u][t][q] = (in && xok[t]) ? *(const uint4*)(xrow[t] + k0 + 32 * q) : zero;
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
      const bool in = k0 + 8 * h + 32 * q < K;
      uint4 wq = in ? ld_stream(wrow + k0 + 32 * q) : zero;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        uint4 xq = (in && xok[t]) ? *(const uint4*)(xrow[t] + k0 + 32 * q) : zero;
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

template <int MT, bool GROUPED, bool NT, int WT>
static hipError_t launch_ring(const void* x, const GvGroups& g, int tiles, int64_t M, int64_t K, int dev,
                              hipStream_t stream) {
  auto kern = gemv_bf16_kernel<MT, GROUPED, NT, WT>;
  constexpr int lds = gv_lds_bytes<MT, WT>();
  static bool attr_done[64] = {};  // benign race: the call is idempotent
  if (dev < 0 || dev >= 64 || !attr_done[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_done[dev] = true;
  }
  log_launch("gemv_bf16_kernel", tiles, kGvWaves * 64, lds,
             "column_tiles=%d row_tiles=%d grouped=%d nt=%d M=%lld K=%lld groups=%d", MT, WT, (int)GROUPED, (int)NT,
             (long long)M, (long long)K, g.ngroup);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kGvWaves * 64), lds, stream, (const uint16_t*)x, g, (int)M,
                     (int)K, K >= kGvRotateK ? 1 : 0);
  return hipGetLastError();
}

// W's copies are non-temporal when the grid fills the CUs: measured 4-11%
// faster on such bandwidth-bound grids (e.g. 4096 x 14336 at M=1: 23.2 ->
// 20.9 us), but 15-30% slower on the 64-workgroup 1024 x 4096 one.
template <int MT, bool GROUPED, int WT = 1>
static hipError_t launch_ring_nt(const void* x, const GvGroups& g, int tiles, int64_t M, int64_t K,
                                 const DeviceInfo& dev, hipStream_t stream) {
  return tiles >= dev.num_cu ? launch_ring<MT, GROUPED, true, WT>(x, g, tiles, M, K, dev.device, stream)
                             : launch_ring<MT, GROUPED, false, WT>(x, g, tiles, M, K, dev.device, stream);
}

template <bool GROUPED, bool NT, int WT, int NW = kGv2Waves>
static hipError_t launch_m32(const void* x, const GvGroups& g, int tiles, int64_t M, int64_t K, int dev,
                             hipStream_t stream) {
  auto kern = gemv_bf16_m32_kernel<GROUPED, NT, WT, NW>;
  constexpr int lds = gv2_lds_bytes<WT, NW>();
  static bool attr_done[64] = {};  // benign race: the call is idempotent
  if (dev < 0 || dev >= 64 || !attr_done[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_done[dev] = true;
  }
  log_launch("gemv_bf16_m32_kernel", tiles, NW * 64, lds,
             "row_tiles=%d grouped=%d nt=%d M=%lld K=%lld groups=%d", WT, (int)GROUPED, (int)NT, (long long)M,
             (long long)K, g.ngroup);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(NW * 64), lds, stream, (const uint16_t*)x, g, (int)M,
                     (int)K, K >= kGvRotateK ? 1 : 0);
  return hipGetLastError();
}
template <bool GROUPED, int WT, int NW = kGv2Waves>
static hipError_t launch_m32_nt(const void* x, const GvGroups& g, int tiles, int64_t M, int64_t K,
                                const DeviceInfo& dev, hipStream_t stream) {
  return tiles >= dev.num_cu ? launch_m32<GROUPED, true, WT, NW>(x, g, tiles, M, K, dev.device, stream)
                             : launch_m32<GROUPED, false, WT, NW>(x, g, tiles, M, K, dev.device, stream);
}

template <bool GROUPED>
static hipError_t launch_ragged(const void* x, const GvGroups& g, int tiles, int64_t M, int64_t K,
                                const DeviceInfo& dev, hipStream_t stream) {
  const int nchunks = (int)((K + kGvChunk - 1) / kGvChunk);
  // aim for about eight waves per CU over the whole grid
  int nw = (8 * dev.num_cu + tiles - 1) / tiles;
  nw = nw < 4 ? 4 : nw;
  nw = nw > kGvMaxWaves ? kGvMaxWaves : nw;
  nw = nw > nchunks ? (nchunks < 1 ? 1 : nchunks) : nw;
  log_launch("gemv_bf16_ragged_kernel", tiles, nw * 64, 0, "grouped=%d M=%lld K=%lld groups=%d", (int)GROUPED,
             (long long)M, (long long)K, g.ngroup);
  if (M <= 16) {
    hipLaunchKernelGGL((gemv_bf16_ragged_kernel<1, GROUPED>), dim3(tiles), dim3(nw * 64), 0, stream, (const uint16_t*)x, g,
                       (int)M, (int)K);
  } else {
    hipLaunchKernelGGL((gemv_bf16_ragged_kernel<2, GROUPED>), dim3(tiles), dim3(nw * 64), 0, stream, (const uint16_t*)x, g,
                       (int)M, (int)K);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const void* x, const GemvWeight* w, int ngroup, int64_t M, int64_t K,
                               const DeviceInfo& dev, hipStream_t stream) {
  // the ring kernel needs whole chunks and buffer offsets of 32 rows below 2^31
  const bool ring = K % kGvChunk == 0 && K < (int64_t(1) << 25);
  // At M > 16 a workgroup takes 32 W rows when that still leaves a workgroup
  // for every CU: twice the W bytes in flight per CU, half the X bytes per W
  // byte.  Smaller grids keep 16 rows (more workgroups).
  int64_t rows = 0, rows64 = 0;
  for (int k = 0; k < ngroup; ++k) {
    rows += (w[k].n + 31) / 32;
    rows64 += (w[k].n + 63) / 64;
  }
  int wt = ring && M > 16 && rows >= dev.num_cu ? 2 : 1;
  // wide weights at M > 16 and K below the rotation length: 64 W rows per
  // four-wave workgroup, X read once per 64 W rows
  if (ring && M > 16 && K < kGvRotateK && rows64 * 4 >= (int64_t)dev.num_cu * 3) wt = 4;
  GvGroups g{};
  int tiles = 0;
  for (int k = 0; k < ngroup; ++k) {
    g.w[k] = (const uint16_t*)w[k].w;
    g.y[k] = (uint16_t*)w[k].y;
    g.n[k] = (int)w[k].n;
    tiles += (int)((w[k].n + 16 * wt - 1) / (16 * wt));
    g.tile_end[k] = tiles;
  }
  g.ngroup = ngroup;
  if (ngroup == 1) {
    if (!ring) return launch_ragged<false>(x, g, tiles, M, K, dev, stream);
    if (M <= 16) return launch_ring_nt<1, false>(x, g, tiles, M, K, dev, stream);
    if (K < kGvRotateK) return wt == 4   ? launch_m32_nt<false, 4, 4>(x, g, tiles, M, K, dev, stream)
                               : wt == 2 ? launch_m32_nt<false, 2>(x, g, tiles, M, K, dev, stream)
                                         : launch_m32_nt<false, 1>(x, g, tiles, M, K, dev, stream);
    return wt == 2 ? launch_ring_nt<2, false, 2>(x, g, tiles, M, K, dev, stream)
                   : launch_ring_nt<2, false>(x, g, tiles, M, K, dev, stream);
  }
  if (!ring) return launch_ragged<true>(x, g, tiles, M, K, dev, stream);
  if (M <= 16) return launch_ring_nt<1, true>(x, g, tiles, M, K, dev, stream);
  if (K < kGvRotateK) return wt == 4   ? launch_m32_nt<true, 4, 4>(x, g, tiles, M, K, dev, stream)
                             : wt == 2 ? launch_m32_nt<true, 2>(x, g, tiles, M, K, dev, stream)
                                       : launch_m32_nt<true, 1>(x, g, tiles, M, K, dev, stream);
  return wt == 2 ? launch_ring_nt<2, true, 2>(x, g, tiles, M, K, dev, stream)
                 : launch_ring_nt<2, true>(x, g, tiles, M, K, dev, stream);
}

hipError_t launch_gemv(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                       const DeviceInfo& dev, hipStream_t stream) {
  const GemvWeight one{w, y, N};
  return launch_gemv_grouped(x, &one, 1, M, K, dev, stream);
}

}  // namespace mq
