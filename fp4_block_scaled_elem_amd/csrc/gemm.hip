// gemm.hip - NVFP4 x NVFP4 prefill GEMM, C = A . W^T (gfx950).
//
// The W4A4 prefill linear of "Mix-Quant: Quantized Prefilling, Precise
// Decoding for Agentic LLMs" (gist.science English explainer, Technical
// Summary s.2, System-Level Deployment: prefill workers run weights and
// activations in NVFP4).
//
// Contraction scheme.  gfx950's block-scaled MFMA takes power-of-two (E8M0)
// scales per 32 elements; NVFP4 has E4M3 scales per 16, so it cannot be fed
// to that instruction exactly.  Instead each operand element is dequantized
// to g * sigma (an E2M1 magnitude times the group's E4M3 scale): at most
// 2 + 4 significant bits, between 2^-10 and 2688, hence an exact normal
// binary16.  The products are then exact in the binary32 accumulator of
// v_mfma_f32_32x32x16_f16, and the two tensor scales are applied once in the
// epilogue.  The result equals the float64 product of the dequantized
// operands up to binary32 accumulation and the final bf16 rounding.
//
// Data flow per workgroup (256 threads = 4 waves in a 2x2 grid, one wave per
// SIMD; tile BM x BN; K advanced 128 elements = 8 groups per stage):
//   HBM --direct-to-LDS loads (no registers)--> LDS ring of four stages
//   (packed codes + scale bytes); the fused prologue and shapes with
//   K % 128 != 0 go through registers instead
//   LDS --16-byte reads--> registers: four dwords = codes of four K16 steps
//   cvt fp4->f16 (hardware) * sigma (packed f16 multiply) -> MFMA operand.
// Every wave runs a register pipeline: the operands of step s+1 are
// dequantized while the MFMAs of step s run, and the next stage's codes,
// scales and first operands are prepared inside the current stage, so the
// MFMA stream only pauses at the one barrier per stage.  The K order inside
// a stage is permuted identically for A and W (the sum is unchanged).
#include <atomic>

#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

constexpr int kThreads = 256;
constexpr int kBK = 128;            // K elements per stage
constexpr int kRowBytes = kBK / 2;  // packed code bytes per row per stage
// An LDS ring slot holds two consecutive stages (a "double stage", 256 K
// elements): per row 128 bytes of codes (one full cache line of the row-major
// operand) and 16 bytes of scales, so the direct-to-LDS copies fetch whole
// lines.
constexpr int kRowStride = 2 * kRowBytes;  // 128: LDS bytes per code row of a slot
constexpr int kScaleStride = 16;           // LDS bytes per scale row of a slot

// Code rows in LDS hold eight 16-byte chunks (chunk 4p + c = chunk c of the
// slot's stage p), chunk L of row r at position L ^ swz(r).  Two 128-byte rows
// span the banks; the swizzle spreads rows r, r+2, ..., r+14 over all eight
// positions, which a probe measured free of SQ_LDS_BANK_CONFLICT for the
// pipe's 16-byte reads of 32 rows.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// One launch computes C_g = A . W_g^T for up to kMaxGroup weights sharing A;
// the column tiles of the groups follow each other (group g owns column
// tiles [tn_end[g-1], tn_end[g])).
constexpr int kMaxGroup = MQ_MAX_GROUP;

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const void* a_bf16;        // fused mode only
  mq_scale_rec* a_rec;
  const uint8_t* w_codes[kMaxGroup];
  const uint8_t* w_scales[kMaxGroup];
  const mq_scale_rec* w_rec[kMaxGroup];
  void* c[kMaxGroup];
  int n[kMaxGroup];
  int tn_end[kMaxGroup];
  int ngroup;
  int M, K;
  int tiles_m, tiles_n;      // tiles_n: all groups
  int a_given;               // fused mode: take s_t from a_rec
  int a_inline;              // fused mode, small A: every workgroup takes max|A| itself
};

// The group of column tile tn and its operands, selected with constant
// indices only (the argument arrays stay in the kernel-argument segment).
struct GroupView {
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const mq_scale_rec* w_rec;
  void* c;
  int N, tn0;
};

__device__ __forceinline__ GroupView group_of(const GemmArgs& a, int tn) {
  GroupView v{a.w_codes[0], a.w_scales[0], a.w_rec[0], a.c[0], a.n[0], 0};
#pragma unroll
  for (int g = 1; g < kMaxGroup; ++g) {
    if (g < a.ngroup && tn >= a.tn_end[g - 1]) {
      v = GroupView{a.w_codes[g], a.w_scales[g], a.w_rec[g], a.c[g], a.n[g], a.tn_end[g - 1]};
    }
  }
  return v;
}

template <int BM, int BN>
struct Smem {
  static constexpr int kA = 0;
  static constexpr int kW = kA + BM * kRowStride;
  static constexpr int kAs = kW + BN * kRowStride;
  static constexpr int kWs = kAs + BM * kScaleStride;
  static constexpr int kSlot = kWs + BN * kScaleStride;
  static constexpr int kTotal = 2 * kSlot;  // two slots = four stages
};


// ---------------------------------------------------------------- loaders --

// Packed operand (A or W) rows [r0, r0+ROWS) x stage kt into registers.
template <int ROWS, bool FAST>
struct PackedLoader {
  static constexpr int kChunks = ROWS * 4 / kThreads;  // 16-byte pieces per thread
  u32x4_t code[kChunks > 0 ? kChunks : 1];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes, int r0, int nrows, int K, int kt) {
    const int tid = threadIdx.x;
    const int64_t ldc = K / 2;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = tid + kThreads * j;
      const int row = c >> 2, col = c & 3;
      int r = r0 + row;
      r = r < nrows ? r : nrows - 1;  // clamped rows are computed and discarded
      const uint8_t* p = codes + (int64_t)r * ldc + (int64_t)kt * kRowBytes + col * 16;
      if (FAST) {
        code[j] = *(const u32x4_t*)p;
      } else {
        // K % 16 == 0 only: rows are 8-byte aligned; load each group alone
        const int e0 = kt * kBK + col * 32;
        u32x2_t lo = {0u, 0u}, hi = {0u, 0u};
        if (e0 < K) lo = *(const u32x2_t*)p;
        if (e0 + 16 < K) hi = *(const u32x2_t*)(p + 8);
        code[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
    }
  }
  // into stage half p of a slot's code rows
  __device__ __forceinline__ void store(uint8_t* lds, int p) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = tid + kThreads * j;
      const int row = c >> 2, col = c & 3;
      *(u32x4_t*)(lds + row * kRowStride + (((4 * p + col) ^ swz(row)) << 4)) = code[j];
    }
  }
};

// Scale bytes for A rows then W rows (BM + BN rows of 8 bytes per stage);
// with WITH_A false (fused prologue) only the W rows.
template <int BM, int BN, bool FAST, bool WITH_A>
struct ScaleLoader {
  static constexpr int kA = WITH_A ? BM : 0;
  static constexpr int kRows = kA + BN;
  static constexpr int kPer = (kRows + kThreads - 1) / kThreads;
  static constexpr bool kFull = kRows % kThreads == 0;
  u32x2_t v[kPer];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ as, const uint8_t* __restrict__ ws,
                                       int m0, int n0, int M, int N, int K, int kt) {
    const int ng = K / kGroup;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int r = threadIdx.x + kThreads * j;
      v[j] = u32x2_t{0u, 0u};
      if (kFull || r < kRows) {
        const uint8_t* base;
        int row;
        if (r < kA) { row = m0 + r; row = row < M ? row : M - 1; base = as; }
        else        { row = n0 + r - kA; row = row < N ? row : N - 1; base = ws; }
        const uint8_t* p = base + (int64_t)row * ng + kt * 8;
        if (FAST) {
          v[j] = *(const u32x2_t*)p;
        } else {
          uint32_t b[8];
#pragma unroll
          for (int g = 0; g < 8; ++g) b[g] = (kt * 8 + g < ng) ? p[g] : 0u;
          v[j] = u32x2_t{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                         b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
        }
      }
    }
  }
  // into stage half h of a slot's scale rows
  __device__ __forceinline__ void store(uint8_t* slot, int h) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int r = threadIdx.x + kThreads * j;
      if (kFull || r < kRows) {
        uint8_t* p = r < kA ? slot + Smem<BM, BN>::kAs + r * kScaleStride
                            : slot + Smem<BM, BN>::kWs + (r - kA) * kScaleStride;
        *(u32x2_t*)(p + 8 * h) = v[j];
      }
    }
  }
};

// bf16 activations quantized on the fly (fused prologue): BM rows x 128
// elements per stage = BM*8 groups, each thread owning whole groups.  The
// arithmetic is quantize_group16, bit-identical to the standalone quantizer.
// Tiles of more than 128 rows take a stage in kParts parts (loaded and
// quantized at different pipeline steps) so that at most two groups of raw
// bf16 data per thread are held in registers.
template <int BM, bool FAST>
struct FusedALoader {
  static constexpr int kGroupsAll = BM * 8 / kThreads;
  static constexpr int kParts = kGroupsAll > 4 ? kGroupsAll / 2 : 1;
  static constexpr int kGroupsPer = kGroupsAll / kParts;
  u32x4_t raw[kGroupsPer][2];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ a, int m0, int M, int K, int kt, int part) {
#pragma unroll
    for (int j = 0; j < kGroupsPer; ++j) {
      const int gi = threadIdx.x + kThreads * (part * kGroupsPer + j);
      const int row = gi >> 3, grp = gi & 7;
      int r = m0 + row;
      r = r < M ? r : M - 1;
      const int e0 = kt * kBK + grp * kGroup;
      const uint16_t* p = a + (int64_t)r * K + e0;
      if (FAST || e0 < K) {
        raw[j][0] = *(const u32x4_t*)p;
        raw[j][1] = *(const u32x4_t*)(p + 8);
      } else {
        raw[j][0] = u32x4_t{0u, 0u, 0u, 0u};
        raw[j][1] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  // Quantize the loaded groups into stage half p of a slot's A codes and
  // scale bytes.  STORE_G: also into A's NVFP4 in global memory (standard
  // layout) when the stage kt exists (kt < nk) and the row is inside A.
  template <int BN, bool OVF, bool STORE_G = false>
  __device__ __forceinline__ void quantize_store(uint8_t* stage, int p, const GroupScaleTab& tab, int part,
                                                 uint8_t* gcodes = nullptr, uint8_t* gscales = nullptr, int m0 = 0,
                                                 int M = 0, int K = 0, int kt = 0, int nk = 0) const {
#pragma unroll
    for (int j = 0; j < kGroupsPer; ++j) {
      const int gi = threadIdx.x + kThreads * (part * kGroupsPer + j);
      const int row = gi >> 3, grp = gi & 7;
      uint32_t w[8] = {raw[j][0][0], raw[j][0][1], raw[j][0][2], raw[j][0][3],
                       raw[j][1][0], raw[j][1][1], raw[j][1][2], raw[j][1][3]};
      uint32_t lo, hi;
      uint32_t S = quantize_group16<OVF>(w, tab, lo, hi);
      const int chunk = (4 * p + (grp >> 1)) ^ swz(row);
      *(u32x2_t*)(stage + Smem<BM, BN>::kA + row * kRowStride + chunk * 16 + (grp & 1) * 8) = u32x2_t{lo, hi};
      stage[Smem<BM, BN>::kAs + row * kScaleStride + 8 * p + grp] = (uint8_t)S;
      if constexpr (STORE_G) {
        // buffer stores through resources covering the tile's rows inside A
        // (none past the last stage): the rest are dropped, with no branch
        const bool live = kt < nk;
        const int rows = min(BM, M - m0);
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            gcodes + (int64_t)m0 * (K / 2), 0, live ? rows * (K / 2) : 0, 0x00020000);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            gscales + (int64_t)m0 * (K / kGroup), 0, live ? rows * (K / kGroup) : 0, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, rc, row * (K / 2) + grp * 8, kt * kRowBytes, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)S, rs, row * (K / kGroup) + grp, kt * 8, 0);
      }
    }
  }
};

// Direct global->LDS copies of one double stage (FAST shapes, K % 256 == 0).
// One buffer_load ... lds instruction fills a contiguous kilobyte of LDS,
// lane l writing bytes [16l, 16l + 16): 8 code rows of 128 bytes (8 lanes
// per row, one full line each) or 64 scale rows of 16 bytes.  The chunk
// swizzle is applied by the choice of the global chunk each lane copies.
// Tiles whose row count is not a multiple of 256 copy scales in 4-byte
// pieces instead (4 lanes per row, 16 rows per instruction), which keeps the
// instruction count per wave whole.  The rows of a slot are A's then W's
// (WITH_A) or W's alone (fused prologue), contiguous in LDS.  Each operand is
// addressed through a buffer resource covering exactly its tile's valid rows:
// the lane offsets are fixed, the double-stage offset is a scalar, and rows
// past the matrix read zeros rather than other memory.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kBufferWord3);
}

template <int BM, int BN, bool WITH_A>
struct DmaLoader {
  static constexpr int kRA = WITH_A ? BM : 0;
  static constexpr int kRows = kRA + BN;
  static constexpr int kCode = kRows / 8 / 4;             // code copies per wave
  static constexpr int kScaleBytes = kRows % 256 == 0 ? 16 : 4;
  static constexpr int kScaleRowsPer = 64 * kScaleBytes / kScaleStride;  // rows per scale copy
  static constexpr int kScale = kRows / kScaleRowsPer / 4;  // scale copies per wave
  static_assert(kCode * 32 == kRows && kScale * 4 * kScaleRowsPer == kRows, "tile rows");
  uint32_t coff[kCode], soff[kScale];
  // the tiles' valid rows (of A, of W): resources over exactly their bytes
  __amdgpu_buffer_rsrc_t ra_c, rw_c, ra_s, rw_s;
  int wave;

  // Requires BM * K / 2 < 2^31 (checked by the host).
  __device__ __forceinline__ void init(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                                       const uint8_t* w_scales, int M, int N, int K, int m0, int n0, int tid) {
    const int lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ldc = K / 2, ng = K / kGroup;
    const int ma = min(BM, M - m0), nw = min(BN, N - n0);  // valid rows of the tiles
    if (WITH_A) {
      ra_c = tile_rsrc(a_codes + (int64_t)m0 * ldc, ma * ldc);
      ra_s = tile_rsrc(a_scales + (int64_t)m0 * ng, ma * ng);
    }
    rw_c = tile_rsrc(w_codes + (int64_t)n0 * ldc, nw * ldc);
    rw_s = tile_rsrc(w_scales + (int64_t)n0 * ng, nw * ng);
    // rows past the valid ones fall outside the resource and read zeros
#pragma unroll
    for (int j = 0; j < kCode; ++j) {
      const int r = 8 * (wave + 4 * j) + (lane >> 3);
      const int row = r < kRA ? r : r - kRA;
      coff[j] = (uint32_t)(row * ldc + (((lane & 7) ^ swz(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < kScale; ++j) {
      const int t = wave + 4 * j;
      const int r = kScaleBytes == 16 ? 64 * t + lane : 16 * t + (lane >> 2);
      const int row = r < kRA ? r : r - kRA;
      soff[j] = (uint32_t)(row * ng + (kScaleBytes == 16 ? 0 : (lane & 3) << 2));
    }
  }
  // Double stage ds into `slot`; with live false (past the end) the copies
  // go through resources of no bytes, so they move no data (they write
  // zeros).  (The scalar offset is no help there: buffer range checks
  // cover the lane offset only.)  Copies j with j % nparts == part are
  // issued (the stage spreads them).  Copy j of codes holds rows 32j .. 32j
  // + 31 of the slot (eight per wave), so whether it reads A or W is known
  // from j.
  __device__ __forceinline__ void codes(uint8_t* slot, int ds, bool live, int part, int nparts) const {
    uint8_t* lds = slot + (WITH_A ? Smem<BM, BN>::kA : Smem<BM, BN>::kW);
    const __amdgpu_buffer_rsrc_t ra = live ? ra_c : dead(), rw = live ? rw_c : dead();
#pragma unroll
    for (int j = 0; j < kCode; ++j) {
      if (j % nparts != part) continue;
      const int t = wave + 4 * j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(WITH_A && 32 * j < kRA ? ra : rw, (lds_void_t*)(lds + 1024 * t), 16,
                                               (int)coff[j], ds * kRowStride, 0, 0);
    }
  }
  __device__ __forceinline__ void scales(uint8_t* slot, int ds, bool live) const {
    uint8_t* lds = slot + (WITH_A ? Smem<BM, BN>::kAs : Smem<BM, BN>::kWs);
    const __amdgpu_buffer_rsrc_t ra = live ? ra_s : dead(), rw = live ? rw_s : dead();
#pragma unroll
    for (int j = 0; j < kScale; ++j) {
      const int t = wave + 4 * j;
      // copy j covers rows kScaleRowsPer * (4j + wave): all of A, all of W,
      // or (a 128-row A tile under 64-row copies) A for some waves only
      const bool all_a = WITH_A && kScaleRowsPer * (4 * j + 3) < kRA;
      const bool all_w = !WITH_A || kScaleRowsPer * 4 * j >= kRA;
      const __amdgpu_buffer_rsrc_t r = all_a ? ra : all_w ? rw : kScaleRowsPer * t < kRA ? ra : rw;
      if constexpr (kScaleBytes == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds + 1024 * t), 16, (int)soff[j],
                                                 ds * kScaleStride, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds + 256 * t), 4, (int)soff[j],
                                                 ds * kScaleStride, 0, 0);
    }
  }
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t dead() { return tile_rsrc(nullptr, 0); }
};

// --------------------------------------------------------------- compute --

// Per-wave register pipeline over 128-deep stages (TM x TN fragments of
// 32x32, eight K16 steps per stage).  A lane (i, h) handles, in step s, the
// eight codes at byte 32h + 4s of its fragment row (K elements 64h + 8s ..
// +7, group 4h + s/2): the two lane halves split the stage's K range, so a
// step's 16 K elements are 8 from each half, the same for A and W.  Codes
// come from LDS four steps at a time (chunk 2h + q of the stage for steps
// 4q..4q+3), each chunk into its own buffer; the lane's four scales are
// dword h of the stage's eight scale bytes of the row.  A stage is half P of
// an LDS slot.
template <int BM, int BN>
struct WavePipe {
  static constexpr int TM = BM / 64, TN = BN / 64;
  u32x4_t ca[2][TM], cw[2][TN];   // codes of steps 0..3 and 4..7
  uint32_t sa[TM], sw[TN];        // the lane's four scale bytes per fragment
  half2_t pa[2][TM], pw[2][TN];   // sigma pairs, sub-chunks 0 and 1
  half8_t oa[2][TM], ow[2][TN];   // dequantized operands, double-buffered
  int a_off[2][2], w_off[2][2], as_off, ws_off;  // [stage half][chunk buffer]

  __device__ __forceinline__ void init(int wave_m, int wave_n, int li, int lh) {
    // fragment rows differ by multiples of 32, which leave swz unchanged
    const int x = swz(li);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        a_off[p][q] = Smem<BM, BN>::kA + (wave_m + li) * kRowStride + (((4 * p + 2 * lh + q) ^ x) << 4);
        w_off[p][q] = Smem<BM, BN>::kW + (wave_n + li) * kRowStride + (((4 * p + 2 * lh + q) ^ x) << 4);
      }
    as_off = Smem<BM, BN>::kAs + (wave_m + li) * kScaleStride + 4 * lh;
    ws_off = Smem<BM, BN>::kWs + (wave_n + li) * kScaleStride + 4 * lh;
  }
  // codes of steps 4Q..4Q+3 of stage half P of a slot
  template <int P, int Q>
  __device__ __forceinline__ void read_chunk(const uint8_t* slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i) ca[Q][i] = *(const u32x4_t*)(slot + a_off[P][Q] + i * 32 * kRowStride);
#pragma unroll
    for (int j = 0; j < TN; ++j) cw[Q][j] = *(const u32x4_t*)(slot + w_off[P][Q] + j * 32 * kRowStride);
  }
  template <int P>
  __device__ __forceinline__ void read_scales(const uint8_t* slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = *(const uint32_t*)(slot + as_off + 8 * P + i * 32 * kScaleStride);
#pragma unroll
    for (int j = 0; j < TN; ++j) sw[j] = *(const uint32_t*)(slot + ws_off + 8 * P + j * 32 * kScaleStride);
  }
  __device__ __forceinline__ void sigmas() {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      pa[0][i] = sigma_pair<false>(sa[i]);
      pa[1][i] = sigma_pair<true>(sa[i]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      pw[0][j] = sigma_pair<false>(sw[j]);
      pw[1][j] = sigma_pair<true>(sw[j]);
    }
  }
  // operands of step S into operand buffer B
  template <int S, int B>
  __device__ __forceinline__ void dequant() {
    constexpr int q = S >> 2, w = S & 3, g = (S & 3) >> 1;
#pragma unroll
    for (int i = 0; i < TM; ++i) oa[B][i] = dequant8(ca[q][i][w], pa[q][i][g]);
#pragma unroll
    for (int j = 0; j < TN; ++j) ow[B][j] = dequant8(cw[q][j][w], pw[q][j][g]);
  }
  template <int B>
  __device__ __forceinline__ void mfma(f32x16_t (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ow[B][j], oa[B][i], acc[i][j], 0, 0, 0);
  }
};

// Interleave the MFMAs of one step with the VALU issued for the next one:
// a share of the dequantization, then one MFMA (measured faster on gfx950
// than MFMA-first slots).  The sched_barrier at the end keeps each step a
// scheduling region of its own, so the groups cannot pull work from later
// steps (which would stretch register live ranges).
// NVMEM memory instructions (the step's direct copies) are spread evenly
// over the MFMA slots, slot k taking floor((k+1) NVMEM / NMFMA) -
// floor(k NVMEM / NMFMA) of them.
template <int NMFMA, int NVALU, int NVMEM = 0>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int k = 0; k < NMFMA; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x002, (NVALU + NMFMA - 1) / NMFMA, 0);
#pragma unroll
    for (int r = k * NVMEM / NMFMA; r < (k + 1) * NVMEM / NMFMA; ++r)
      __builtin_amdgcn_sched_group_barrier(0x060, 1, 0);  // one memory instruction
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Step S of a stage: LDS reads for the next stage (half PN of slot nxt:
// first chunk in step 3, scales in step 4, second chunk in step 7, each after
// the buffer's last use in this stage), dequantization of step S+1 (or of the
// next stage's step 0), the MFMAs of step S, and step S's part of the fills.
template <int S, int PN, int BM, int BN, int NVMEM = 0, typename Fill>
__device__ __forceinline__ void run_step(WavePipe<BM, BN>& p, f32x16_t (&acc)[BM / 64][BN / 64],
                                         const uint8_t* nxt, Fill& fill) {
  constexpr int TM = BM / 64, TN = BN / 64, NM = TM * TN, ND = 8 * (TM + TN);
  if (S == 3) p.template read_chunk<PN, 0>(nxt);
  if (S == 4) p.template read_scales<PN>(nxt);
  if (S == 7) p.template read_chunk<PN, 1>(nxt);
  if (S == 7) p.sigmas();  // the next stage's; this stage's were last used in step 6
  if (S < 7) p.template dequant<(S + 1) & 7, (S + 1) & 1>();
  else p.template dequant<0, 0>();
  if constexpr (NVMEM > 0) fill(S);  // its NVMEM copies go between the MFMAs
  p.template mfma<S & 1>(acc);
  interleave<NM, ND + (S == 7 ? 2 * (TM + TN) : 0), NVMEM>();
  if constexpr (NVMEM == 0) fill(S);
}

// Epilogue.  Each 32x32 accumulator holds D = W_j . A_i^T, so lane l owns
// output row m = l%32 of the fragment and, in register group g, the four
// consecutive columns 8g + 4(l/32) .. +3.  They are scaled by s_tA * s_tW and
// rounded (nearest-even, hardware conversion).  Storing straight from the
// accumulators would scatter every store instruction over 32 rows (32
// partial cache lines).  Instead the tile goes to LDS 64 rows at a time (32
// rows from each wave row) and is stored back row-contiguously: every lane
// stores 4 consecutive columns and a wave covers whole rows.  The LDS row
// pitch is padded by one lane access, which keeps both the column-scattered
// writes and the row reads free of bank conflicts; ragged or unaligned edges
// fall back to single elements.  Whole-row stores are non-temporal: the
// output is not read again by this launch, and streaming it keeps the L2
// lines of the A and W panels that later tiles reuse (1% faster over the
// prefill step's GEMMs, measured).
template <int BM, int BN, bool OUT_F32>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[BM / 64][BN / 64], uint8_t* smem, void* c, int M,
                                         int N, int m0, int n0, int wave, int lane, float scale) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  constexpr int TM = BM / 64, TN = BN / 64;
  constexpr int E = OUT_F32 ? 4 : 2;       // bytes per output element
  constexpr int W = 4 * E;                 // bytes per lane access
  constexpr int P = BN * E + W;            // LDS row pitch
  constexpr int R = 64 * P;                // LDS bytes of one 64-row pass
  constexpr bool kDouble = 2 * R <= Smem<BM, BN>::kTotal;
  static_assert(R <= Smem<BM, BN>::kTotal, "output pass must fit the operand ring");
  constexpr int kLanesRow = BN / 4;
  constexpr int kRowsIter = kThreads / kLanesRow;
  const int li = lane & 31, lh = lane >> 5;
  const int wr = wave >> 1, wc = wave & 1;
  const int tid = wave * 64 + lane;
  const int cl = tid % kLanesRow, rl0 = tid / kLanesRow;
  const int n = n0 + 4 * cl;
  const bool vec = (N & 3) == 0 && n + 3 < N;
  // full tiles: 16-byte pieces, BN * E / 16 of them per row
  constexpr int kLanesRow16 = BN * E / 16;
  constexpr int kRowsIter16 = kThreads / kLanesRow16;
  const int c16 = tid % kLanesRow16, rl16 = tid / kLanesRow16;
  const bool full = m0 + BM <= M && n0 + BN <= N && (N * E) % 16 == 0;
  __syncthreads();  // every wave is done with the operand ring
#pragma unroll
  for (int fm = 0; fm < TM; ++fm) {
    uint8_t* buf = smem + (kDouble ? (fm & 1) * R : 0);
    if (!kDouble && fm > 0) __syncthreads();
#pragma unroll
    for (int fn = 0; fn < TN; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wc * (BN / 2) + fn * 32 + 8 * g + 4 * lh;
        uint8_t* dst = buf + (wr * 32 + li) * P + col * E;
        const f32x4_t r = f32x4_t{acc[fm][fn][4 * g], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2],
                                  acc[fm][fn][4 * g + 3]} * scale;
        if (OUT_F32) {
          *(f32x4_t*)dst = r;
        } else {
          const bf16x2_t lo = __builtin_convertvector(f32x2_t{r[0], r[1]}, bf16x2_t);
          const bf16x2_t hi = __builtin_convertvector(f32x2_t{r[2], r[3]}, bf16x2_t);
          *(u32x2_t*)dst = u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
      }
    }
    __syncthreads();
    if (full) {
      // whole tile inside C (the common case): every lane stores 8 (bf16) or
      // 4 (binary32) consecutive columns, 16 bytes, with no bounds checks
#pragma unroll
      for (int it = 0; it < 64 / kRowsIter16; ++it) {
        const int lr = it * kRowsIter16 + rl16;
        const int m = m0 + (lr >> 5) * (BM / 2) + fm * 32 + (lr & 31);
        const uint8_t* src = buf + lr * P + c16 * 16;  // 8-byte aligned (the pitch is padded by 8)
        const u32x2_t lo = *(const u32x2_t*)src, hi = *(const u32x2_t*)(src + 8);
        const u32x4_t v = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        __builtin_nontemporal_store(v, (u32x4_t*)((uint8_t*)c + ((int64_t)m * N + n0) * E + c16 * 16));
      }
    } else {
#pragma unroll
      for (int it = 0; it < 64 / kRowsIter; ++it) {
        const int lr = it * kRowsIter + rl0;
        const int m = m0 + (lr >> 5) * (BM / 2) + fm * 32 + (lr & 31);
        if (m >= M) continue;
        const uint8_t* src = buf + lr * P + cl * W;
        const int64_t off = (int64_t)m * N + n;
        if (OUT_F32) {
          const f32x4_t v = *(const f32x4_t*)src;
          if (vec) {
            __builtin_nontemporal_store(v, (f32x4_t*)((float*)c + off));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (n + q < N) ((float*)c)[off + q] = v[q];
          }
        } else {
          const u32x2_t v = *(const u32x2_t*)src;
          if (vec) {
            __builtin_nontemporal_store(v, (u32x2_t*)((uint16_t*)c + off));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (n + q < N) ((uint16_t*)c)[off + q] = (uint16_t)(v[q >> 1] >> (16 * (q & 1)));
          }
        }
      }
    }
  }
}

// Tile order: workgroups go round-robin to the 8 XCDs; consecutive logical
// tiles are put on one XCD (its own L2), and walked in column groups of
// kGroupM row-tiles so neighbouring workgroups share A and W panels.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = tiles_m * tiles_n;
  int logical = bid;
  if ((nwg & 7) == 0) logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
  constexpr int kGroupM = 8;
  const int per_group = kGroupM * tiles_n;
  const int g = logical / per_group;
  const int first = g * kGroupM;
  const int gm = min(tiles_m - first, kGroupM);
  const int in = logical - g * per_group;
  tm = first + in % gm;
  tn = in / gm;
}

// A's tensor scale: from the record, or (REDUCE: the fused prologue without
// a given scale) reduced from the amax pass's partial maxima by the
// quantizer's rule, workgroup 0 storing it in the record.  With a_inline (A
// small enough that every workgroup reads all of it from L2 in about a
// microsecond) there is no amax pass: each workgroup takes max|A| itself,
// the same maximum, so the whole fused GEMM is one launch.
// LOADS: loads in flight per lane while taking max|A| (the small-problem
// kernel has the registers for 16; the tiled kernels keep 8).
template <bool REDUCE, int LOADS = 8>
__device__ __forceinline__ float a_tensor_scale(const GemmArgs& args) {
  if (!REDUCE || args.a_given) return args.a_rec->s_t;
  __shared__ uint32_t red[kThreads / 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint32_t m = 0;
  if (args.a_inline) {
    const uint4* x = (const uint4*)args.a_bf16;
    const int nvec = args.M * args.K / 8;  // at most 2^14 (host-checked)
    for (int base = 0; base < nvec; base += LOADS * kThreads) {
      uint4 v[LOADS];
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int i = base + u * kThreads + tid;
        v[u] = x[i < nvec ? i : nvec - 1];  // a repeated element leaves the maximum unchanged
      }
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        const uint32_t a = bf16_absmax_bits<4>(w) << 16;  // binary32 bits, as the partial maxima
        m = m > a ? m : a;
      }
    }
  } else {
    const uint32_t np = min(args.a_rec->nparts, (uint32_t)MQ_AMAX_PARTS);  // never past the record
    for (uint32_t j = tid; j < np; j += kThreads) {
      uint32_t v = args.a_rec->part[j];
      m = m > v ? m : v;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(m, off, 64);
    m = m > o ? m : o;
  }
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
  for (int i = 1; i < kThreads / 64; ++i) m = m > red[i] ? m : red[i];
  const float s_ta = tensor_scale_from_amax(m);
  if (blockIdx.x == 0 && tid == 0) {
    args.a_rec->s_t = s_ta;
    args.a_rec->amax_bits = m;
  }
  return s_ta;
}

// One output tile (tm, tn): the LDS ring, the main loop and the epilogue.
// s_ta is A's tensor scale; tid is threadIdx.x (a caller that loops over
// tiles passes it through an opaque copy, so that the tile's lane-dependent
// addressing is not hoisted out of its loop and kept live across it).  The
// LDS is free again when it returns.
template <int BM, int BN, bool FAST, bool OUT_F32, bool FUSED, bool WRITE_A = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& args, int tm, int tn, float s_ta, uint8_t* smem,
                                          int tid) {
  constexpr int TM = BM / 64, TN = BN / 64;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int wave_m = (wave >> 1) * (BM / 2), wave_n = (wave & 1) * (BN / 2);
  const GroupView grp = group_of(args, tn);
  const int m0 = tm * BM, n0 = (tn - grp.tn0) * BN;
  const int M = args.M, N = grp.N, K = args.K;
  const int nk = (K + kBK - 1) / kBK;
  const float scale = s_ta * grp.w_rec->s_t;
  // fused prologue: the group-scale constants of A's tensor scale
  GroupScaleTab gtab{};
  if constexpr (FUSED) {
    __shared__ float recip_tab[128];
    gtab = group_scale_tab<kThreads>(s_ta, recip_tab);
  }

  // Main loop and epilogue.  The fused prologue's kernels carry two copies,
  // with and without the quantizer's overflow fix-up, chosen once per
  // workgroup: the common copy has no branches in its loop.
  auto run = [&](auto ovf_c) __attribute__((always_inline)) {
    constexpr bool OVF = decltype(ovf_c)::value;
    f32x16_t acc[TM][TN];
  #pragma unroll
    for (int i = 0; i < TM; ++i)
  #pragma unroll
      for (int j = 0; j < TN; ++j)
  #pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    using SM = Smem<BM, BN>;
    // FAST shapes copy packed operands straight into LDS (A too unless it is
    // quantized here); the fused A tile and all operands of ragged-K shapes go
    // through registers.
    DmaLoader<BM, BN, !FUSED> dma;
    PackedLoader<BM, FAST> la;
    FusedALoader<BM, FAST> fa;
    PackedLoader<BN, FAST> lw;
    ScaleLoader<BM, BN, FAST, !FUSED> ls;
    if constexpr (FAST) dma.init(args.a_codes, args.a_scales, grp.w_codes, grp.w_scales, M, N, K, m0, n0, tid);

    // Register-path fill of stage k into half (k & 1) of a slot.  FAST (only
    // the fused A tile goes this way) clamps k to the last stage; the ragged
    // loaders' bounds checks zero a stage past the end instead, which lets an
    // odd stage count finish on a zero half.
    // The A operand of a stage goes through registers in kParts parts (the
    // fused prologue of a 256-row tile: four), part p loaded at pipeline step
    // 2p and stored at step min(2p + 2, 7), a store before a load in one step.
    constexpr int kParts = FUSED ? FusedALoader<BM, FAST>::kParts : 1;
    auto reg_load = [&](int k, int part) __attribute__((always_inline)) {
      const int kc = FAST ? min(k, nk - 1) : k;
      if constexpr (FUSED) fa.load((const uint16_t*)args.a_bf16, m0, M, K, kc, part);
      else if constexpr (!FAST) la.load(args.a_codes, m0, M, K, kc);
    };
    auto reg_store = [&](uint8_t* slot, int k, int part) __attribute__((always_inline)) {
      if constexpr (FUSED && WRITE_A)
        fa.template quantize_store<BN, OVF, true>(slot, k & 1, gtab, part, (uint8_t*)args.a_codes,
                                                  (uint8_t*)args.a_scales, m0, M, K, k, nk);
      else if constexpr (FUSED)
        fa.template quantize_store<BN, OVF>(slot, k & 1, gtab, part);
      else if constexpr (!FAST) la.store(slot + SM::kA, k & 1);
    };
    // the A parts' register traffic at pipeline step `step` (0..7)
    auto reg_step = [&](uint8_t* slot, int k, int step) __attribute__((always_inline)) {
#pragma unroll
      for (int part = 0; part < kParts; ++part)
        if (step == min(2 * part + 2, 7)) reg_store(slot, k, part);
#pragma unroll
      for (int part = 0; part < kParts; ++part)
        if (step == 2 * part) reg_load(k, part);
    };
    auto load_stage_reg = [&](uint8_t* slot, int k) __attribute__((always_inline)) {
  #pragma unroll
      for (int part = 0; part < kParts; ++part) {
        reg_load(k, part);
        reg_store(slot, k, part);
      }
      if constexpr (!FAST) {
        lw.load(grp.w_codes, n0, N, K, k);
        lw.store(slot + SM::kW, k & 1);
        ls.load(args.a_scales, grp.w_scales, m0, n0, M, N, K, k);
        ls.store(slot, k & 1);
      }
    };
    const int nd = (nk + 1) / 2;  // double stages (FAST shapes have nk even)
    // The direct copies of a double stage go out in the odd stage before it
    // is needed: code copy j in step j % kCodeSteps and the scale copies in
    // step kScaleStep, each placed between two of its step's MFMAs (packed
    // path only: the fused prologue's register traffic keeps its own order).
    // Early steps leave the copies most of a stage to land; spreading them
    // over all eight steps measured slower.
    constexpr int kCodeSteps = 4, kScaleStep = 4;
    constexpr auto copies_in_step = [](int step) constexpr {
      if (!FAST || FUSED) return 0;
      constexpr int kc = DmaLoader<BM, BN, true>::kCode;
      return (step < kCodeSteps && kc > step ? (kc - 1 - step) / kCodeSteps + 1 : 0) +
             (step == kScaleStep ? DmaLoader<BM, BN, true>::kScale : 0);
    };

    // prologue: double stages 0 and 1 into the two slots (stage 3, the second
    // half of slot 1, comes from the register path in stage 0), then the pipe
    // is primed with stage 0
    if constexpr (FAST) {
      dma.codes(smem, 0, true, 0, 1);
      dma.scales(smem, 0, true);
      dma.codes(smem + SM::kSlot, 1, nd > 1, 0, 1);
      dma.scales(smem + SM::kSlot, 1, nd > 1);
    }
    if constexpr (FUSED || !FAST) {
      load_stage_reg(smem, 0);
      load_stage_reg(smem, 1);
      load_stage_reg(smem + SM::kSlot, 2);
    }
    if constexpr (FAST && !FUSED) {
      // only slot 0 is read before the first even barrier (which waits for
      // everything): wait for double stage 0's copies, issued first, and
      // leave double stage 1's in flight (vmcnt counts in issue order); a
      // bare barrier, since __syncthreads() would wait for all copies
      constexpr int kLater = DmaLoader<BM, BN, true>::kCode + DmaLoader<BM, BN, true>::kScale;
      static_assert(kLater < 64, "vmcnt range");
      __builtin_amdgcn_s_waitcnt((kLater & 15) | ((kLater >> 4) << 14) | 0x0070);  // vmcnt(kLater) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
    } else {
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): direct-to-LDS copies included
      __syncthreads();
    }
    WavePipe<BM, BN> pipe;
    pipe.init(wave_m, wave_n, li, lh);
    pipe.template read_chunk<0, 0>(smem);
    pipe.template read_chunk<0, 1>(smem);
    pipe.template read_scales<0>(smem);
    pipe.sigmas();
    pipe.template dequant<0, 0>();

    // Two LDS slots of two stages each.  In double stage d (slot cur; slot nxt
    // holds d+1):
    //  - even stage 2d pre-reads stage 2d+1 (cur, half 1); the register path
    //    fills stage 2d+3 (nxt, half 1).  It ends with every wave's copies and
    //    LDS operations complete and a barrier: afterwards slot nxt is whole
    //    and nobody reads slot cur any more.
    //  - odd stage 2d+1 pre-reads stage 2d+2 (nxt, half 0) and fills slot cur
    //    with double stage d+2: direct copies (two stages to land, before the
    //    next even barrier) and, on the register path, stage 2d+4 (half 0).
    //    No barrier: the next writes to slot nxt come after the next one.
    // Past the end the copies move nothing and register loads are clamped or
    // zeroed; the reads' results are then ignored, so the loop has no branches.
    uint8_t* cur = smem;
    uint8_t* nxt = smem + SM::kSlot;
    for (int d = 0; d < nd; ++d) {
      const int k0 = 2 * d;
      auto fill_even = [&](int step) __attribute__((always_inline)) {
        if constexpr (FUSED || !FAST) {
          const int k = k0 + 3;
          reg_step(nxt, k, step);
          if (step == 2) {
            if constexpr (!FAST) lw.load(grp.w_codes, n0, N, K, k);
          }
          if constexpr (!FAST) {
            if (step == 4) {
              lw.store(nxt + SM::kW, 1);
              ls.load(args.a_scales, grp.w_scales, m0, n0, M, N, K, k);
            }
            if (step == 6) ls.store(nxt, 1);
          }
        }
      };
      auto fill_odd = [&](int step) __attribute__((always_inline)) {
        if constexpr (FUSED || !FAST) {
          // register loads first: waiting for them then does not wait for
          // this stage's direct copies (vmcnt counts in issue order)
          const int k = k0 + 4;
          reg_step(cur, k, step);
          if (step == 2) {
            if constexpr (!FAST) lw.load(grp.w_codes, n0, N, K, k);
          }
          if constexpr (!FAST) {
            if (step == 4) {
              lw.store(cur + SM::kW, 0);
              ls.load(args.a_scales, grp.w_scales, m0, n0, M, N, K, k);
            }
            if (step == 6) ls.store(cur, 0);
          }
        }
        if constexpr (FAST) {
          const bool live = d + 2 < nd;
          if (step < kCodeSteps) dma.codes(cur, d + 2, live, step, kCodeSteps);
          if (step == kScaleStep) dma.scales(cur, d + 2, live);
        }
      };
      run_step<0, 1>(pipe, acc, cur, fill_even);
      run_step<1, 1>(pipe, acc, cur, fill_even);
      run_step<2, 1>(pipe, acc, cur, fill_even);
      run_step<3, 1>(pipe, acc, cur, fill_even);
      run_step<4, 1>(pipe, acc, cur, fill_even);
      run_step<5, 1>(pipe, acc, cur, fill_even);
      run_step<6, 1>(pipe, acc, cur, fill_even);
      run_step<7, 1>(pipe, acc, cur, fill_even);
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      // the direct copies of the packed path: interleaved with the MFMAs
      run_step<0, 0, BM, BN, copies_in_step(0)>(pipe, acc, nxt, fill_odd);
      run_step<1, 0, BM, BN, copies_in_step(1)>(pipe, acc, nxt, fill_odd);
      run_step<2, 0, BM, BN, copies_in_step(2)>(pipe, acc, nxt, fill_odd);
      run_step<3, 0, BM, BN, copies_in_step(3)>(pipe, acc, nxt, fill_odd);
      run_step<4, 0, BM, BN, copies_in_step(4)>(pipe, acc, nxt, fill_odd);
      run_step<5, 0, BM, BN, copies_in_step(5)>(pipe, acc, nxt, fill_odd);
      run_step<6, 0, BM, BN, copies_in_step(6)>(pipe, acc, nxt, fill_odd);
      run_step<7, 0, BM, BN, copies_in_step(7)>(pipe, acc, nxt, fill_odd);
      uint8_t* t = cur;
      cur = nxt;
      nxt = t;
    }
    epilogue<BM, BN, OUT_F32>(acc, smem, grp.c, M, N, m0, n0, wave, lane, scale);
  };
  if constexpr (FUSED) {
    if (gtab.ovf)
      run(BoolC<true>{});
    else
      run(BoolC<false>{});
  } else {
    run(BoolC<false>{});
  }
}

template <int BM, int BN, bool FAST, bool OUT_F32, bool FUSED>
__global__ __launch_bounds__(kThreads, 1) void gemm_nvfp4_kernel(GemmArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_of(blockIdx.x, args.tiles_m, args.tiles_n, tm, tn);
  const float s_ta = a_tensor_scale<FUSED>(args);
  gemm_tile<BM, BN, FAST, OUT_F32, FUSED>(args, tm, tn, s_ta, smem, threadIdx.x);
}

// Fused prologue, quantize-once form.  A workgroup takes the column tiles
// tn = share, share + per_panel, ... of one 256-row panel tm of A.  Its
// first tile runs the fused pipeline (A's stages quantized in registers
// while the MFMAs run) and also stores the quantized stages into the
// caller's NVFP4 buffers for A (standard layout: the bytes mq_quantize_nvfp4
// writes); its other tiles copy A from there with the direct-to-LDS path.
// So an A element is quantized once per workgroup of its panel instead of
// once per column tile.  The per_panel workgroups of a panel each quantize
// all of it (identical bytes; no synchronisation between workgroups).  A
// workgroup's own stores have reached L2 (all waves waited for them, then a
// barrier) before its next tile copies them, and no line of the panel was in
// its L1 before: only this workgroup reads the panel, and only afterwards.
template <bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void gemm_panel_kernel(GemmArgs args, int per_panel) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // workgroups go round-robin to the 8 XCDs; in the XCD-major order a
  // panel's sharers are consecutive, so they share an L2 whenever per_panel
  // divides the grid's share of one XCD (as for M = 16384 or 32768 on 256 CUs)
  const int nwg = gridDim.x;
  int logical = blockIdx.x;
  if ((nwg & 7) == 0) logical = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int tm = logical / per_panel, share = logical - tm * per_panel;
  const float s_ta = a_tensor_scale<true>(args);
  gemm_tile<256, 256, true, OUT_F32, true, true>(args, tm, share, s_ta, smem, threadIdx.x);
  // every wave's stores of A acknowledged (in L2), then the barrier; a
  // device-scope fence here would write back and invalidate the whole L2
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __syncthreads();
  for (int tn = share + per_panel; tn < args.tiles_n; tn += per_panel) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    gemm_tile<256, 256, true, OUT_F32, false>(args, tm, tn, s_ta, smem, tid);
    __syncthreads();  // the epilogue's LDS staging is done before the next fill
  }
}

// ------------------------------------------------------------- small GEMM --
//
// Problems too small to fill the CUs with 128- or 256-row tiles (a short
// prompt's M rows; chosen by row count alone, gemm_small_rows): a workgroup
// owns 16 * WT rows of W and 16 * MT rows of A, its four waves take the K
// chunks (128 elements) in turn, and their partial tiles are summed through
// LDS in wave order (deterministic).  The arithmetic is the tiled kernel's
// (exact binary16 operands g * sigma, binary32 accumulation, the sum scaled
// by fp32(s_tA * s_tW) and rounded to nearest-even bf16), here on
// v_mfma_f32_16x16x32_f16: lane (i, h) holds row i's chunk elements
// 32h .. 32h + 31 (groups 2h and 2h + 1, eight elements per MFMA step) of
// both operands, so the K order is the same for A and W.  A comes packed,
// or (FUSED) as bf16 that each workgroup quantizes in registers by the
// quantizer's rules; with WRITE_A the workgroups also store A's NVFP4
// (standard layout), each chunk of it once.  The summation order differs
// from the tiled kernel's: results agree with it within the GEMM
// tolerance, and with this kernel bit for bit across the A forms,
// groupings and streams.
constexpr int kSmChunk = 128;                      // K elements per chunk
constexpr int kSmWaves = kThreads / 64;            // four: the chunks of K in turn
constexpr int kSmallMaxRows = 128;                 // gemm_small_rows

// One operand row's share of a chunk for one lane: 4 code dwords (steps
// 0..3) and the scale bytes of its two groups (bits 0..15).
struct SmFrag {
  uint32_t c[4];
  uint32_t s;
};
// The same share as bf16 values (fused A): 32 elements, two per word.
struct SmRaw {
  uint4 v[4];
};
template <bool FUSED> struct SmA { typedef SmFrag T; };
template <> struct SmA<true> { typedef SmRaw T; };

// Loads of a valid row (rows past M or N are clamped by the caller: they
// only feed outputs that are never stored).  FAST: K % 128 == 0, whole
// 16-byte pieces; otherwise group by group, groups past K loaded from a
// clamped index and zeroed by a select (zero codes and scales add nothing).
template <bool FAST>
__device__ __forceinline__ SmFrag sm_load_packed(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales, int row, int K, int chunk,
                                                 int h) {
  SmFrag f;
  const int g0 = chunk * (kSmChunk / 16) + 2 * h;  // first group of the lane
  const uint8_t* crow = codes + (int64_t)row * (K / 2);
  const uint8_t* srow = scales + (int64_t)row * (K / 16);
  if constexpr (FAST) {
    const u32x4_t a = *(const u32x4_t*)(crow + g0 * 8);
    f.c[0] = a[0]; f.c[1] = a[1]; f.c[2] = a[2]; f.c[3] = a[3];
    f.s = *(const uint16_t*)(srow + g0);
  } else {
    const int G = K / 16;
    f.s = 0u;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
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

template <bool FAST>
__device__ __forceinline__ SmRaw sm_load_bf16(const void* __restrict__ x, int row, int K, int chunk, int h) {
  SmRaw r;
  const int g0 = chunk * (kSmChunk / 16) + 2 * h;
  const uint4* xr = (const uint4*)((const uint16_t*)x + (int64_t)row * K);  // two uint4 per group
  if constexpr (FAST) {
#pragma unroll
    for (int q = 0; q < 4; ++q) r.v[q] = xr[2 * g0 + q];
  } else {
    const int G = K / 16;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const bool ok = g0 + g < G;
      const int gc = ok ? g0 + g : G - 1;
      const uint4 a = xr[2 * gc], b = xr[2 * gc + 1];
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      r.v[2 * g] = ok ? a : z;
      r.v[2 * g + 1] = ok ? b : z;
    }
  }
  return r;
}

// The quantizer's encoding of the lane's two groups (zeroed groups past K
// get scale byte 0 and zero codes).
template <bool OVF>
__device__ __forceinline__ SmFrag sm_quantize(const SmRaw& r, const GroupScaleTab& tab) {
  SmFrag f;
  f.s = 0u;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint32_t w[8] = {r.v[2 * g].x,     r.v[2 * g].y,     r.v[2 * g].z,     r.v[2 * g].w,
                           r.v[2 * g + 1].x, r.v[2 * g + 1].y, r.v[2 * g + 1].z, r.v[2 * g + 1].w};
    const uint32_t S = quantize_group16<OVF>(w, tab, f.c[2 * g], f.c[2 * g + 1]);
    f.s |= S << (8 * g);
  }
  return f;
}

// Packed A: registers held to two workgroups per CU (more waves to hide the
// loads' latency: 128 x 28672 x 4096 71.9 -> 67.7 us); the fused forms keep
// the whole register file (held to two, they spill: 64 -> 96 us).
template <int WT, int MT, bool FAST, bool OUT_F32, bool FUSED, bool WRITE_A>
__global__ __launch_bounds__(kThreads, FUSED ? 1 : 2) void gemm_small_kernel(GemmArgs args) {
  typedef typename SmA<FUSED>::T AFrag;
  constexpr int NT = WT * MT;  // 16x16 output tiles per workgroup
  __shared__ f32x4_t red[kSmWaves][NT][64];
  __shared__ float recip_tab[128];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int i = lane & 15, h = lane >> 4;
  const int tn = blockIdx.x % args.tiles_n, tm = blockIdx.x / args.tiles_n;
  const GroupView grp = group_of(args, tn);
  const int N = grp.N, K = args.K, M = args.M;
  const int n0 = (tn - grp.tn0) * 16 * WT, m0 = tm * 16 * MT;
  int wrow[WT], arow[MT];
#pragma unroll
  for (int w = 0; w < WT; ++w) wrow[w] = min(n0 + 16 * w + i, N - 1);
#pragma unroll
  for (int u = 0; u < MT; ++u) arow[u] = min(m0 + 16 * u + i, M - 1);
  const int nchunks = (K + kSmChunk - 1) / kSmChunk;
  const int mine = nchunks > wave ? (nchunks - wave + kSmWaves - 1) / kSmWaves : 0;  // this wave's chunks
  // A's NVFP4 is stored once: chunk c of an A tile by the workgroup of W
  // tile c mod tiles_n (spread over the grid, so that no workgroup waits
  // for all of a row's stores)

  f32x4_t acc[WT][MT];
#pragma unroll
  for (int w = 0; w < WT; ++w)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[w][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // chunk t of this wave.  Past the last chunk it re-reads that chunk (the
  // loads stay unconditional, so waiting for one chunk never waits for the
  // next); compute then zeroes W's scales, and the chunk adds nothing.
  auto chunk_of = [&](int t) __attribute__((always_inline)) { return wave + kSmWaves * min(t, mine - 1); };
  auto load = [&](int t, SmFrag (&fw)[WT], AFrag (&fa)[MT]) __attribute__((always_inline)) {
    const int c = chunk_of(t);
#pragma unroll
    for (int w = 0; w < WT; ++w) fw[w] = sm_load_packed<FAST>(grp.w_codes, grp.w_scales, wrow[w], K, c, h);
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      if constexpr (FUSED)
        fa[u] = sm_load_bf16<FAST>(args.a_bf16, arow[u], K, c, h);
      else
        fa[u] = sm_load_packed<FAST>(args.a_codes, args.a_scales, arow[u], K, c, h);
    }
  };
  // the first chunk's operands go out before the tensor scale is known:
  // their latency overlaps the maximum (fused) and the table build
  SmFrag aw[WT], bw[WT];
  AFrag ax[MT], bx[MT];
  if (mine > 0) load(0, aw, ax);
  const float s_ta = a_tensor_scale<FUSED, 16>(args);
  GroupScaleTab gtab{};
  if constexpr (FUSED) gtab = group_scale_tab<kThreads>(s_ta, recip_tab);
  auto run = [&](auto ovf_c) __attribute__((always_inline)) {
    constexpr bool OVF = decltype(ovf_c)::value;
    auto compute = [&](const SmFrag (&fw)[WT], const AFrag (&fa)[MT], int t) __attribute__((always_inline)) {
      const bool live = t < mine;
      SmFrag qa[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        if constexpr (FUSED) {
          qa[u] = sm_quantize<OVF>(fa[u], gtab);
          if (WRITE_A && live && chunk_of(t) % args.tiles_n == tn && m0 + 16 * u + i < M) {
            const int g0 = chunk_of(t) * (kSmChunk / 16) + 2 * h;
            uint8_t* crow = (uint8_t*)args.a_codes + (int64_t)arow[u] * (K / 2);
            uint8_t* srow = (uint8_t*)args.a_scales + (int64_t)arow[u] * (K / 16);
            if constexpr (FAST) {
              // whole chunks: 16-byte aligned codes, 2-byte aligned scales
              *(u32x4_t*)(crow + g0 * 8) = u32x4_t{qa[u].c[0], qa[u].c[1], qa[u].c[2], qa[u].c[3]};
              *(uint16_t*)(srow + g0) = (uint16_t)qa[u].s;
            } else {
#pragma unroll
              for (int g = 0; g < 2; ++g) {
                if (g0 + g < K / 16) {
                  *(u32x2_t*)(crow + (g0 + g) * 8) = u32x2_t{qa[u].c[2 * g], qa[u].c[2 * g + 1]};
                  srow[g0 + g] = (uint8_t)(qa[u].s >> (8 * g));
                }
              }
            }
          }
        } else {
          qa[u] = fa[u];
        }
      }
      half2_t sw[WT], sa[MT];
#pragma unroll
      for (int w = 0; w < WT; ++w) sw[w] = sigma_pair<false>(live ? fw[w].s : 0u);
#pragma unroll
      for (int u = 0; u < MT; ++u) sa[u] = sigma_pair<false>(qa[u].s);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        half8_t ao[MT];
#pragma unroll
        for (int u = 0; u < MT; ++u) ao[u] = dequant8(qa[u].c[q], sa[u][q >> 1]);
#pragma unroll
        for (int w = 0; w < WT; ++w) {
          const half8_t wo = dequant8(fw[w].c[q], sw[w][q >> 1]);
#pragma unroll
          for (int u = 0; u < MT; ++u) acc[w][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wo, ao[u], acc[w][u], 0, 0, 0);
        }
      }
    };
    // two register buffers in turn, one chunk ahead; an odd share ends on a
    // zeroed chunk
    if (mine > 0) {
      for (int t = 0; t < mine; t += 2) {
        load(t + 1, bw, bx);
        __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before this chunk's math
        compute(aw, ax, t);
        load(t + 2, aw, ax);
        __builtin_amdgcn_sched_barrier(0);
        compute(bw, bx, t + 1);
      }
    }
  };
  if constexpr (FUSED) {
    if (gtab.ovf)
      run(BoolC<true>{});
    else
      run(BoolC<false>{});
  } else {
    run(BoolC<false>{});
  }
#pragma unroll
  for (int w = 0; w < WT; ++w)
#pragma unroll
    for (int u = 0; u < MT; ++u) red[wave][w * MT + u][lane] = acc[w][u];
  __syncthreads();
  // wave v finishes output tiles v, v + 4, ...: the waves' partials in wave
  // order.  In tile (w, u) lane l holds rows 4 (l >> 4) .. + 3 of W tile w
  // (output columns) for row l & 15 of A tile u (output row).
  const float scale = s_ta * grp.w_rec->s_t;
  for (int tile = wave; tile < NT; tile += kSmWaves) {
    const int w = tile / MT, u = tile - w * MT;
    f32x4_t s = red[0][tile][lane];
#pragma unroll
    for (int v = 1; v < kSmWaves; ++v) s += red[v][tile][lane];
    const f32x4_t r = s * scale;
    const int m = m0 + 16 * u + i;
    const int n = n0 + 16 * w + 4 * h;
    if (m < M) {
      const int64_t off = (int64_t)m * N + n;
      const bool vec = (N & 3) == 0 && n + 3 < N;
      if constexpr (OUT_F32) {
        float* c = (float*)grp.c;
        if (vec) {
          *(f32x4_t*)(c + off) = r;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) c[off + q] = r[q];
        }
      } else {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
        const bf16x4_t b = __builtin_convertvector(r, bf16x4_t);
        uint16_t* c = (uint16_t*)grp.c;
        if (vec) {
          *(bf16x4_t*)(c + off) = b;
        } else {
          const u16x4_t bb = __builtin_bit_cast(u16x4_t, b);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) c[off + q] = bb[q];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host --

constexpr int kMaxDevices = 64;

template <int BM, int BN, bool FAST, bool OUT_F32, bool FUSED>
static hipError_t launch_cfg(const GemmArgs& a0, int dev, hipStream_t stream) {
  GemmArgs a = a0;
  a.tiles_m = (a.M + BM - 1) / BM;
  int tn = 0;
  for (int g = 0; g < a.ngroup; ++g) {
    tn += (a.n[g] + BN - 1) / BN;
    a.tn_end[g] = tn;
  }
  a.tiles_n = tn;
  auto kern = gemm_nvfp4_kernel<BM, BN, FAST, OUT_F32, FUSED>;
  constexpr int lds = Smem<BM, BN>::kTotal;
  static bool attr_done[kMaxDevices] = {};  // benign race: the call is idempotent
  if (dev < 0 || dev >= kMaxDevices || !attr_done[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) attr_done[dev] = true;
  }
  log_launch("gemm_nvfp4_kernel", a.tiles_m * a.tiles_n, kThreads, lds,
             "tile=%dx%d fast=%d out_f32=%d fused=%d M=%d K=%d tiles=%dx%d groups=%d", BM, BN, (int)FAST,
             (int)OUT_F32, (int)FUSED, a.M, a.K, a.tiles_m, a.tiles_n, a.ngroup);
  hipLaunchKernelGGL(kern, dim3(a.tiles_m * a.tiles_n), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

// The fast variant needs whole double stages (K % 256 == 0) and buffer
// offsets of a 256-row tile below 2^31 (256 * K/2 < 2^31).
static bool fast_shape(int64_t K) { return K % (2 * kBK) == 0 && K < (int64_t(1) << 24); }

// Quantize-once fused launch: one workgroup per (panel, share), with as many
// sharers per panel as fill the CUs (at most one per column tile).
template <bool OUT_F32>
static hipError_t launch_panel(const GemmArgs& a0, uint8_t* codes, uint8_t* scales, const DeviceInfo& dev,
                               hipStream_t stream) {
  GemmArgs a = a0;
  a.a_codes = codes;
  a.a_scales = scales;
  a.tiles_m = (a.M + 255) / 256;
  int tn = 0;
  for (int g = 0; g < a.ngroup; ++g) {
    tn += (a.n[g] + 255) / 256;
    a.tn_end[g] = tn;
  }
  a.tiles_n = tn;
  int per = dev.num_cu / a.tiles_m;
  per = per < 1 ? 1 : (per > tn ? tn : per);
  auto kern = gemm_panel_kernel<OUT_F32>;
  constexpr int lds = Smem<256, 256>::kTotal;
  static bool attr_done[kMaxDevices] = {};  // benign race: the call is idempotent
  if (dev.device < 0 || dev.device >= kMaxDevices || !attr_done[dev.device]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    if (dev.device >= 0 && dev.device < kMaxDevices) attr_done[dev.device] = true;
  }
  log_launch("gemm_panel_kernel", a.tiles_m * per, kThreads, lds,
             "out_f32=%d M=%d K=%d panels=%d per_panel=%d column_tiles=%d groups=%d", (int)OUT_F32, a.M, a.K,
             a.tiles_m, per, tn, a.ngroup);
  hipLaunchKernelGGL(kern, dim3(a.tiles_m * per), dim3(kThreads), lds, stream, a, per);
  return hipGetLastError();
}

template <int BM, int BN, bool FUSED>
static hipError_t dispatch_flags(const GemmArgs& a, bool out_f32, int d, hipStream_t s) {
  // the 16-byte scale copies want 16-byte aligned scale rows
  bool fast = fast_shape(a.K) && (a.a_bf16 || ((uintptr_t)a.a_scales & 15) == 0);
  for (int g = 0; g < a.ngroup; ++g) fast = fast && ((uintptr_t)a.w_scales[g] & 15) == 0;
  if (fast) return out_f32 ? launch_cfg<BM, BN, true, true, FUSED>(a, d, s) : launch_cfg<BM, BN, true, false, FUSED>(a, d, s);
  return out_f32 ? launch_cfg<BM, BN, false, true, FUSED>(a, d, s) : launch_cfg<BM, BN, false, false, FUSED>(a, d, s);
}

bool gemm_small_rows(int64_t M) { return M <= kSmallMaxRows; }

template <int WT, int MT, bool FAST, bool OUT_F32, bool FUSED, bool WRITE_A>
static hipError_t launch_small_cfg(const GemmArgs& a0, hipStream_t stream) {
  GemmArgs a = a0;
  a.tiles_m = (a.M + 16 * MT - 1) / (16 * MT);
  int tn = 0;
  for (int g = 0; g < a.ngroup; ++g) {
    tn += (a.n[g] + 16 * WT - 1) / (16 * WT);
    a.tn_end[g] = tn;
  }
  a.tiles_n = tn;
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
  log_launch("gemm_small_kernel", (unsigned)grid, kThreads, 0,
             "w_rows_per_wg=%d a_rows_per_wg=%d fast=%d out_f32=%d fused=%d write_a=%d M=%d K=%d tiles=%dx%d "
             "groups=%d",
             16 * WT, 16 * MT, (int)FAST, (int)OUT_F32, (int)FUSED, (int)WRITE_A, a.M, a.K, a.tiles_m, a.tiles_n,
             a.ngroup);
  hipLaunchKernelGGL((gemm_small_kernel<WT, MT, FAST, OUT_F32, FUSED, WRITE_A>), dim3((unsigned)grid),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int WT, int MT, bool FAST, bool OUT_F32>
static hipError_t launch_small_form(const GemmArgs& a, bool fused, bool write_a, hipStream_t s) {
  if constexpr (MT > 2) {
    // the fused forms take at most two A tiles (launch_small)
    if (fused) return hipErrorInvalidValue;
    return launch_small_cfg<WT, MT, FAST, OUT_F32, false, false>(a, s);
  } else {
    if (!fused) return launch_small_cfg<WT, MT, FAST, OUT_F32, false, false>(a, s);
    if (write_a) return launch_small_cfg<WT, MT, FAST, OUT_F32, true, true>(a, s);
    return launch_small_cfg<WT, MT, FAST, OUT_F32, true, false>(a, s);
  }
}

template <int WT, int MT>
static hipError_t launch_small_wm(const GemmArgs& a, bool fast, bool out_f32, bool fused, bool write_a,
                                  hipStream_t s) {
  if (fast)
    return out_f32 ? launch_small_form<WT, MT, true, true>(a, fused, write_a, s)
                   : launch_small_form<WT, MT, true, false>(a, fused, write_a, s);
  return out_f32 ? launch_small_form<WT, MT, false, true>(a, fused, write_a, s)
                 : launch_small_form<WT, MT, false, false>(a, fused, write_a, s);
}

// Tiles per workgroup: as many W and A tiles (up to 4 x 4: fewer operand
// re-reads through L2, fewer dequantizations per MFMA) as still leave a
// workgroup per CU; below that, the smallest, so that a latency-bound
// problem spreads over as many CUs as it can.  Halving the larger count
// first reaches 4x4, 2x4, 2x2, 1x2, 1x1 (M > 32), 4x2, 2x2, 1x2, 1x1
// (17..32 rows) or 4x1, 2x1, 1x1 (M <= 16).  The fused forms, whose
// workgroups also quantize their A rows, start from two A tiles (measured
// 18-26% faster at 128 x 4096 x 4096, 64 x 14336 x 4096 and
// 128 x 4096 x 14336, 9% slower at 128 x 14336 x 4096; packed A is 35%
// slower that way at the wide weights).  The tile counts do not change
// any output element's summation order (that is fixed by the K chunks and
// the wave order), so every choice gives the same bits.
static hipError_t launch_small(const GemmArgs& a, const int64_t* n, int ngroup, bool fast, bool out_f32, bool fused,
                               bool write_a, int num_cu, hipStream_t s) {
  int wt = 4, mt = a.M <= 16 ? 1 : (a.M <= 32 || fused) ? 2 : 4;
  auto grid = [&](int w, int m) {
    int64_t t = 0;
    for (int g = 0; g < ngroup; ++g) t += (n[g] + 16 * w - 1) / (16 * w);
    return t * ((a.M + 16 * m - 1) / (16 * m));
  };
  while (grid(wt, mt) < num_cu && (wt > 1 || mt > 1)) {
    if (wt >= mt) wt /= 2;
    else mt /= 2;
  }
  switch (wt * 8 + mt) {
    case 4 * 8 + 4: return launch_small_wm<4, 4>(a, fast, out_f32, fused, write_a, s);
    case 4 * 8 + 2: return launch_small_wm<4, 2>(a, fast, out_f32, fused, write_a, s);
    case 4 * 8 + 1: return launch_small_wm<4, 1>(a, fast, out_f32, fused, write_a, s);
    case 2 * 8 + 4: return launch_small_wm<2, 4>(a, fast, out_f32, fused, write_a, s);
    case 2 * 8 + 2: return launch_small_wm<2, 2>(a, fast, out_f32, fused, write_a, s);
    case 2 * 8 + 1: return launch_small_wm<2, 1>(a, fast, out_f32, fused, write_a, s);
    case 1 * 8 + 2: return launch_small_wm<1, 2>(a, fast, out_f32, fused, write_a, s);
    default: return launch_small_wm<1, 1>(a, fast, out_f32, fused, write_a, s);
  }
}

// Tile shape: estimated time = rounds of workgroups over the CUs x tile
// area / relative efficiency.  Smaller wave tiles dequantize more operand
// fragments per MFMA; the efficiencies are measured MI355X rates relative to
// the 256x256 tile.
// The ragged-K variant of the 256x256 tile does not fit its registers, so
// shapes outside the fast variant start from the next size.
static int pick_tile(int64_t M, const int64_t* N, int ngroup, int64_t K, int num_cu) {
  struct Cand { int bm, bn; double eff; };
  const Cand cands[] = {{256, 256, 1.0}, {256, 128, 0.65}, {128, 256, 0.65}, {128, 128, 0.57}};
  int best = 1;
  double best_t = 1e300;
  for (int i = fast_shape(K) ? 0 : 1; i < 4; ++i) {
    int64_t tn = 0;
    for (int g = 0; g < ngroup; ++g) tn += (N[g] + cands[i].bn - 1) / cands[i].bn;
    const int64_t tiles = ((M + cands[i].bm - 1) / cands[i].bm) * tn;
    const int64_t rounds = (tiles + num_cu - 1) / num_cu;
    const double t = (double)rounds * cands[i].bm * cands[i].bn / cands[i].eff;
    if (t < best_t * 0.999) { best_t = t; best = i; }
  }
  return best;
}

// The quantize-once form runs one fused tile per sharer of a panel, which
// takes about 1.4 plain tiles' time: it pays only where each sharer goes on
// to enough plain tiles (measured at M = 32768: 4 tiles per sharer 6.6%, 8
// tiles 0.5-3% behind the separate encode pass + plain GEMM; at M = 4096
// and below, with one tile per sharer, up to 3.7x behind).  Elsewhere the
// call takes the separate path, whose output is bit-identical.
static std::atomic<int> g_panel_min_tiles{4};

int set_panel_min_tiles(int tiles) { return g_panel_min_tiles.exchange(tiles); }

static bool panel_pays(int64_t M, const int64_t* n, int ngroup, int num_cu) {
  const int64_t tiles_m = (M + 255) / 256;
  int64_t tn = 0;
  for (int g = 0; g < ngroup; ++g) tn += (n[g] + 255) / 256;
  int64_t per = num_cu / tiles_m;
  per = per < 1 ? 1 : (per > tn ? tn : per);
  return (tn + per - 1) / per >= g_panel_min_tiles.load();
}

hipError_t launch_gemm(const GemmOperandA& A, const GemmWeight* w, int ngroup, int64_t M, int64_t K, bool out_f32,
                       const DeviceInfo& dev, hipStream_t stream) {
  GemmArgs a{};
  a.a_codes = A.codes; a.a_scales = A.scales; a.a_bf16 = A.bf16; a.a_rec = A.rec;
  a.a_given = A.given ? 1 : 0;
  a.a_inline = A.inline_amax ? 1 : 0;
  int64_t n[kMaxGroup];
  for (int g = 0; g < ngroup; ++g) {
    a.w_codes[g] = w[g].codes; a.w_scales[g] = w[g].scales; a.w_rec[g] = w[g].rec;
    a.c[g] = w[g].c; a.n[g] = (int)w[g].n;
    n[g] = w[g].n;
  }
  a.ngroup = ngroup;
  a.M = (int)M; a.K = (int)K;
  if (gemm_small_rows(M)) {
    // whole chunks of K take 16-byte loads (bases are 16-byte aligned and
    // scale rows then even-sized)
    const bool fast = K % kSmChunk == 0;
    const bool fused = A.bf16 != nullptr, write_a = fused && A.out_codes;
    if (write_a) {
      a.a_codes = A.out_codes;
      a.a_scales = A.out_scales;
    }
    return launch_small(a, n, ngroup, fast, out_f32, fused, write_a, dev.num_cu, stream);
  }
  if (A.bf16 && A.out_codes) {
    // fused, A's NVFP4 kept: quantize once per panel, or (other shapes, and
    // where the panel form does not pay) the standalone encode pass into the
    // same buffers and the plain GEMM
    bool fast = fast_shape(K) && ((uintptr_t)A.out_codes & 15) == 0 && ((uintptr_t)A.out_scales & 15) == 0;
    for (int g = 0; g < ngroup; ++g) fast = fast && ((uintptr_t)a.w_scales[g] & 15) == 0;
    if (fast && panel_pays(M, n, ngroup, dev.num_cu))
      return out_f32 ? launch_panel<true>(a, A.out_codes, A.out_scales, dev, stream)
                     : launch_panel<false>(a, A.out_codes, A.out_scales, dev, stream);
    hipError_t e = launch_quantize(A.bf16, M * K, A.out_codes, A.out_scales, A.rec, A.given, dev, stream);
    if (e != hipSuccess) return e;
    a.a_codes = A.out_codes;
    a.a_scales = A.out_scales;
    a.a_bf16 = nullptr;
  } else if (A.bf16) {
    // fused: an A tile is re-quantized once per column tile, so wide tiles
    // keep the quantize work per MFMA low; but where 256x256 tiles would
    // leave half the CUs idle (short prompts past the small-problem kernel),
    // 128x256 tiles double the workgroups (M = 256, N = K = 4096: 125 ->
    // 70 us; 512 x 4096 x 14336: 401 -> 228 us)
    bool fast = fast_shape(K);  // 256x256 where the direct W copies apply
    for (int g = 0; g < ngroup; ++g) fast = fast && ((uintptr_t)a.w_scales[g] & 15) == 0;
    int64_t tiles256 = 0;
    for (int g = 0; g < ngroup; ++g) tiles256 += (n[g] + 255) / 256;
    tiles256 *= (M + 255) / 256;
    if (fast && 2 * tiles256 > dev.num_cu)
      return out_f32 ? launch_cfg<256, 256, true, true, true>(a, dev.device, stream)
                     : launch_cfg<256, 256, true, false, true>(a, dev.device, stream);
    return dispatch_flags<128, 256, true>(a, out_f32, dev.device, stream);
  }
  switch (pick_tile(M, n, ngroup, K, dev.num_cu)) {
    case 0: return dispatch_flags<256, 256, false>(a, out_f32, dev.device, stream);
    case 1: return dispatch_flags<256, 128, false>(a, out_f32, dev.device, stream);
    case 2: return dispatch_flags<128, 256, false>(a, out_f32, dev.device, stream);
    default: return dispatch_flags<128, 128, false>(a, out_f32, dev.device, stream);
  }
}

}  // namespace mq
