/*
 * mq.h - C ABI of the NVFP4 prefill linear and BF16 decode GEMV library
 *        (libmq.so, HIP for AMD Instinct MI355X / gfx950).
 *
 * The method ("Mix-Quant: Quantized Prefilling, Precise Decoding for Agentic
 * LLMs"; gist.science English explainer, Technical Summary s.2 Methodology):
 * prefill linears run with weights and activations both in NVFP4 (W4A4; s.2
 * System-Level Deployment), a format with one local scale per group of 16
 * elements plus a tensor-level scale, elements rounded to nearest (s.2
 * Hybrid Precision Strategy); decode keeps the original BF16 weights (same
 * passage, Decoding).  This library is that data-parallel path on one GPU:
 *
 *   mq_quantize_nvfp4      bf16 [rows][cols] -> NVFP4 (dynamic tensor scale)
 *   mq_gemm_nvfp4_prefill  C = A . W^T with A, W in NVFP4, fp32 accumulate,
 *                          bf16 (or fp32) output
 *   mq_gemm_nvfp4_prefill_grouped
 *                          the same for several weights that share A, in one
 *                          launch
 *   mq_gemv_bf16_decode    Y = X . W^T on bf16 X [M][K] and W [N][K]
 *   mq_gemv_bf16_decode_grouped
 *                          the same for several weights that share X, in one
 *                          launch
 *   mq_rmsnorm_amax / mq_swiglu_amax
 *                          the ops that write the linears' activations,
 *                          emitting the amax pass's partial maxima
 *   mq_rmsnorm_quantize_nvfp4
 *                          RMSNorm whose output goes straight to NVFP4
 *                          (the bf16 output is never stored)
 *   mq_gemv_nvfp4_decode   the decode GEMV with X and W in NVFP4 (the
 *                          uniform-quantization baseline the method avoids)
 *   mq_linear_prepare / mq_linear_forward / mq_linear_path
 *                          one weight kept in both formats (original BF16
 *                          and an NVFP4 copy), each call routed to the
 *                          prefill (NVFP4) or decode (BF16) path
 *
 * Formats (readings where the pages are silent):
 *   element   OCP E2M1 4-bit code = sign<<3 | magnitude index, magnitudes
 *             {0, .5, 1, 1.5, 2, 3, 4, 6}; two codes per byte, even column in
 *             the low nibble; codes stored [rows][cols/2], row-major.
 *   group     one OCP E4M3 ("fn", bias 7, max 448) byte per 16 consecutive
 *             elements of a row, stored [rows][cols/16], row-major.
 *   tensor    binary32 decode scale s_t = amax/2688 (1.0 if amax == 0), kept
 *             in a device-resident mq_scale_rec.
 *   Quantization, per group: rho = (a/6)/s_t, S = E4M3_rne_sat(rho),
 *   d = value(S)*s_t, e = 1/d (0 if d == 0); per element y = x*e,
 *   code = signbit(x)<<3 | E2M1_rne_sat(|y|) (NaN y -> 0): each a single
 *   IEEE binary32 operation.  Results are bit-exact and unique.
 *
 * Conventions for every entry point:
 *   - All data pointers are caller-owned DEVICE memory on the current HIP
 *     device; the struct arguments themselves (mq_nvfp4) live in host
 *     memory.  The library allocates no device memory and frees nothing.
 *   - Arguments are checked synchronously on the host.  On failure the call
 *     returns an MQ_ERR_* code and launches nothing; mq_last_error() gives a
 *     thread-local message.  Nothing is thrown or aborted across the ABI.
 *   - On success, work is queued asynchronously on hip_stream (a
 *     hipStream_t; NULL = the default stream) and MQ_OK is returned without
 *     synchronising.  Launch failures seen by hipGetLastError() right after
 *     the launch give MQ_ERR_LAUNCH.
 *   - The queued work is kernel launches only (no memset, copy or host
 *     synchronisation), so calls may be captured into a HIP graph and
 *     replayed; the first call of each kernel on a device sets its
 *     dynamic-LDS attribute, so make one eager call before capturing.
 *   - Matrices are contiguous and row-major (leading dimension = columns).
 *   - Outputs are bit-deterministic: no atomics touch output values.
 *   - Calls are thread-safe.  Two calls in flight at once must not share an
 *     output buffer or an mq_scale_rec.
 *   - With MQ_LOG=1 in the environment (read once per process), every launch
 *     prints its kernel, grid, block, dynamic LDS and shape to stderr.
 */
#ifndef MQ_H_
#define MQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mq_status;
#define MQ_OK           0
#define MQ_ERR_INVALID  1 /* NULL pointer, unknown flag, bad combination   */
#define MQ_ERR_SHAPE    2 /* a size <= 0, cols or K not a multiple of 16,
                             or a size whose byte count overflows int64     */
#define MQ_ERR_ALIGN    3 /* a device pointer not aligned as documented     */
#define MQ_ERR_DEVICE   4 /* no HIP device, or the current one is not gfx950 */
#define MQ_ERR_LAUNCH   5 /* a kernel launch reported an error              */

/* Number of per-workgroup partial maxima an mq_scale_rec can hold. */
#define MQ_AMAX_PARTS 1020

/* Most weights one mq_gemm_nvfp4_prefill_grouped call takes. */
#define MQ_MAX_GROUP 4

/* Tensor-scale record, DEVICE memory, 4096 bytes, 16-byte aligned.
 * s_t       binary32 decode scale of the tensor (read by the GEMM epilogue).
 * amax_bits bit pattern of max|x| that s_t came from (0 when given).
 * nparts    number of valid entries in part[] (written by the amax pass).
 * flags     call counter of the single-launch quantizer (mq_quantize_nvfp4),
 *           whose workgroups meet at the tensor maximum through it; only
 *           that kernel reads or writes it.
 * part[]    per-workgroup maxima of |x| as binary32 bit patterns; written by
 *           the amax pass (or the single-launch quantizer) and reduced by
 *           whichever kernel consumes the scale.
 * Zero the record once when allocating it (flags must start at 0); no call
 * needs it re-initialised afterwards: every other field a call reads was
 * written earlier in the same call, except s_t under MQ_SCALE_GIVEN
 * (caller-set).  One record serves one call at a time: calls that share a
 * record must be ordered (same stream, or synchronised). */
typedef struct mq_scale_rec {
  float s_t;
  uint32_t amax_bits;
  uint32_t nparts;
  uint32_t flags;
  uint32_t part[MQ_AMAX_PARTS];
} mq_scale_rec;

/* An NVFP4 matrix of [rows][cols] elements.  HOST struct of DEVICE pointers.
 * codes  uint8 [rows][cols/2]  (16-byte aligned)
 * scales uint8 [rows][cols/16] (8-byte aligned)
 * rec    mq_scale_rec          (16-byte aligned)
 * Every entry point checks these alignments and returns MQ_ERR_ALIGN
 * otherwise. */
typedef struct mq_nvfp4 {
  uint8_t* codes;
  uint8_t* scales;
  mq_scale_rec* rec;
} mq_nvfp4;

/* flags */
#define MQ_SCALE_DYNAMIC 0u  /* tensor scale from max|x| of this call (default) */
#define MQ_SCALE_GIVEN   1u  /* use rec->s_t as already set (finite, > 0)      */
#define MQ_OUT_BF16      0u  /* GEMM output bf16 (default)                      */
#define MQ_OUT_F32       2u  /* GEMM output binary32 (pre-rounding value)       */
#define MQ_A_FUSED_BF16  4u  /* GEMM: A given as bf16, quantized in-kernel      */
#define MQ_PHASE_PREFILL 8u  /* linear: this call is a prefill (NVFP4 path)     */
#define MQ_PHASE_DECODE 16u  /* linear: this call is a decode step (BF16 path)  */
#define MQ_SCALE_PARTIALS 32u /* rec already holds the input's partial maxima,
                                 written by mq_rmsnorm_amax / mq_swiglu_amax
                                 earlier on the same stream: no amax pass    */

/*
 * mq_quantize_nvfp4 - quantize a bf16 matrix to NVFP4.
 *   The two-level scaling of the gist.science explainer, s.2 Hybrid
 *   Precision Strategy: tensor scale from the absolute maximum of the whole
 *   input (taken at run time), an E4M3 scale per 16-element group of a row,
 *   round-to-nearest-even E2M1 codes.
 * x_bf16   DEVICE bf16 [rows][cols], 16-byte aligned, finite values.
 * rows     >= 1.   cols >= 16, cols % 16 == 0.
 * out      HOST pointer to an mq_nvfp4 whose codes/scales/rec are written.
 *          out->rec->s_t, amax_bits, nparts and part[] are overwritten
 *          (with MQ_SCALE_GIVEN only out->rec->s_t is read).
 * flags    MQ_SCALE_DYNAMIC, MQ_SCALE_GIVEN or MQ_SCALE_PARTIALS (out->rec's
 *          nparts and part[] already hold x's partial maxima from a producer
 *          op: s_t is derived from them, bit-identical to the dynamic case).
 * Launches: given scale or partials, the encode alone.  Dynamic scale:
 *          for rows*cols <= 2^17 the encode alone too, every workgroup
 *          taking max|x| itself (out->rec then receives s_t and amax_bits,
 *          not nparts / part[]).  Where each lane of a grid of one
 *          512-thread workgroup per CU holds 17 to 64 groups of 8 elements
 *          (on 256 CUs: 2^24 < rows*cols <= 2^26), one launch: the lanes
 *          keep their share of x in registers (and LDS), the workgroups meet at
 *          the tensor maximum through out->rec (part[] and flags; a bounded
 *          wait: a workgroup whose partners are not resident in time reads
 *          all of x for the maximum itself, same result; nparts is left 0),
 *          then encode.  Otherwise an amax pass, then the encode.
 */
mq_status mq_quantize_nvfp4(const void* x_bf16, int64_t rows, int64_t cols,
                            const mq_nvfp4* out, uint32_t flags,
                            void* hip_stream);

/*
 * mq_gemm_nvfp4_prefill - C[M][N] = A[M][K] . W[N][K]^T, NVFP4 operands.
 *   The W4A4 prefill linear (gist.science explainer, s.2 System-Level
 *   Deployment, prefill workers).  Every product uses the exact dequantized
 *   operands g*sigma; accumulation is binary32; the result is multiplied by
 *   s_tA*s_tW and rounded to nearest-even bf16 (or stored as binary32 with
 *   MQ_OUT_F32).  No bias.  Up to M = 128 every form of the call runs one
 *   small-problem kernel that splits K over its waves (its sums are ordered
 *   differently from the tiled kernel's, so results for M <= 128 and M > 128
 *   agree within the GEMM tolerance, not bit for bit; at any one M every
 *   form, grouping and stream gives the same bits).
 * a        HOST pointer to the quantized activations (codes, scales, rec;
 *          rec->s_t must already hold A's scale, e.g. from
 *          mq_quantize_nvfp4 earlier on the same stream).  With
 *          MQ_A_FUSED_BF16, a->rec receives the amax pass of a_bf16 (or
 *          supplies s_t under MQ_SCALE_GIVEN; when M*K <= 2^17 and either
 *          a->codes is NULL or M <= 128 there is no amax pass: every
 *          workgroup of the GEMM takes max|a_bf16| itself, and a->rec
 *          receives s_t and amax_bits only, so the whole call is one launch)
 *          and a->codes / a->scales are
 *          either both NULL (every A tile is re-quantized inside the GEMM's
 *          pipeline for each column tile) or both given, [M][K/2] and
 *          [M][K/16] bytes, 16- and 8-byte aligned: then A's NVFP4 is
 *          written there (the bytes mq_quantize_nvfp4 writes) and each
 *          workgroup quantizes the 256-row panel of A it reads once, in its
 *          first tile, and copies it from there for its other tiles (the
 *          form for long activations, taken where each panel's workgroups
 *          get at least four column tiles; other shapes, and those outside
 *          the direct-copy path, run the encode pass into the buffers, then
 *          the plain GEMM, with the same result).
 *          Nothing else may read or write those buffers during the call.
 * a_bf16   DEVICE bf16 [M][K], 16-byte aligned; only with MQ_A_FUSED_BF16,
 *          else must be NULL.  The fused path computes exactly the codes
 *          mq_quantize_nvfp4 would, inside the GEMM.
 * w        HOST pointer to the quantized weights [N][K] (rec->s_t set).
 * c        DEVICE output [M][N], bf16 (16-byte aligned) or binary32.
 * M, N     >= 1.  K >= 16, K % 16 == 0.
 * flags    MQ_OUT_BF16 | MQ_OUT_F32, optionally | MQ_A_FUSED_BF16, and with
 *          it optionally | MQ_SCALE_GIVEN or | MQ_SCALE_PARTIALS (a->rec
 *          holds a_bf16's partial maxima: no amax pass).
 */
mq_status mq_gemm_nvfp4_prefill(const mq_nvfp4* a, const void* a_bf16,
                                const mq_nvfp4* w, void* c,
                                int64_t M, int64_t N, int64_t K,
                                uint32_t flags, void* hip_stream);

/*
 * mq_gemm_nvfp4_prefill_grouped - C_g[M][N_g] = A[M][K] . W_g[N_g][K]^T for
 *   g = 0 .. n_group-1: the prefill linears that read one activation (the
 *   gate and up projections of an MLP, or k and v) as a single launch, whose
 *   workgroups cover all the outputs' tiles.  Same arithmetic as
 *   mq_gemm_nvfp4_prefill (gist.science explainer, s.2 System-Level
 *   Deployment); each C_g is bit-identical to what mq_gemm_nvfp4_prefill(a,
 *   a_bf16, &w[g], c[g], M, N[g], K, flags, hip_stream) writes.
 * a, a_bf16, M, K, flags   as for mq_gemm_nvfp4_prefill; with
 *          MQ_A_FUSED_BF16 the amax pass over a_bf16 runs once for all
 *          groups.
 * n_group  1 .. MQ_MAX_GROUP.
 * w        HOST array of n_group weights W_g [N_g][K] (rec->s_t set each).
 * c        HOST array of n_group DEVICE outputs C_g [M][N_g], same element
 *          type and alignment rules as c of mq_gemm_nvfp4_prefill; the
 *          outputs must not overlap.
 * N        HOST array of the n_group column counts, each >= 1.
 */
mq_status mq_gemm_nvfp4_prefill_grouped(const mq_nvfp4* a, const void* a_bf16,
                                        int32_t n_group, const mq_nvfp4* w,
                                        void* const* c, const int64_t* N,
                                        int64_t M, int64_t K,
                                        uint32_t flags, void* hip_stream);

/*
 * mq_gemv_bf16_decode - Y[M][N] = X[M][K] . W[N][K]^T in bf16.
 *   The decode step's linear on the original BF16 weights (gist.science
 *   explainer, s.2 Hybrid Precision Strategy, Decoding; s.2 System-Level
 *   Deployment, decode workers).  bf16 products, binary32 accumulation,
 *   nearest-even bf16 output.  Memory-bound on W.
 * x_bf16   DEVICE bf16 [M][K], 16-byte aligned.
 * w_bf16   DEVICE bf16 [N][K], 16-byte aligned.
 * y_bf16   DEVICE bf16 [M][N].
 * M        1..32 (decode batch).  N >= 1.  K >= 16, K % 16 == 0.
 * flags    0.
 */
mq_status mq_gemv_bf16_decode(const void* x_bf16, const void* w_bf16,
                              void* y_bf16, int64_t M, int64_t N, int64_t K,
                              uint32_t flags, void* hip_stream);

/*
 * mq_gemv_bf16_decode_grouped - Y_g[M][N_g] = X[M][K] . W_g[N_g][K]^T for
 *   g = 0 .. n_group-1: the decode linears that read one input (q, k and v
 *   of attention; gate and up of an MLP) as a single launch, whose
 *   workgroups cover all the weights' row tiles.  Same arithmetic as
 *   mq_gemv_bf16_decode (gist.science explainer, s.2 Hybrid Precision
 *   Strategy, Decoding); each Y_g is bit-identical to what
 *   mq_gemv_bf16_decode(x, W_g, Y_g) writes.  A decode step is short, so
 *   fewer launches matter.
 * x_bf16   DEVICE bf16 [M][K], 16-byte aligned.
 * n_group  1 .. MQ_MAX_GROUP.
 * w_bf16   HOST array of n_group DEVICE pointers, W_g bf16 [N_g][K], 16-byte
 *          aligned.
 * y_bf16   HOST array of n_group DEVICE pointers, Y_g bf16 [M][N_g].
 * N        HOST array of n_group row counts, each >= 1, at most 2^30 in all.
 * M        1..32.  K >= 16, K % 16 == 0.
 * flags    0.
 */
mq_status mq_gemv_bf16_decode_grouped(const void* x_bf16, int32_t n_group,
                                      const void* const* w_bf16,
                                      void* const* y_bf16, const int64_t* N,
                                      int64_t M, int64_t K, uint32_t flags,
                                      void* hip_stream);

/*
 * Producer ops with the amax pass folded in.  NVFP4's tensor scale of an
 * activation is taken from the absolute maximum of the whole tensor at run
 * time (gist.science explainer, Technical Summary s.2 Hybrid Precision
 * Strategy), which costs the quantizer a full read of the activation before
 * it can encode.  These two ops write the activations of an 8B-shaped
 * layer's prefill linears and, on the way out, one partial maximum of the
 * bf16 values stored per workgroup into rec (the layout the amax pass
 * writes: nparts, part[]); quantizing their output with MQ_SCALE_PARTIALS
 * then skips the amax pass and gives exactly the codes, scales and s_t of
 * the dynamic quantization of that output.  Outputs are bf16, rounded to
 * nearest-even from binary32 arithmetic.
 *
 * mq_rmsnorm_amax - y[r][c] = bf16(x[r][c] * rstd_r * g[c]),
 *   rstd_r = 1/sqrt(mean_c x[r][c]^2 + eps).
 * x_bf16, y_bf16  DEVICE bf16 [rows][cols], 16-byte aligned (y may not alias x).
 * gamma_bf16      DEVICE bf16 [cols], 16-byte aligned.
 * rec             DEVICE mq_scale_rec, 16-byte aligned; nparts and part[]
 *                 are overwritten (s_t and amax_bits are not touched).
 * rows >= 1; cols >= 16, cols % 16 == 0; eps finite, >= 0.  flags 0.
 */
mq_status mq_rmsnorm_amax(const void* x_bf16, const void* gamma_bf16, void* y_bf16,
                          mq_scale_rec* rec, int64_t rows, int64_t cols, float eps,
                          uint32_t flags, void* hip_stream);

/*
 * mq_rmsnorm_quantize_nvfp4 - out = NVFP4(RMSNorm(x) * gamma), the bf16
 *   output of the RMSNorm never stored.  For an RMSNorm whose output feeds
 *   only prefill linears (the q/k/v and gate/up inputs of a layer): the
 *   dynamic tensor scale of the quantizer (gist.science explainer, s.2
 *   Hybrid Precision Strategy) taken on the op's own output.  Two passes
 *   over x: the first takes y's partial maxima into out->rec without
 *   storing y, the second recomputes y and encodes it.  Codes, scale bytes
 *   and s_t are bit-identical to mq_rmsnorm_amax(x, gamma, y, out->rec, ...)
 *   followed by mq_quantize_nvfp4(y, out, MQ_SCALE_PARTIALS), and y is the
 *   same bf16 tensor mq_rmsnorm_amax writes.
 * x_bf16      DEVICE bf16 [rows][cols], 16-byte aligned.
 * gamma_bf16  DEVICE bf16 [cols], 16-byte aligned.
 * out         HOST pointer to caller-owned NVFP4 buffers [rows][cols]:
 *             codes 16-byte, scales 8-byte, rec 16-byte aligned (no
 *             initialisation needed).
 * rows, cols  >= 1; cols % 16 == 0.
 * eps         finite, >= 0.
 * flags       0.
 */
mq_status mq_rmsnorm_quantize_nvfp4(const void* x_bf16, const void* gamma_bf16, int64_t rows, int64_t cols,
                                    float eps, const mq_nvfp4* out, uint32_t flags, void* hip_stream);

/*
 * mq_swiglu_amax - y = bf16(silu(a) * b) elementwise, silu(a) = a/(1+exp(-a))
 *   (exp and the reciprocal from the hardware's approximate instructions).
 * a_bf16, b_bf16, y_bf16  DEVICE bf16 [rows][cols], 16-byte aligned (y may
 *                 not alias a or b).
 * rec, flags      as for mq_rmsnorm_amax.
 * rows >= 1; cols >= 16, cols % 16 == 0.
 */
mq_status mq_swiglu_amax(const void* a_bf16, const void* b_bf16, void* y_bf16,
                         mq_scale_rec* rec, int64_t rows, int64_t cols,
                         uint32_t flags, void* hip_stream);

/*
 * mq_gemv_nvfp4_decode - Y[M][N] = X[M][K] . W[N][K]^T with X and W in
 *   NVFP4: the decode step run the uniform way, in the prefill format, which
 *   the method avoids because decode errors accumulate (gist.science
 *   explainer, Technical Summary s.1 Problem Statement; s.4 Experimental
 *   Results).  Kept to compare the two decode paths on bytes moved: W is
 *   read at 0.5625 bytes per weight instead of 2.  Same arithmetic as
 *   mq_gemm_nvfp4_prefill (exact g*sigma operands, binary32 accumulation,
 *   times s_tX*s_tW, nearest-even bf16), summed in another order.
 * x        HOST pointer to the quantized rows X [M][K] (e.g. from
 *          mq_quantize_nvfp4 earlier on the same stream; rec->s_t set).
 * w        HOST pointer to the quantized weights [N][K] (rec->s_t set).
 * y_bf16   DEVICE bf16 [M][N].
 * M        1..32.  N >= 1.  K >= 16, K % 16 == 0 (K % 256 == 0 is fastest).
 *          codes 16-byte, scales 8-byte, rec 16-byte, y 2-byte aligned.
 * flags    0.
 */
mq_status mq_gemv_nvfp4_decode(const mq_nvfp4* x, const mq_nvfp4* w, void* y_bf16,
                               int64_t M, int64_t N, int64_t K,
                               uint32_t flags, void* hip_stream);

/*
 * Phase-aware linear layer.  The method keeps each weight matrix in two
 * formats and picks one per inference phase (gist.science English explainer,
 * s.2 Hybrid Precision Strategy: prefill in NVFP4 for weights and
 * activations, decode on the original BF16 weights; s.2 System-Level
 * Deployment: the two phases run on separate prefill and decode workers).
 * mq_linear holds both formats of one weight W [N][K]; a call names its
 * phase in its flags, or leaves it to the row count (decode steps carry one
 * row per sequence of the batch, prefills the prompt's tokens): calls with
 * M >= prefill_min_rows are taken as prefill.  The row threshold is this
 * library's reading; the pages name the phases, not a size.
 */
typedef struct mq_linear {
  const void* w_bf16;        /* DEVICE bf16 [N][K], 16-byte aligned: the
                                original weights (decode path)              */
  mq_nvfp4 w_nvfp4;          /* DEVICE NVFP4 copy of w_bf16 [N][K] (prefill
                                path), written by mq_linear_prepare          */
  int64_t N, K;              /* N >= 1; K >= 16, K % 16 == 0                */
  int64_t prefill_min_rows;  /* 1..33: rows at which a call without a phase
                                flag counts as prefill (33: every batch the
                                decode path supports stays on it)           */
} mq_linear;

#define MQ_PATH_DECODE_BF16   1  /* mq_gemv_bf16_decode on w_bf16              */
#define MQ_PATH_PREFILL_NVFP4 2  /* quantize X, mq_gemm_nvfp4_prefill on w_nvfp4 */

/*
 * mq_linear_path - the path a call with M rows and these flags takes:
 *   MQ_PHASE_PREFILL -> MQ_PATH_PREFILL_NVFP4; MQ_PHASE_DECODE ->
 *   MQ_PATH_DECODE_BF16 (M <= 32); neither -> by prefill_min_rows.
 *   Returns 0 for arguments mq_linear_forward would reject on that ground
 *   (L NULL, M < 1, both phase flags, a decode call with M > 32,
 *   prefill_min_rows outside 1..33).  Host only: no device work.
 */
int32_t mq_linear_path(const mq_linear* L, int64_t M, uint32_t flags);

/*
 * mq_linear_prepare - the offline step: quantize L->w_bf16 into L->w_nvfp4
 *   with its own tensor scale over the whole matrix (mq_quantize_nvfp4,
 *   dynamic).  Queued on hip_stream like every call; the NVFP4 copy is
 *   valid for calls queued after it on the same stream.
 */
mq_status mq_linear_prepare(const mq_linear* L, void* hip_stream);

/*
 * mq_linear_forward - Y[M][N] = X[M][K] . W^T through the call's phase.
 *   Decode (MQ_PATH_DECODE_BF16): mq_gemv_bf16_decode(x, L->w_bf16, y);
 *   M <= 32; a_work is not used (may be NULL); MQ_A_FUSED_BF16 is ignored.
 *   Prefill (MQ_PATH_PREFILL_NVFP4): X is quantized on the fly into a_work
 *   (mq_quantize_nvfp4, dynamic scale), then mq_gemm_nvfp4_prefill with
 *   L->w_nvfp4, bf16 output; with MQ_A_FUSED_BF16 the quantization runs in
 *   the GEMM's prologue instead (a_work->rec is still used; codes and scales
 *   may both be NULL, or both given: then the GEMM takes its quantize-once
 *   form and leaves X's NVFP4 in them, as mq_gemm_nvfp4_prefill describes).
 *   Each path's output is bit-identical to the direct calls it names.
 * L        HOST pointer; L->w_nvfp4 must hold mq_linear_prepare's result
 *          before a prefill call runs.
 * x_bf16   DEVICE bf16 [M][K], 16-byte aligned.
 * a_work   HOST pointer to caller-owned NVFP4 buffers for X [M][K] (codes
 *          16-byte, scales 8-byte, rec 16-byte aligned); prefill only.
 * y_bf16   DEVICE bf16 [M][N]; 16-byte aligned for prefill, 2 for decode.
 * flags    0, MQ_PHASE_PREFILL or MQ_PHASE_DECODE, optionally
 *          | MQ_A_FUSED_BF16, optionally | MQ_SCALE_PARTIALS (a_work->rec
 *          holds x's partial maxima; prefill path).
 * All arguments of the chosen path are checked before anything is queued.
 */
mq_status mq_linear_forward(const mq_linear* L, const void* x_bf16, int64_t M,
                            const mq_nvfp4* a_work, void* y_bf16,
                            uint32_t flags, void* hip_stream);

/*
 * mq_gemm_nvfp4_prefill_fused_noalloc - mq_gemm_nvfp4_prefill with
 *   MQ_A_FUSED_BF16 for callers that cannot allocate device memory (code
 *   under HIP graph capture, tight serving loops, harnesses that forbid
 *   hipMalloc): the activation's scale record and its NVFP4 copy live in a
 *   scratch buffer inside the library instead of caller buffers.  Same
 *   kernels and the same output, bit for bit, as
 *     mq_gemm_nvfp4_prefill(&a, a_bf16, w, c, M, N, K,
 *                           flags | MQ_A_FUSED_BF16, hip_stream)
 *   with a = caller-owned codes [M][K/2], scales [M][K/16] and a record.
 * a_bf16   DEVICE bf16 [M][K], 16-byte aligned.
 * w, c, N  as for mq_gemm_nvfp4_prefill.
 * M, K     M >= 1; K >= 16, K % 16 == 0; M * K <= MQ_NOALLOC_MAX_ELEMS,
 *          else MQ_ERR_SHAPE.
 * flags    MQ_OUT_BF16 or MQ_OUT_F32 (MQ_A_FUSED_BF16 is implied; the
 *          tensor scale is always dynamic).
 * The scratch buffer (MQ_NOALLOC_MAX_ELEMS * 9/16 bytes + 4 KB) is allocated
 * by the HIP runtime when the library's code is loaded on a device and held
 * until the process ends; the call itself allocates nothing.  Every call on
 * one device shares that device's buffer: calls that may run at the same
 * time on one device (different streams, or different threads without
 * ordering) race on it and must not be made.  Nothing in it needs clearing:
 * every byte a call reads was written earlier in the same call.
 */
#define MQ_NOALLOC_MAX_ELEMS 67108864 /* 2^26 */
mq_status mq_gemm_nvfp4_prefill_fused_noalloc(const void* a_bf16, const mq_nvfp4* w,
                                              void* c, int64_t M, int64_t N, int64_t K,
                                              uint32_t flags, void* hip_stream);

/* Static string naming a status code. */
const char* mq_status_str(mq_status s);

/* Thread-local detail of the last error returned on this thread ("" if none). */
const char* mq_last_error(void);

/* Library version string. */
const char* mq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MQ_H_ */
