/*
 * dg.h -- C ABI of the MI355X (gfx950) block-scaled FP8 GEMM library.
 *
 * Computes D = A . B^T in bf16 from e4m3 operands with fine-grained fp32
 * scales, and its two MoE grouped forms.  The operation is the one defined by
 * Lesson 13 "DeepSeek DeepGEMM core architecture and Hopper FP8 operator
 * breakdown" (hpc.payai.win), Fig. 13-1 and its closed-form equation:
 *
 *   D[i,j] = sum_g alpha[i,g] * beta[j/128, g] * sum_{k<128} A[i,128g+k] * B[j,128g+k]
 *
 * where each 128-wide K block's partial product is scaled by alpha*beta and
 * added into an fp32 accumulator inside the main loop, and the epilogue only
 * converts to bf16 (round to nearest even).  Layout is NT: A is [M,K] and B is
 * [N,K], both K-contiguous (DeepGEMM architecture deep dive, blog.123qwe.co.kr,
 * section 3, "D = A @ B.T").
 *
 * Conventions shared by every entry point
 *   - e4m3 means OCP FP8 E4M3FN (bias 7, max 448, 0x7F/0xFF NaN), passed as
 *     uint8_t bytes; bf16 is passed as uint16_t bit patterns.
 *   - Every array pointer is a DEVICE pointer owned by the caller; the library
 *     never allocates, frees or synchronises on these calls.  Pointers must be
 *     16-byte aligned (DG_ERR_ALIGN otherwise) except the scale, index and
 *     workspace arrays, which need 4-byte alignment.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on that stream and returns; the calls
 *     allocate nothing and never read device data on the host, so they may be
 *     captured into a hipGraph.  Kernel faults surface through the usual HIP
 *     stream error reporting.
 *   - Shapes are int64_t.  K must be a positive multiple of 128, N a positive
 *     multiple of 16, row counts >= 0 (0 rows = nothing to do, DG_OK).
 *   - Return value: DG_OK or one of the DG_ERR_* codes below; on error nothing
 *     is enqueued and dg_get_last_error() returns a message (thread-local).
 *   - Scale layouts: activation scales alpha are MN-major, [K/128][rows] fp32
 *     (per expert for the masked form); weight scales beta are
 *     [ceil(N/128)][K/128] fp32 per expert.  alpha = amax/448 over each 1x128
 *     row group; beta = amax/448 over each 128x128 block (Lesson 13,
 *     Fig. 13-1).
 *   - D rows that the operation does not define (padding rows of the
 *     contiguous form, rows past masked_m of the masked form) are never
 *     written.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Sizes: the kernels address one launch's activations, scales and
 *     outputs, and one expert's weights, with 32-bit byte offsets from 64-bit
 *     bases.  A call with more rows than that allows runs as several row
 *     chunks enqueued back to back on `stream` (each planned on its own; the
 *     results are those of one launch per chunk).  Rejected with DG_ERR_SHAPE:
 *     one expert's weights of 4 GiB or more ((N + 256) * K bytes, bf16: twice
 *     that), activation scales of 4 GiB or more, more than 1024 groups, and
 *     the K-grouped form past 32-bit offsets (see there).
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = 1, /* null pointer, bad enum value */
  DG_ERR_SHAPE = 2,       /* K % 128 (K % 64 for bf16), N % 16, negative sizes, G out of [1, 1024],
                             weights of 4 GiB or more per expert */
  DG_ERR_ALIGN = 3,       /* pointer alignment */
  DG_ERR_WORKSPACE = 4,   /* workspace pointer given with a size that is not a multiple of 4 */
  DG_ERR_DEVICE = 5,      /* no HIP device, or the current device is not gfx950 */
  DG_ERR_LAUNCH = 6       /* the kernel launch itself failed */
};

/* Operation ids for dg_get_workspace_size. */
enum {
  DG_OP_GEMM_NT = 0,
  DG_OP_CONTIGUOUS = 1,
  DG_OP_MASKED = 2,
  DG_OP_BF16_GEMM_NT = 3,
  DG_OP_GEMM_NT_UE8M0 = 4,
  DG_OP_K_GROUPED = 5 /* dg_k_grouped_fp8_gemm_nt_contiguous (plan description only) */
};

/*
 * Dense GEMM.  Lesson 13, Fig. 13-1; DeepGEMM's "normal" GEMM (the Feb-2025
 * release article on dakule.com, usage section).
 *   A   [M,K]  e4m3, row-major          sfa [K/128][M] fp32
 *   B   [N,K]  e4m3, row-major          sfb [ceil(N/128)][K/128] fp32
 *   D   [M,N]  bf16, row-major (written)
 * workspace: optional scratch for splitting K across workgroups when the
 *   output has too few tiles to fill the GPU (small M).  Pass NULL/0 to run
 *   without it (possibly slower; the split changes only the fp32 summation
 *   order, so results agree within rounding, and each configuration is
 *   deterministic).  Required size for the full split is
 *   dg_get_workspace_size(DG_OP_GEMM_NT, M, N, K, 1); a smaller buffer limits
 *   the split.  The workspace MUST be zero-filled before its first use (e.g.
 *   hipMemset once after allocation): whenever the plan splits K (the
 *   skinny kernel, at up to 2048 rows, or a partial last round of 256 x 128
 *   tiles) its first 4 KiB hold per-tile completion counters and the fp32
 *   partials follow; every call leaves the counters at zero again, so a workspace stays reusable across calls and
 *   shapes without clearing.  Calls that share one workspace must be ordered
 *   on one stream.
 */
int dg_fp8_gemm_nt(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb,
                   uint16_t* D, int64_t M, int64_t N, int64_t K, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Allocation-free dense GEMM, for callers that cannot allocate (code under
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * dg_fp8_gemm_nt with no workspace argument.  Same operands, result and plan
 * as dg_fp8_gemm_nt given a workspace of dg_get_workspace_size(DG_OP_GEMM_NT,
 * M, N, K, 1) bytes (so the outputs are bit-identical); the K-split partials
 * and counters live in a static device array of 40 MiB that every GPU the
 * library runs on holds until the process ends.  Shapes whose split-K scratch
 * would exceed 40 MiB return DG_ERR_WORKSPACE (none does under the default
 * plans on 256 CUs).  Nothing is allocated; the first call on a device
 * resolves the array's address and clears its counter area with a small
 * kernel on `stream`.  Calls that overlap on one GPU (other streams, other
 * threads, concurrent graph replays) share the array and race: order them.
 */
int dg_fp8_gemm_nt_noalloc(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb,
                           uint16_t* D, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * M-grouped contiguous GEMM (MoE training forward / prefill).  Lesson 13,
 * Fig. 13-3 (contiguous layout); deep-dive blog section 3 (grouped API table,
 * per-expert segments aligned to the M block).
 *   A         [M_total,K] e4m3, rows of all experts concatenated
 *   sfa       [K/128][M_total] fp32
 *   B         [G,N,K] e4m3 (one weight per expert, same N and K for all)
 *   sfb       [G][ceil(N/128)][K/128] fp32
 *   m_indices [M_total] int32, device: expert of each row; a value outside
 *             [0,G) marks a padding row, whose D row is not written
 *   D         [M_total,N] bf16
 * Each aligned block of dg_get_m_alignment_for_contiguous_layout() rows must
 * hold rows of at most one expert (segments padded to that alignment); rows
 * of a block whose index differs from the block's expert are not written.
 * G must be in [1, 1024]; each expert's weights are addressed from the
 * expert's own base.  workspace: unused, pass NULL/0.
 */
int dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* A, const float* sfa, const uint8_t* B,
                                        const float* sfb, uint16_t* D, const int32_t* m_indices,
                                        int64_t M_total, int64_t N, int64_t K, int64_t G,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * M-grouped masked GEMM (MoE decode under graph capture).  Lesson 13,
 * Fig. 13-3 (masked layout) and the answer to Q3: fixed-capacity buffers per
 * expert and a device array of valid row counts read by the kernel, so the
 * launch never depends on host knowledge of the counts.
 *   A        [G,max_m,K] e4m3             sfa [G][K/128][max_m] fp32
 *   B        [G,N,K] e4m3                 sfb [G][ceil(N/128)][K/128] fp32
 *   masked_m [G] int32, device: expert g's rows [0, clamp(masked_m[g],0,max_m))
 *            are computed; all other rows of D are not written
 *   D        [G,max_m,N] bf16
 * G must be in [1, 1024]; each expert's A, alpha, weights and D are
 * addressed from the expert's own base, so one expert's rows must fit 32-bit
 * offsets ((max_m + 256) * K and max_m * N * 2 bytes below 4 GiB).
 * expected_m: host hint of the typical masked_m (0 = unknown); it is not
 *   used (the launch shape and the results never depend on it).
 * workspace: unused, pass NULL/0.
 */
int dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* A, const float* sfa, const uint8_t* B,
                                    const float* sfb, uint16_t* D, const int32_t* masked_m,
                                    int64_t G, int64_t max_m, int64_t N, int64_t K,
                                    int64_t expected_m, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * Accumulating dense GEMM, D = C + A . B^T in fp32.  Deep-dive blog, section 3:
 * every GEMM of the library has the form D = C + A @ B (NT: A @ B^T).
 *   A, sfa, B, sfb as for dg_fp8_gemm_nt
 *   C [M,N] fp32, row-major, or NULL (read as zeros); may equal D (in place)
 *   D [M,N] fp32, row-major (written)
 * D = fl32(C + acc): the fp32 accumulator of the promoted GEMM plus C, rounded
 * once.  workspace as for dg_fp8_gemm_nt (same size query, DG_OP_GEMM_NT,
 * which covers both forms).
 */
int dg_fp8_gemm_nt_acc(const uint8_t* A, const float* sfa, const uint8_t* B, const float* sfb,
                       const float* C, float* D, int64_t M, int64_t N, int64_t K, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * K-grouped contiguous GEMM (MoE weight gradient), D[g] = C[g] + A_g . B_g^T
 * in fp32.  Deep-dive blog, section 3: the K-grouped contiguous family groups
 * along K with M and N fixed and serves the backward pass of MoE weights;
 * every GEMM there has the form D = C + A @ B, and contiguous segments are
 * aligned to the block size (M and K).  Group g owns the K range that starts
 * after the first g segments: A_g = A[:, seg g], B_g = B[:, seg g].
 *   A   [M,K] e4m3, row-major (K = the sum of the segments, e.g. tokens)
 *   sfa [K/128][M] fp32: one scale per row per 128 K (1x128, Lesson 13 Fig. 13-1)
 *   B   [N,K] e4m3, row-major
 *   sfb [K/128][N] fp32: also per row per 128 K (both operands are activations)
 *   ks  [G] int32, device: K length of each group, a multiple of 128 (zero
 *       allowed).  Read by the kernel: group g covers K blocks
 *       [sum_{h<g} floor(ks[h]/128), + floor(ks[g]/128)), negative lengths
 *       count as 0 and blocks past K/128 are dropped; K positions after the
 *       last segment belong to no group.
 *   C   [G,M,N] fp32 or NULL (zeros); may equal D (in place)
 *   D   [G,M,N] fp32 (written, every group; a group without K blocks gets C[g])
 * D[g] = fl32(C[g] + acc_g), acc_g the fp32 accumulator of the promoted
 * products over the group's blocks.  G must be in [1, 1024]; problems whose
 * A, B or per-group D byte offsets exceed 32 bits are rejected with
 * DG_ERR_SHAPE.  workspace: unused, pass NULL/0.
 */
int dg_k_grouped_fp8_gemm_nt_contiguous(const uint8_t* A, const float* sfa, const uint8_t* B,
                                        const float* sfb, const float* C, float* D,
                                        const int32_t* ks, int64_t G, int64_t M, int64_t N,
                                        int64_t K, void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * BF16 dense GEMM, D = A . B^T, no scales.  BF16 is among the library's
 * precisions (deep-dive blog, section 1 overview table); the Ascend 950
 * article (benchmarks section) measures this GEMM at M=4096, N=7168, K=16384.
 *   A [M,K] bf16, row-major      B [N,K] bf16, row-major
 *   D [M,N] bf16, row-major (written); fp32 accumulation, round-to-nearest-even
 * K must be a multiple of 64, N of 16.  workspace: as for dg_fp8_gemm_nt
 * (optional, lets a partial last round of tiles split along K; size from
 * dg_get_workspace_size(DG_OP_BF16_GEMM_NT, M, N, K, 1); zero-filled before
 * first use, left reusable).
 */
int dg_bf16_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* D, int64_t M, int64_t N, int64_t K,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * 1x128 activation quantiser.  Lesson 13, Fig. 13-1 (one scale per token per
 * 128 K elements, scale = amax/448).
 *   x   [G,M,K] fp32 (G=1 for a plain [M,K] matrix)
 *   q   [G,M,K] e4m3 (written)
 *   sfa [G][K/128][M] fp32 (written)
 * alpha = fl32(amax / 448) by IEEE division; q = e4m3_RNE(fl32(x / alpha)),
 * ties to even, sign of zero kept, saturating at +-448; a group with amax = 0
 * (or amax/448 underflowing to 0) gets alpha = 1.  Non-finite inputs give
 * unspecified codes.  Bit-exact and deterministic.  Limits: G <= 65535,
 * M <= 2^31 - 16 and ceil(M / 16) * (K / 128) < 2^31 (else DG_ERR_SHAPE); x and q 16-byte
 * aligned, sfa 4-byte aligned (else DG_ERR_ALIGN).
 */
int dg_quant_1x128(const float* x, uint8_t* q, float* sfa, int64_t G, int64_t M, int64_t K,
                   void* stream);

/*
 * 128x128 weight quantiser.  Lesson 13, Fig. 13-1 (one scale per 128x128
 * block of the weight, stored fp32).
 *   x   [G,N,K] fp32       q [G,N,K] e4m3 (written)
 *   sfb [G][ceil(N/128)][K/128] fp32 (written)
 * Same rounding rules as dg_quant_1x128; when N is not a multiple of 128 the
 * last block's amax covers only its existing rows.
 */
int dg_quant_128x128(const float* x, uint8_t* q, float* sfb, int64_t G, int64_t N, int64_t K,
                     void* stream);

/*
 * UE8M0 (power-of-two) scale variant.  Lesson 13 (the notes after Fig. 13-1):
 * newer library versions accept UE8M0 scales besides fp32; deep-dive blog,
 * section 3: on the newer architecture four UE8M0 scales are packed into one
 * 32-bit integer.  Same granularity and per-128-K promotion as the fp32 form.
 * A code c means 2^(c - 127); codes of four consecutive K blocks share one
 * int32, block 4w + j in byte j (bits 8j..8j+7), unused bytes zero.
 *   sfa [ceil(K/512)][M] int32 (MN-major, as the fp32 layout)
 *   sfb [ceil(N/128)][ceil(K/512)] int32
 * The quantisers choose c so that 2^(c-127) is the smallest power of two not
 * below amax/448 (clamped to codes [0, 254]; an all-zero group gets 127) and
 * write q = e4m3_RNE(x * 2^(127-c)), an exact power-of-two scaling.
 * dg_fp8_gemm_nt_ue8m0: D [M,N] bf16 = A . B^T with those scales; the matrix
 * cores apply the scales and add each K block's product to the fp32
 * accumulator, rounded once.  workspace as for dg_fp8_gemm_nt (size from
 * dg_get_workspace_size(DG_OP_GEMM_NT_UE8M0, M, N, K, 1)).
 */
int dg_quant_1x128_ue8m0(const float* x, uint8_t* q, int32_t* sfa, int64_t G, int64_t M, int64_t K,
                         void* stream);
int dg_quant_128x128_ue8m0(const float* x, uint8_t* q, int32_t* sfb, int64_t G, int64_t N, int64_t K,
                           void* stream);
int dg_fp8_gemm_nt_ue8m0(const uint8_t* A, const int32_t* sfa, const uint8_t* B, const int32_t* sfb,
                         uint16_t* D, int64_t M, int64_t N, int64_t K, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * M-grouped contiguous and masked GEMMs with UE8M0 scales (the grouped forms
 * of dg_fp8_gemm_nt_ue8m0; deep-dive blog, section 3: the grouped GEMMs take
 * the scale formats of the plain ones).  Operands, index arrays, outputs and
 * rules as for dg_m_grouped_fp8_gemm_nt_contiguous / _masked, with packed
 * int32 scales (four K blocks per word, block 4w + j in byte j):
 *   contiguous: sfa [ceil(K/512)][M_total], sfb [G][ceil(N/128)][ceil(K/512)]
 *   masked:     sfa [G][ceil(K/512)][max_m], sfb [G][ceil(N/128)][ceil(K/512)]
 * (dg_quant_1x128_ue8m0 with G groups writes the masked activation layout,
 * dg_quant_128x128_ue8m0 with G experts the weight layout).
 */
int dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const uint8_t* A, const int32_t* sfa, const uint8_t* B,
                                              const int32_t* sfb, uint16_t* D, const int32_t* m_indices,
                                              int64_t M_total, int64_t N, int64_t K, int64_t G,
                                              void* workspace, size_t workspace_bytes, void* stream);
int dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const uint8_t* A, const int32_t* sfa, const uint8_t* B,
                                          const int32_t* sfb, uint16_t* D, const int32_t* masked_m,
                                          int64_t G, int64_t max_m, int64_t N, int64_t K, int64_t expected_m,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes that let `op` use its full K split for this shape with the
 * current CU cap (0 = none used); a call split into row chunks reuses it for
 * every chunk. */
size_t dg_get_workspace_size(int op, int64_t rows, int64_t N, int64_t K, int64_t G);

/* Text description of the launch plan the library would use for `op` at this
 * shape on the current device with a full workspace, e.g. "kernel=wide
 * tile=256x256 grid=256 tiles=448 whole=448 tail=0x1" (DG_OP_GEMM_NT,
 * DG_OP_GEMM_NT_UE8M0, DG_OP_BF16_GEMM_NT, DG_OP_CONTIGUOUS with rows = M_total
 * and G the expert count, DG_OP_K_GROUPED with rows = M, G the group count
 * and K the total K, and DG_OP_MASKED with rows = max_m and G the expert
 * count, whose task count depends on masked_m and is given as its maximum;
 * "" for invalid shapes); for a call split into row chunks it describes the
 * first chunk and ends in "chunks=n".  "weights=nt" marks plans whose weight
 * loads carry the non-temporal cache policy (each weight line read by one
 * workgroup: dense calls with M <= 64, masked calls with max_m <= 128).
 * The pointer stays valid until the next call on the same thread.
 * Debugging aids, read from the environment on every call:
 *   DG_FORCE_CONFIG   comma-separated; "kernel=wide" / "kernel=persistent"
 *                     force the 256x256 or the 256x128 (128x256 grouped) tile
 *                     kernel wherever the planner chooses between them, and
 *                     "chunk_rows=<n>" splits calls into row chunks of at
 *                     most n rows (rounded down to a multiple of 256, at
 *                     least 256), and "skinny=<bm>x<wn>x<s>x<p>" makes calls
 *                     with at most 2048 rows use bm-row tiles (64 or 128) of
 *                     4 wn columns (wn 16 or 32), a K split of s (bounded by
 *                     the K blocks and the workspace) and ring depth p (one
 *                     of the compiled depths; other values are ignored);
 *                     results stay within the same bounds
 *   DG_PRINT_CONFIGS  print every launch's plan on stderr
 *   DG_CHECK_LAYOUT   the contiguous forms copy m_indices to the host
 *                     (synchronising the stream; skipped while the stream is
 *                     being captured) and reject, with DG_ERR_INVALID_ARG, a
 *                     layout whose aligned 128-row block holds rows of two
 *                     experts */
const char* dg_describe_plan(int op, int64_t rows, int64_t N, int64_t K, int64_t G);

/* Row alignment of expert segments in the contiguous layout (deep-dive blog,
 * section 3: contiguous segments aligned to the M block).  Always 128. */
int dg_get_m_alignment_for_contiguous_layout(void);

/* Cap on the number of compute units the kernels plan for (analog of the
 * "set max SM count" utility in the Feb-2025 release article).  n <= 0 resets
 * to the device's count.  Process-wide; returns DG_OK. */
int dg_set_num_cus(int n);
/* Current cap (the device's CU count when no cap is set; 0 if no device). */
int dg_get_num_cus(void);

/* Message of the last error on this thread ("" if none). */
const char* dg_get_last_error(void);
/* Library version string. */
const char* dg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
