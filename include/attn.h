/*
 * attn.h - exact attention forward on AMD Instinct MI355X (gfx950).
 *
 * The operation (all entry points):
 *
 *     O   = softmax(scale * Q K^T + mask) V
 *     LSE = per query row, ln( sum_j exp(scale * q_i . k_j + mask_ij) )
 *
 * where mask_ij is 0 for a visible key and -inf otherwise.  This is the
 * attention of "Flash Attention và IO" (aihero.vn): each query row is compared
 * with the keys, the scores are normalised with a softmax, and the values are
 * summed with those weights.  The kernels compute it tile by tile with the
 * running-statistics softmax of that page's section "Softmax qua nhiều khối cần
 * thống kê chạy" (running maximum m, normaliser l, weighted sum u; the result
 * is u / l), so the N x N score and probability matrices never reach device
 * memory.  The page's section "Tiling giữ công việc ở gần nơi tính" makes the
 * result exact: it differs from the plain definition only by floating-point
 * evaluation order.  Loop order and sequence-level parallelism follow the
 * FlashAttention-2 part of "FlashAttention, pelatihan multi-GPU, dan
 * kuantisasi bobot", section 1 (Q blocks outer, K/V blocks inner, one
 * normalisation at the end).
 *
 * Masks
 *   causal = 0   every key of the sequence is visible.
 *   causal = 1   key j is visible to query i iff j <= i (the same sequence
 *                length for queries and keys, aligned at the first token).
 *   cu_seqlens   packed documents: a query sees only keys of its own document
 *                (combined with the causal rule inside the document when
 *                causal = 1).  Packed layouts follow the document-local,
 *                no-repacking design of "FLAMIA: Blackwell Üzerinde Hızlı ve
 *                Nedensel Olarak Güvenli Eğitim İçin Flash Mikro-Ölçeklemeli
 *                Dikkat Mekanizması", section "FLAMIA Mimarisi ve Temel
 *                Tasarım İlkeleri".
 *
 * Layouts (row-major, contiguous, element strides implied by the sizes)
 *   fixed length (cu_seqlens == NULL):
 *     q, k, v, o : [B][N][H][d]          lse : [B][H][N]  (fp32)
 *   packed (cu_seqlens != NULL):  B = number of documents, N = total tokens
 *     q, k, v, o : [N][H][d]             lse : [H][N]     (fp32)
 *     cu_seqlens : B + 1 int32 prefix offsets in DEVICE memory,
 *                  cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] = N.
 *
 * Supported set
 *   d in {64, 128}; B, H, N >= 1; B * H * N < 2^31 (elements per tensor
 *   < 2^31 * d); scale finite (any sign, zero allowed).
 *   attn_fwd:     bf16 q/k/v; o bf16 (ATTN_BF16) or fp32 (ATTN_BF16_OUT_F32).
 *   attn_fwd_fp8: e4m3 q/k/v with per-128-token block scales, o bf16, d = 128,
 *                 fixed length or packed documents.
 *   attn_quantize_fp8: bf16 -> e4m3 with those block scales, d in {64, 128}.
 *   attn_quantize_fp8_rotated: the same after a random-sign Hadamard rotation.
 *   attn_quantize_mxfp8: bf16 -> MXFP8 (E8M0 scale per 32 elements), d in {64, 128}.
 *   attn_fwd_mxfp8: MXFP8 q/k/v, o bf16, d = 128, fixed length or packed documents.
 *   attn_bwd:     bf16 gradients of attn_fwd (bf16 output), d in {64, 128}.
 *   Anything else returns an error; there is no fallback path.
 *   Range: the forward kernels weigh keys against a reference maximum that
 *   moves only when a tile's weights for a query sum past 2^64, so the
 *   running sums l and u stay finite while N * max|v| < 2^68 (N the sequence
 *   or document length, v the dequantised values).  Beyond that O may
 *   overflow to inf or NaN although the exact result is finite.
 *   fp8 / MXFP8 scores: dequantised Q and K values must be 0 or lie within
 *   bf16's normal range (2^-126 <= |x| < 2^128); the scores are formed from
 *   them as bf16 numbers.
 *
 * Ownership and concurrency
 *   Every pointer is device memory owned by the caller (except that `stream`
 *   is a HIP stream handle, NULL for the null stream).  The library allocates
 *   nothing, keeps no pointer after returning, has no mutable global state
 *   (except the fixed scratch of attn_bwd_noalloc and its cached per-device
 *   address) and may be called from several threads at once.  Every pointer must be
 *   16-byte aligned.  Inputs are never written; o and lse are fully
 *   overwritten.
 *
 * Errors
 *   The return value is an attn_status.  A nonzero status means nothing was
 *   enqueued and the outputs are untouched, except ATTN_ERR_HIP, which reports
 *   a failed launch (the HIP error of the launch).  Calls return as soon as the
 *   work is enqueued on `stream`; device-side problems (including invalid
 *   cu_seqlens contents, which the host never reads) show at the caller's
 *   next synchronisation and leave the outputs undefined.
 */
#ifndef IAEA_ATTN_H
#define IAEA_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_API __attribute__((visibility("default")))

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,         /* a required pointer is NULL                         */
    ATTN_ERR_SHAPE = 2,        /* B, H or N < 1, or the tensors are too large        */
                               /* (B*N*H >= 2^31; bf16: H*d > 2^24)                  */
    ATTN_ERR_UNSUPPORTED = 3,  /* d, dtype or causal flag not supported              */
    ATTN_ERR_SCALE = 4,        /* scale is NaN or infinite                           */
    ATTN_ERR_ALIGN = 5,        /* a pointer is not 16-byte aligned                   */
    ATTN_ERR_HIP = 6,          /* the kernel launch failed                           */
    ATTN_ERR_SCRATCH = 7       /* attn_bwd_noalloc: more rows than its fixed scratch */
} attn_status;

typedef enum {
    ATTN_BF16 = 0,             /* bf16 q/k/v, bf16 o (round to nearest even)         */
    ATTN_BF16_OUT_F32 = 1,     /* bf16 q/k/v, fp32 o                                 */
    ATTN_FP8_E4M3 = 2          /* e4m3 operands: use attn_fwd_fp8 (attn_fwd rejects) */
} attn_dtype;

/*
 * attn_fwd - bf16 exact attention forward.
 *   q, k, v     bf16 inputs, layout above.
 *   o           output, bf16 or fp32 per `dtype`, layout above.
 *   lse         fp32 per-row log-sum-exp (natural log, of the scaled and
 *               masked scores), layout above.
 *   B, H, N, d  sizes (packed: B documents, N total tokens).
 *   scale       multiplies q . k before the softmax (for example 1/sqrt(d)).
 *   causal      0 or 1.
 *   cu_seqlens  NULL for fixed length; else device int32[B + 1] (packed).
 *   dtype       ATTN_BF16 or ATTN_BF16_OUT_F32.
 *   stream      HIP stream (hipStream_t) to enqueue on.
 */
ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal,
                      const int32_t* cu_seqlens, int dtype, void* stream);

/*
 * attn_fwd_fp8 - block-scaled fp8 exact attention forward (d = 128).  The FP8
 * path with per-tile scales follows the FlashAttention-3
 * part of "FlashAttention, pelatihan multi-GPU, dan kuantisasi bobot",
 * section 1 (block quantisation: each tile carries its own scale); the scale
 * blocks never mix tokens of different 128-token blocks, the causal-leakage
 * concern of the FLAMIA page (sections "Uzun Bağlamlarda Dikkat (Attention)
 * Maliyeti ve Blackwell Mimarisi" and "FLAMIA Mimarisi ve Temel Tasarım
 * İlkeleri").
 *   q, k, v     OCP e4m3 ("e4m3fn") bytes, [B][N][H][128] (packed [N][H][128]).
 *   q_scale, k_scale, v_scale
 *               fixed length: fp32 [B][H][ceil(N / 128)]; token t of (b, h)
 *               has the value e4m3(byte) * scale[b][h][t / 128].
 *               packed: fp32 [H][ceil(N / 128) + B]; the 128-token blocks
 *               restart at every document's first token, and token
 *               cu_seqlens[b] + t of document b (0 <= t < its length) has the
 *               value e4m3(byte) * scale[h][cu_seqlens[b] / 128 + b + t / 128].
 *               Distinct blocks have distinct slots; other slots are not read.
 *               attn_quantize_fp8 writes both layouts.
 *   o           bf16 [B][N][H][128] (packed [N][H][128]);  lse fp32 [B][H][N]
 *               (packed [H][N]).
 *   The scores are formed on the bf16 matrix instruction from the e4m3
 *   values converted to bf16 (exact), with fp32 accumulation; the fp8 matrix
 *   instruction truncates its partial sums too coarsely for them (see
 *   attn_fwd_fp8.hip).  The probabilities P enter the P.V contraction as
 *   e4m3, on the fp8 matrix instruction, with one power-of-two scale 2^E per
 *   query row and 64-key tile, E the smallest integer with the row's weights
 *   in that tile summing to less than 2^E (weights of masked keys are 0, so a
 *   scale never depends on keys the row may not see).  P is carried as two
 *   e4m3 terms, P ~ hi + lo with hi = e4m3(P * 2^(8-E)) * 2^(E-8) and
 *   lo = e4m3((P - hi) * 2^(13-E)) * 2^(E-13), each rounded to nearest:
 *   about 8 significant bits, as bf16.  The normaliser l is summed from the
 *   unquantised fp32 P.  Scales must be
 *   positive, finite and normal.
 *   Other arguments as attn_fwd.  H * d must not exceed 2^24 (ATTN_ERR_SHAPE).
 */
ATTN_API int attn_fwd_fp8(const void* q, const void* k, const void* v,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          void* o, float* lse, int B, int H, int N, int d, float scale,
                          int causal, const int32_t* cu_seqlens, void* stream);

/*
 * attn_bwd - bf16 exact attention backward: the gradients dQ, dK, dV of
 * O = softmax(scale * Q K^T + mask) V for an upstream gradient dO, from the
 * forward's saved LSE (no N x N matrix is stored; probabilities are formed
 * again tile by tile).  "Flash Attention và IO" asks for the backward pass to
 * be measured beside the forward when training (section "Kernel đúng còn phải
 * hợp với tải") and for gradients to be compared across implementations
 * (section "Bài tập kiểm tính đúng trước khi đo tốc độ"); the pages print no
 * backward formulas, so the kernels compute the derivative of the forward:
 *     P_ij = exp(scale q_i . k_j - LSE_i) (0 for a masked key),
 *     D_i = dO_i . O_i,  dV_j = sum_i P_ij dO_i,
 *     dS_ij = P_ij (dO_i . v_j - D_i),
 *     dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
 *   q, k, v     bf16, as given to attn_fwd (same layout, B, H, N, d, scale,
 *               causal and cu_seqlens).
 *   o, lse      attn_fwd's bf16 output and fp32 LSE for those inputs.
 *   dout        bf16 dO, layout of o.
 *   delta       fp32 workspace with the layout of lse, owned by the caller;
 *               on return it holds D (rowsum of dO * O).
 *   dq, dk, dv  bf16 outputs, layout of q; fully overwritten.  None of them
 *               may alias an input, delta or each other (other workgroups are
 *               still reading the inputs while a gradient row is written).
 *   d in {64, 128}.  Errors as attn_fwd.  The two kernels are enqueued on
 *   `stream` in order: dQ (which also writes D), then dK and dV.
 */
ATTN_API int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* delta, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, float scale, int causal,
                      const int32_t* cu_seqlens, void* stream);

/*
 * attn_bwd_noalloc - attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, bit for bit, without the `delta`
 * argument.  D per row goes to a fixed scratch array that the library keeps
 * in each GPU's memory until the process ends (2^21 floats, 8 MiB per GPU);
 * its device address is looked up once per device, on the first call made
 * with that device current.  The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine) and reads nothing a previous call
 * left in the scratch (D is written before it is read).
 *   Arguments as attn_bwd, without delta.
 *   Rows of D - B * H * N (fixed length) or H * N (packed) - must not exceed
 *   2^21 (ATTN_ERR_SCRATCH otherwise; nothing is enqueued).
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap
 *   on one GPU (different streams, or several threads) race and give
 *   undefined results; serialise them, or use attn_bwd with a delta buffer
 *   each.  The current device must be the one `stream` belongs to.
 *   Errors as attn_bwd, plus ATTN_ERR_SCRATCH, and ATTN_ERR_HIP when the
 *   scratch's address cannot be obtained.
 */
ATTN_API int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv,
                              int B, int H, int N, int d, float scale, int causal,
                              const int32_t* cu_seqlens, void* stream);

/*
 * attn_fwd_mxfp8 - exact attention forward on MXFP8 operands (d = 128), the
 * micro-scaled FP8 path of FLAMIA ("FLAMIA: Blackwell Üzerinde Hızlı ve
 * Nedensel Olarak Güvenli Eğitim İçin Flash Mikro-Ölçeklemeli Dikkat
 * Mekanizması", section "FLAMIA Mimarisi ve Temel Tasarım İlkeleri"), with the
 * attention itself as attn_fwd.  Operands as attn_quantize_mxfp8 writes them:
 *   q, k        e4m3 bytes [B][N][H][128] (packed [N][H][128]), with
 *   q_scale, k_scale   E8M0 bytes [B][N][H][4] (packed [N][H][4]): element d
 *               of a token and head is e4m3(byte) * 2^(scale[d / 32] - 127).
 *               Each scale depends on its own token only.
 *   v           e4m3 bytes, same layout, with
 *   v_scale     E8M0 bytes [B][H][ceil(N / 32)][128] (packed [H][ceil(N / 32)
 *               + B][128], document-local blocks as attn_quantize_mxfp8):
 *               token t, coordinate d is e4m3(byte) * 2^(v_scale[t / 32][d] -
 *               127).  A V scale can depend on later tokens of its own
 *               32-token block, never on another block.
 *   Scale bytes must not be 0xFF (the format's NaN); slots no block maps to
 *   are never read.  o, lse, B, H, N, scale, causal, cu_seqlens, stream as
 *   attn_fwd_fp8.  P enters P.V as two e4m3 terms with a power of two per
 *   query and 32-key block.
 *   Errors as attn_fwd_fp8.
 */
ATTN_API int attn_fwd_mxfp8(const void* q, const void* k, const void* v, const uint8_t* q_scale,
                            const uint8_t* k_scale, const uint8_t* v_scale, void* o, float* lse, int B, int H,
                            int N, int d, float scale, int causal, const int32_t* cu_seqlens, void* stream);

/*
 * attn_quantize_fp8 - block-scaled e4m3 quantisation of a bf16 tensor, the
 * step upstream of attn_fwd_fp8: the per-tile scales of the FlashAttention-3
 * part of "FlashAttention, pelatihan multi-GPU, dan kuantisasi bobot"
 * (section 1), with no scale spanning two 128-token blocks or two documents
 * (the FLAMIA page, sections "Uzun Bağlamlarda Dikkat (Attention) Maliyeti ve
 * Blackwell Mimarisi" and "FLAMIA Mimarisi ve Temel Tasarım İlkeleri").  For
 * every block (up to 128 consecutive tokens of one sequence or document and
 * one head, all d):
 *     s = amax / 448 in fp32 (s = 1 when the block is all zero),
 *     y = e4m3(x / s): x / s rounded to fp32, then to the nearest e4m3 value
 *         (ties to the even mantissa; 448 is the largest).
 *   x           bf16 [B][N][H][d] (packed [N][H][d]), finite.
 *   y           e4m3 bytes, same layout; fully overwritten.
 *   scales      fp32 [B][H][ceil(N / 128)] (packed [H][ceil(N / 128) + B]),
 *               the layouts attn_fwd_fp8 reads; packed slots that no block
 *               maps to are left untouched.
 *   B, H, N, d  sizes as attn_fwd; d in {64, 128}.
 *   cu_seqlens  NULL, or device int32[B + 1] (packed documents).
 *   stream      HIP stream to enqueue on.
 *   Errors as attn_fwd (ATTN_ERR_NULL, _SHAPE, _UNSUPPORTED for d, _ALIGN
 *   for pointers not 16-byte aligned, _HIP).
 */
ATTN_API int attn_quantize_fp8(const void* x, void* y, float* scales, int B, int H, int N, int d,
                               const int32_t* cu_seqlens, void* stream);

/*
 * attn_quantize_fp8_rotated - incoherent processing before the block
 * quantisation: the FlashAttention-3 part of "FlashAttention, pelatihan
 * multi-GPU, dan kuantisasi bobot" (section 1) multiplies Q and K by a random
 * orthogonal matrix so that outliers are spread before fp8 rounding.  Each
 * row x (one token, one head, d coordinates) becomes
 *     z = x diag(signs) H_d,
 * H_d the Sylvester Hadamard matrix (entry (i, j) = (-1)^popcount(i & j)),
 * unnormalised: diag(signs) H_d times its transpose is d I, so
 * (Q M)(K M)^T = d Q K^T and attention on the rotated operands takes
 * scale / d.  z is the exact signed sum rounded once to fp32 (exact whenever
 * the nonzero entries of a row span at most 38 binades of exponent; beyond
 * that the fp64 sum may be rounded before the fp32 rounding).  z then goes
 * through the block quantisation of attn_quantize_fp8 (amax of |z| per
 * block, s = amax / 448, e4m3(z / s)).  Rotate Q and K with the same signs;
 * V is quantised unrotated (attn_quantize_fp8).
 *   x, y, scales, B, H, N, d, cu_seqlens, stream
 *               as attn_quantize_fp8 (x finite, |x| < 2^119 so that sums of d
 *               values stay finite in fp32).
 *   signs       device int8[d], 16-byte aligned: coordinate i is negated when
 *               signs[i] < 0 (so +1 / -1 as drawn; any other value counts by
 *               its sign).  Read only.
 *   Errors as attn_quantize_fp8, plus ATTN_ERR_NULL / _ALIGN for signs.
 */
ATTN_API int attn_quantize_fp8_rotated(const void* x, void* y, float* scales, const int8_t* signs, int B, int H,
                                       int N, int d, const int32_t* cu_seqlens, void* stream);

/*
 * attn_quantize_mxfp8 - MXFP8 quantisation of a bf16 tensor: e4m3 elements
 * with one power-of-two scale per block of 32 elements, stored as an E8M0
 * byte (exponent + 127).  FLAMIA ("FLAMIA: Blackwell Üzerinde Hızlı ve
 * Nedensel Olarak Güvenli Eğitim İçin Flash Mikro-Ölçeklemeli Dikkat
 * Mekanizması", section "FLAMIA Mimarisi ve Temel Tasarım İlkeleri") runs
 * attention on MXFP8 operands.  For a block with maximum magnitude amax:
 *     e = floor(log2 amax) - 8, clamped to [-127, 127] (e = 0 if all zero),
 *     byte = e4m3(x / 2^e), nearest with ties to even, clamped to +-448.
 *   along_tokens = 0 (Q and K): blocks are 32 consecutive coordinates of one
 *               token and head; scales uint8 [B][N][H][d / 32] (packed
 *               [N][H][d / 32]); cu_seqlens is accepted and not used (these
 *               blocks never cross a token).
 *   along_tokens = 1 (V): blocks are 32 consecutive tokens of one head and
 *               coordinate; scales uint8 [B][H][ceil(N / 32)][d], block k of
 *               (b, h) covering tokens 32k .. 32k + 31; packed:
 *               [H][ceil(N / 32) + B][d], blocks restarting at each document's
 *               first token, block k of document j in slot cu[j] / 32 + j + k
 *               (slots no block maps to are left untouched).
 *   x, y, B, H, N, d, cu_seqlens, stream
 *               as attn_quantize_fp8 (x finite; y fully overwritten).
 *   Errors as attn_quantize_fp8, plus ATTN_ERR_UNSUPPORTED for along_tokens
 *   other than 0 or 1.
 */
ATTN_API int attn_quantize_mxfp8(const void* x, void* y, uint8_t* scales, int B, int H, int N, int d,
                                 const int32_t* cu_seqlens, int along_tokens, void* stream);

/* attn_status_str - static, NUL-terminated description of a status code
 * (unknown codes give "unknown status").  Never NULL; do not free. */
ATTN_API const char* attn_status_str(int status);

/* attn_kernel_name - static name of the kernel attn_fwd / attn_fwd_fp8 would
 * launch for these arguments ("" when the arguments are not supported), so a
 * caller can confirm which code path runs.  fp8 = 1 selects attn_fwd_fp8,
 * fp8 = 2 attn_fwd_mxfp8. */
ATTN_API const char* attn_kernel_name(int d, int causal, int packed, int dtype, int fp8);

#ifdef __cplusplus
}
#endif

#endif /* IAEA_ATTN_H */
