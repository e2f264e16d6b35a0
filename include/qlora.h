/*
 * qlora.h -- C ABI of libqlora: the frozen NF4 linear layer with a LoRA
 * adapter (QLoRA's data-parallel hot path) on AMD Instinct MI355X (gfx950).
 *
 * What the calls compute is fixed by the pages about QLoRA:
 *   - "QLoRA: Efficient Finetuning of Quantized LLMs" (fugumt.com paper page),
 *     Abstract: gradients flow through a frozen 4-bit base model into LoRA
 *     adapters; (a) 4-bit NormalFloat (NF4); (b) double quantization of the
 *     quantization constants.
 *   - QLoRA news write-up (chatgpt.dh666.cn), innovations list: NF4 is
 *     information-theoretically optimal for normally distributed data;
 *     double quantization saves about 0.37 bit per parameter.
 *   - QLoRA project page (aibars.net), configuration example: 4-bit load,
 *     quant type 'nf4', double quantization on, bf16 compute dtype.  These
 *     options are fixed properties of this ABI, not arguments.
 *   - LoRA tutorial (szsimon.cn), weight-update and rank/alpha sections:
 *     h = W x + dW x, dW = W_A W_B, W frozen, alpha scales the adapter.
 * The pages leave the codebook construction, block sizes, constant format and
 * storage layout open; the readings this library implements are stated with
 * each call below.
 *
 * Conventions for every call
 *   - All array pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors on the current device) unless stated otherwise; the caller owns
 *     and allocates every buffer.  Every pointer must be 16-byte aligned.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *     device work is enqueued asynchronously on it; no call synchronizes.
 *   - Outputs are overwritten, never accumulated into.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and returned as a negative qlora_status; launch failures return
 *     QLORA_ERR_HIP and qlora_last_hip_error() gives the HIP code.  No C++
 *     exception crosses the ABI.  Non-finite inputs give unspecified
 *     (finite or not) outputs but never an out-of-bounds access.
 *   - Sizes of zero elements are accepted where stated and enqueue nothing
 *     (or only the zero-fill the semantics require).
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = -1,        /* a required pointer is NULL */
  QLORA_ERR_SHAPE = -2,       /* a size is negative, zero where not allowed, or not a required multiple */
  QLORA_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned */
  QLORA_ERR_UNSUPPORTED = -4, /* blocksize != 64 / 256, rank outside [8,128] or not a multiple of 8 */
  QLORA_ERR_HIP = -5,         /* a HIP launch or query failed; see qlora_last_hip_error() */
  QLORA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the *_workspace_bytes query */
  QLORA_ERR_DEVICE = -7,      /* a kernel's bounded wait ran out (reported by qlora_device_status) */
  QLORA_ERR_SCRATCH = -8,     /* the problem needs more than the no-allocation entry point's scratch */
  QLORA_ERR_IO = -9           /* a file is missing, unreadable, malformed, or of another type or shape */
} qlora_status;

/*
 * Stored 4-bit types.  NF4 is the type QLoRA introduces (Abstract item (a));
 * Int4 and FP4 are the 4-bit integer and float types the pages compare it
 * with (news write-up, innovations list: NF4 gives better results than
 * 4-bit integers and 4-bit floats).  Each is a 16-entry fp32 decode table
 * (qlora_4bit_table); quantization, double quantization, dequantization and
 * the linear layer are the same for all three with the type's table:
 *   NF4   the codebook described at qlora_quantize_nf4;
 *   INT4  code = k mod 16 (4-bit two's complement), value fp32(k/7),
 *         k = -7..7 (symmetric absmax); code 8 is never produced;
 *   FP4   OCP E2M1: code = sign<<3 | exponent<<1 | mantissa (bias 1,
 *         subnormal at exponent 0), value (-1)^sign * fp32(m/6) for the
 *         magnitudes m = 0, 0.5, 1, 1.5, 2, 3, 4, 6; code 8 (-0) is never
 *         produced.
 * The code of a weight is that of the type's level nearest to w/absmax in
 * exact arithmetic (ties to the lower level); an all-zero block gets the
 * code of 0.
 */
typedef enum { QLORA_QTYPE_NF4 = 0, QLORA_QTYPE_INT4 = 1, QLORA_QTYPE_FP4 = 2 } qlora_qtype;

/* Host: the 16 fp32 decode values of a type, indexed by code.  Returns
 * QLORA_ERR_UNSUPPORTED for an unknown type, QLORA_ERR_NULL for out = NULL. */
int qlora_4bit_table(int32_t qtype, float out[16]);

/*
 * Blockwise NF4 quantization (Abstract item (a); innovations list, NF4).
 *   W       [n]        fp32 weights, the [N,K] matrix flattened row-major.
 *   n                  number of weights; must be even and >= 0 (0 = no-op).
 *   blocksize          must be 64.
 *   codes   [n/2]      out: two 4-bit codes per byte, element 2i in the low
 *                      nibble, element 2i+1 in the high nibble.
 *   absmax  [ceil(n/64)] out: fp32 absmax of each block of 64 consecutive
 *                      weights (the last block may be partial).
 * Codebook: 7 negative values, 0 and 8 positive values, the standard-normal
 * quantiles at probabilities equally spaced on [1/2, p_max] with
 * p_max = 1 - (1/30 + 1/32)/2, divided by the largest magnitude so that the
 * extremes are -1 and +1 (see qlora_nf4_codebook).  Each weight gets the code
 * nearest to w/absmax in exact arithmetic (ties to the lower code); an
 * all-zero block gets code 7 (the value 0) everywhere.  Results are
 * bit-exact and deterministic.
 */
int qlora_quantize_nf4(const float* W, int64_t n, int32_t blocksize,
                       uint8_t* codes, float* absmax, void* stream);

/*
 * The same blockwise NF4 quantization for weights stored as bf16, the 16-bit
 * format in which pretrained base models ship (Abstract item (a); the
 * quantizer is defined on real-valued weights).
 *   W       [n]        bf16 weights (raw bits as uint16_t), the [N,K] matrix
 *                      flattened row-major; 16-byte aligned.
 * n, blocksize, codes, absmax and the error returns are those of
 * qlora_quantize_nf4.  A bf16 value widens to fp32 exactly, so codes and
 * absmax are bit-identical to qlora_quantize_nf4 on the fp32 widening of W.
 */
int qlora_quantize_nf4_bf16(const uint16_t* W, int64_t n, int32_t blocksize,
                            uint8_t* codes, float* absmax, void* stream);

/*
 * Blockwise quantization to any stored 4-bit type (see qlora_qtype).
 *   W          [n] fp32 (w_is_bf16 = 0) or bf16 bits (w_is_bf16 = 1).
 *   Other arguments, outputs and errors as qlora_quantize_nf4; qtype must be
 *   a qlora_qtype (else QLORA_ERR_UNSUPPORTED).
 */
int qlora_quantize_4bit(const void* W, int32_t w_is_bf16, int64_t n, int32_t blocksize, int32_t qtype,
                        uint8_t* codes, float* absmax, void* stream);

/*
 * Quantization and double quantization in one pass (Abstract items (a) and
 * (b)): the same codes, q8 and s2 as qlora_quantize_4bit followed by
 * qlora_double_quant, bit for bit, without writing or re-reading the fp32
 * absmax constants (each group of 256 blocks keeps them on chip).
 *   W      [n]              fp32 (w_is_bf16 = 0) or bf16 bits (w_is_bf16 = 1).
 *   n                       even, >= 0 (0 = no-op).  Block sizes are 64 and 256.
 *   codes  [n/2]            out, as qlora_quantize_4bit.
 *   q8     [ceil(n/64)]     out, as qlora_double_quant.
 *   s2     [ceil(n/16384)]  out, as qlora_double_quant.
 */
int qlora_quantize_dq(const void* W, int32_t w_is_bf16, int64_t n, int32_t qtype,
                      uint8_t* codes, uint8_t* q8, float* s2, void* stream);

/*
 * Double quantization of the absmax constants (Abstract item (b);
 * innovations list: quantizing the quantization constants saves ~0.37 bit
 * per parameter).
 *   absmax  [nb]            fp32 constants from qlora_quantize_nf4 (>= 0).
 *   nb                      number of constants, >= 0 (0 = no-op).
 *   blocksize2              must be 256.
 *   q8      [nb]            out: 8-bit codes, q8_b = nearest integer to
 *                           255 * absmax_b / s2_g (ties to even), 0 if s2_g = 0.
 *   s2      [ceil(nb/256)]  out: fp32 max of each group of 256 constants.
 * The dequantized constant is fp32(q8_b * s2_g / 255), rounded once.
 * Storage with both levels: 4 + 8/64 + 32/(64*256) bit per weight.
 */
int qlora_double_quant(const float* absmax, int64_t nb, int32_t blocksize2,
                       uint8_t* q8, float* s2, void* stream);

/*
 * Forward of the frozen NF4 linear layer with LoRA (Abstract: frozen 4-bit
 * base, LoRA adapters; LoRA tutorial: h = W x + dW x):
 *     Y  = X W'^T + s (X A) B,     s = alpha / r (fp32)
 *     XA = X A                     (fp32, kept for the backward pass)
 * where W' [N,K] is the dequantized weight rounded to bf16 (compute dtype):
 *     W'[n,k] = bf16( c[code] * fp32(q8_b * s2_g / 255) ),  b = (n*K + k)/64.
 *   X     [T,K]  bf16 input, row-major.           T >= 0 (0 = no-op)
 *   codes [N*K/2], q8 [N*K/64], s2 [ceil(N*K/64/256)]: W as produced by
 *                qlora_quantize_nf4 + qlora_double_quant on the [N,K] matrix.
 *   A     [K,r]  bf16 LoRA down-projection, row-major.
 *   B     [r,N]  bf16 LoRA up-projection, row-major.
 *   K            in_features: K >= 64, K % 64 == 0.
 *   N            out_features: N >= 8, N % 8 == 0.
 *   r            LoRA rank: 8 <= r <= 128, r % 8 == 0.
 *   Size limits: every kernel addresses its operands through 32-bit buffer
 *   views, so N*K/2, T*K*2 and T*N*2 bytes (and each internal workspace
 *   region) must each be below 2^31; larger problems return
 *   QLORA_ERR_SHAPE before anything is enqueued (split them along T or N).
 *   Why the rank is narrowed: the kernels move rank-r rows of A, B, XA and
 *   the gradients as 16-byte vectors of 8 values and keep up to 128 fp32
 *   rank columns per lane group in registers.  Ranks that are multiples of
 *   8 up to 128 cover the usual LoRA ranks (8 ... 128).  Another rank r' is
 *   served by padding: pass A with zero columns and B with zero rows up to
 *   r = the next multiple of 8, and alpha * r / r' as alpha so that alpha / r
 *   is the intended alpha / r' (up to one rounding of alpha; exact when both
 *   are powers of two); Y, XA's first r' columns, dX and the first r'
 *   columns/rows of dA/dB are then those of rank r', the padding's are zero.
 *   Why N % 8: rows of Y and dB are stored as 16-byte vectors.
 *   Y     [T,N]  out: bf16.
 *   XA    [T,r]  out: fp32.
 *   workspace    device scratch of at least
 *                qlora_linear_fwd_workspace_bytes(T,K,N,r) bytes (may be NULL
 *                when that is 0); its contents are not preserved.
 * Small token counts (T <= 16) take an HBM-bound dequant-GEMV path; larger
 * ones a dequantize-into-MFMA GEMM with the rank-r update fused into its
 * epilogue.  Accumulation is fp32; results are deterministic.
 */
size_t qlora_linear_fwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r);
int qlora_linear_fwd(const uint16_t* X, int64_t T, int64_t K, int64_t N,
                     const uint8_t* codes, const uint8_t* q8, const float* s2,
                     const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                     uint16_t* Y, float* XA,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped forward: several frozen 4-bit linears with LoRA adapters that share
 * the token count T, the rank r and alpha, in one call (fused q/k/v,
 * gate/up, or every linear of a layer; the small-token path of 4-bit
 * inference and batched generation, QLoRA project page, inference
 * features).  Each linear computes exactly what qlora_linear_fwd_4bit
 * computes for it.  For T <= 16, every run of up to 8 consecutive linears is
 * one XA-partial launch and one dequant-GEMV launch over all their weights,
 * so launch and ramp are paid once per run and the weight streams overlap
 * (results bit for bit those of qlora_linear_fwd_4bit).  For larger T, every
 * run of up to 4 consecutive linears with the same K and N (q/k/v, gate/up)
 * shares one dequant-GEMM launch over all their output tiles, so small token
 * counts fill the GPU with whole-contraction tiles, and one launch of each
 * rank-r kernel; results (Y and XA) equal qlora_linear_fwd_4bit's within the
 * fp32 accumulation-order tolerance (the contractions may be cut into slices
 * differently, sized for the whole run).
 *   descs    host array of `count` linear descriptors (0 <= count <= 4096);
 *            each names its own X [T,K], weight, A [K,r], B [r,N], and
 *            outputs Y [T,N] and XA [T,r] (device pointers; several linears
 *            may share one X).  K and N follow qlora_linear_fwd's rules.
 *   workspace of at least qlora_linear_fwd_grouped_workspace_bytes bytes.
 * Outputs of different linears must not overlap.
 */
typedef struct {
  const uint16_t* X;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* s2;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* Y;
  float* XA;
  int64_t K;
  int64_t N;
} qlora_linear_desc;
size_t qlora_linear_fwd_grouped_workspace_bytes(int32_t count, const qlora_linear_desc* descs, int64_t T,
                                                 int32_t r);
int qlora_linear_fwd_grouped(int32_t qtype, int32_t count, const qlora_linear_desc* descs, int64_t T, int32_t r,
                             float alpha, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped backward, the counterpart of qlora_linear_fwd_grouped: each linear
 * gets what qlora_linear_bwd_4bit computes for it (dX, dA, dB); runs of up to
 * 4 consecutive linears with the same K and N share one dX dequant-GEMM
 * launch over all their tiles and one launch of each rank-r kernel (dX, dA
 * and dB within the accumulation-order tolerance of the single call: the
 * contractions are cut into slices sized for the whole run).  T = 0 zeroes
 * every dA and dB.
 *   descs  host array of `count` descriptors (0 <= count <= 4096), each with
 *          its own dY [T,N], X [T,K], XA [T,r] (from the forward), weight,
 *          A, B and outputs dX [T,K], dA [K,r], dB [r,N].
 *   workspace of at least qlora_linear_bwd_grouped_workspace_bytes bytes.
 */
typedef struct {
  const uint16_t* dY;
  const uint16_t* X;
  const float* XA;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* s2;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* dX;
  uint16_t* dA;
  uint16_t* dB;
  int64_t K;
  int64_t N;
} qlora_linear_bwd_desc;
size_t qlora_linear_bwd_grouped_workspace_bytes(int32_t count, const qlora_linear_bwd_desc* descs, int64_t T,
                                                 int32_t r);
int qlora_linear_bwd_grouped(int32_t qtype, int32_t count, const qlora_linear_bwd_desc* descs, int64_t T, int32_t r,
                             float alpha, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward without any device allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same computation, kernels, arguments and results as
 * qlora_linear_fwd, but the workspace is the library's own static device
 * array of 80 MiB (QLORA_NOALLOC_SCRATCH_BYTES) on each GPU, held until the
 * process ends; the call itself allocates nothing.  A problem whose
 * qlora_linear_fwd_workspace_bytes exceeds it returns QLORA_ERR_SCRATCH
 * before anything is enqueued (every configuration of this library's
 * benchmarks needs at most 69 MiB).  Every call on a GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialized by the caller.  The kernels clear the
 * counters they need at the start of each call, so leftover contents from an
 * earlier call never matter.
 */
#define QLORA_NOALLOC_SCRATCH_BYTES (80u << 20)
int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t T, int64_t K, int64_t N,
                             const uint8_t* codes, const uint8_t* q8, const float* s2,
                             const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                             uint16_t* Y, float* XA, void* stream);

/*
 * Backward of the same layer (Abstract: backpropagation through the frozen
 * 4-bit model into the adapters; the base weight gets no gradient):
 *     G  = dY B^T                         (fp32, internal)
 *     dX = dY W' + s G A^T                (bf16)
 *     dA = s X^T G                        (bf16)
 *     dB = s (XA)^T dY                    (bf16)
 *   dY [T,N] bf16 upstream gradient; X [T,K] the forward input; XA [T,r] the
 *   fp32 buffer qlora_linear_fwd wrote for this X and A, or NULL when the
 *   caller did not keep it (gradient checkpointing, QLoRA project page, core
 *   techniques: activations are recomputed instead of stored): XA is then
 *   recomputed from X and A inside the call (bit for bit the forward's for
 *   T > 16; within fp32 accumulation order for T <= 16).  Other arguments as
 *   in qlora_linear_fwd.  dX [T,K], dA [K,r], dB [r,N] are overwritten.
 *   T = 0 is allowed: dX is empty and dA, dB are set to zero.
 *   workspace of at least qlora_linear_bwd_workspace_bytes(T,K,N,r) bytes.
 * Reductions over tokens are split and summed in a fixed order (no float
 * atomics), so results are deterministic.
 */
size_t qlora_linear_bwd_workspace_bytes(int64_t T, int64_t K, int64_t N, int32_t r);
int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, const float* XA,
                     int64_t T, int64_t K, int64_t N,
                     const uint8_t* codes, const uint8_t* q8, const float* s2,
                     const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                     uint16_t* dX, uint16_t* dA, uint16_t* dB,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * One AdamW step over a flat buffer of adapter parameters (QLoRA project
 * page, technical architecture: the adapters are trained with AdamW and
 * paged optimizers; challenges: gradient clipping keeps training stable).
 * With g = c * grad and t = step (1, 2, ...):
 *     m = b1 m + (1-b1) g,   v = b2 v + (1-b2) g^2,
 *     master = master - lr (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + wd master),
 *     param = bf16(master)   (round to nearest even)
 * where c = min(1, max_grad_norm / (||grad|| + 1e-6)) with ||grad|| the L2
 * norm of the whole buffer (c = 1 when max_grad_norm <= 0).  The adapters of
 * all linears are meant to live in one flat allocation (per-linear views),
 * so one call updates them all.
 *   n                 elements (>= 0; 0 = no-op).
 *   param   [n] bf16  in/out: the adapter values the layer uses.
 *   master  [n] fp32  in/out: master copy of the parameters.
 *   m, v    [n] fp32  in/out: first and second moments (zero before step 1).
 *   grad    [n] bf16  the gradients (dA, dB of qlora_linear_bwd).
 *   grad_norm_out     optional device float: receives ||grad|| (unclipped).
 *   workspace         qlora_adamw_workspace_bytes(n) bytes when clipping or
 *                     grad_norm_out is asked for (else may be NULL).
 * Paged optimizer: master, m and v may be device memory or pinned host
 * memory (hipHostMalloc, e.g. torch pin_memory tensors); the state then takes
 * no GPU memory and the step streams it over the host link.  Pageable host
 * memory returns QLORA_ERR_UNSUPPORTED.  The norm is summed in fp64 in a
 * fixed order, so results are deterministic.  Hyperparameters must satisfy
 * 0 <= b1, b2 < 1, eps > 0, lr >= 0, wd >= 0 (else QLORA_ERR_UNSUPPORTED);
 * step < 1 returns QLORA_ERR_SHAPE.
 */
size_t qlora_adamw_workspace_bytes(int64_t n);
int qlora_adamw_step(int64_t n, uint16_t* param, float* master, float* m, float* v, const uint16_t* grad,
                     int32_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                     float max_grad_norm, float* grad_norm_out, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Support: dequantize codes + double-quantized constants to a dense weight.
 *   out_is_bf16 = 1: out is uint16_t[n] bf16 (the compute weight W' above);
 *   out_is_bf16 = 0: out is float[n], fp32(c[code] * fp32(q8*s2/255)).
 *   n even, >= 0.
 */
int qlora_dequantize_nf4(const uint8_t* codes, const uint8_t* q8, const float* s2,
                         int64_t n, int32_t out_is_bf16, void* out, void* stream);

/* Dequantization for any stored type (as qlora_dequantize_nf4 with the
 * type's table). */
int qlora_dequantize_4bit(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t n, int32_t qtype,
                          int32_t out_is_bf16, void* out, void* stream);

/*
 * The linear layer with a base weight of any stored 4-bit type: exactly
 * qlora_linear_fwd / qlora_linear_bwd (same arguments after qtype, same
 * kernels, results and errors) with W' = bf16(table[code] * c1').
 */
int qlora_linear_fwd_4bit(int32_t qtype, const uint16_t* X, int64_t T, int64_t K, int64_t N,
                          const uint8_t* codes, const uint8_t* q8, const float* s2,
                          const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                          uint16_t* Y, float* XA, void* workspace, size_t workspace_bytes, void* stream);
int qlora_linear_bwd_4bit(int32_t qtype, const uint16_t* dY, const uint16_t* X, const float* XA,
                          int64_t T, int64_t K, int64_t N,
                          const uint8_t* codes, const uint8_t* q8, const float* s2,
                          const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                          uint16_t* dX, uint16_t* dA, uint16_t* dB,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Storage of a quantized weight (the format is deterministic, so a saved
 * weight reloads bit for bit).  The file is a safetensors file: tensors
 * "s2" (F32 [ceil(N*K/16384)]), "codes" (U8 [N*K/2]) and "q8"
 * (U8 [ceil(N*K/64)]), and metadata naming the format ("qlora-4bit"), the
 * type ("nf4", "int4", "fp4"), N, K, the block sizes (64, 256) and the
 * type's decode table as fp32 bit patterns.  These calls wait for `stream`
 * and copy through host memory (they are host-blocking, unlike the others).
 *   qlora_save_4bit       writes the device buffers of an N x K weight.
 *   qlora_load_4bit_info  reads a file's type, N and K (no device access).
 *   qlora_load_4bit       checks that the file holds exactly this type,
 *                         N and K and this library's decode table, then
 *                         copies the tensors into the device buffers.
 * File errors and any mismatch return QLORA_ERR_IO.
 */
int qlora_save_4bit(const char* path, int32_t qtype, int64_t N, int64_t K,
                    const uint8_t* codes, const uint8_t* q8, const float* s2, void* stream);
int qlora_load_4bit_info(const char* path, int32_t* qtype, int64_t* N, int64_t* K);
int qlora_load_4bit(const char* path, int32_t qtype, int64_t N, int64_t K,
                    uint8_t* codes, uint8_t* q8, float* s2, void* stream);

/*
 * Support: per-kernel timing for benchmarks.  While enabled, every kernel the
 * library enqueues is bracketed by two HIP events recorded on the stream it
 * is launched on.  qlora_timing_read waits for those events, writes one line
 * "kernel_name launches total_ms" per kernel (NUL-terminated, truncated to
 * buflen) into the host buffer buf, forgets the records, and returns the
 * length of the full text, or QLORA_ERR_HIP if an event query failed.
 * Timing adds two event records per launch; leave it off otherwise.
 */
void qlora_timing_enable(int on);
int qlora_timing_read(char* buf, size_t buflen);

/* Host: copy the library's 16-entry fp32 NF4 codebook (ascending) to out. */
void qlora_nf4_codebook(float out[16]);

/* Host: a static description of a qlora_status value. */
const char* qlora_status_string(int status);

/* Host: the HIP error code behind the last QLORA_ERR_HIP on this thread. */
int qlora_last_hip_error(void);

/*
 * Support: the device status of the current GPU.  The split-contraction
 * hand-off of the dequant-GEMMs waits a bounded time for the other slices of
 * a tile (a guard that is never reached when every slice runs); if the
 * bound ever ran out, the finishing workgroup sets a status bit on the
 * device and stores an incomplete sum.  This call waits for `stream`,
 * returns QLORA_ERR_DEVICE if any bit is set (the outputs of the calls since
 * the previous query are then unreliable) and clears the bits; QLORA_OK
 * otherwise, or QLORA_ERR_HIP if the wait or the read failed.  Host-blocking.
 */
int qlora_device_status(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
