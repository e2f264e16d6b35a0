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
  QLORA_ERR_WORKSPACE = -6    /* workspace NULL or smaller than the *_workspace_bytes query */
} qlora_status;

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
 * Backward of the same layer (Abstract: backpropagation through the frozen
 * 4-bit model into the adapters; the base weight gets no gradient):
 *     G  = dY B^T                         (fp32, internal)
 *     dX = dY W' + s G A^T                (bf16)
 *     dA = s X^T G                        (bf16)
 *     dB = s (XA)^T dY                    (bf16)
 *   dY [T,N] bf16 upstream gradient; X [T,K] the forward input; XA [T,r] the
 *   fp32 buffer qlora_linear_fwd wrote for this X and A.  Other arguments as
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
 * Support: dequantize codes + double-quantized constants to a dense weight.
 *   out_is_bf16 = 1: out is uint16_t[n] bf16 (the compute weight W' above);
 *   out_is_bf16 = 0: out is float[n], fp32(c[code] * fp32(q8*s2/255)).
 *   n even, >= 0.
 */
int qlora_dequantize_nf4(const uint8_t* codes, const uint8_t* q8, const float* s2,
                         int64_t n, int32_t out_is_bf16, void* out, void* stream);

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

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
