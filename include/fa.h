/*
 * fa.h -- C ABI of libfa: fused exact attention on AMD Instinct MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T) V
 * (the attention formula of the bjdmk.com.cn FlashAttention page, section
 * "性能引擎") in one fused kernel with an online softmax, and its exact
 * gradients by recomputing P from the stored row logsumexp (recomputation:
 * pwwt.cn page, section "3. 重计算"; keeping only the logsumexp: hotelren.com
 * FlashAttention-2 walkthrough, section 3.1).  The causal variant masks keys
 * j > query i (lower-triangular mask: bjdmk.com.cn page, section "实战集成").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The
 *   library never allocates, frees or keeps a pointer after it returns
 *   (fa_bwd_noalloc's static scratch array, below, is the one piece of
 *   device memory the library itself holds).
 * - Work is enqueued asynchronously on `stream` (NULL = the null stream).
 *   The library never synchronises; kernel faults surface at the caller's
 *   next synchronisation, as usual in HIP.
 * - Element type of q, k, v, o, dout, dq, dk, dv: `dtype` (FA_F16 or
 *   FA_BF16).  lse is fp32; the workspace layout is given below.
 * - Tensor layout: logical [B, N, H, D] (batch, sequence, head, head_dim),
 *   the flash_attn_func layout of the hotelren.com walkthrough, section 5.
 *   Element strides (b, n, h) per tensor are given by the optional strides
 *   struct; the d stride is always 1.  NULL strides mean contiguous
 *   [B, N, H, D] for every tensor.  A packed qkv [B, N, 3, H, D] tensor
 *   (bjdmk.com.cn page, section "实战集成") is passed as three views with
 *   n-stride 3*H*D and h-stride D.
 * - lse is fp32, contiguous [B, H, N]: LSE[b,h,i] = ln sum_j exp(scale*q_i.k_j)
 *   over the unmasked keys j (natural logarithm of the scaled scores).
 * - Sizes: B, H, N >= 1 (N_q = N_k = N); D in {64, 128}.
 * - Return value: FA_OK or an error status.  Argument errors are detected
 *   before any HIP call and leave every buffer untouched.  The functions
 *   never print and never abort.
 * - Stateless and reentrant; concurrent calls on different streams are safe
 *   as long as their output and workspace buffers do not overlap.  The
 *   exception is fa_bwd_noalloc: its calls share one scratch array per
 *   device and must not overlap in time on a device.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, size <= 0, non-finite scale,
                             causal not 0/1, unknown dtype, workspace too small */
  FA_ERR_UNSUPPORTED = 2, /* D not 64/128, tensor pointer not 16-byte aligned
                             (lse: 4-byte; workspace: 256-byte),
                             b/n/h stride not a multiple of 8 elements, an
                             n stride of 2^24 elements or more, a size
                             whose element offsets overflow int64, more
                             than 2^31 rows B*H*N, or (fa_bwd) N*D*4 bytes
                             per head at or above 2^31 */
  FA_ERR_HIP = 3,         /* a HIP runtime call failed (no device, launch error) */
  FA_ERR_TOO_LARGE = 4    /* fa_bwd_noalloc: the problem needs more scratch than
                             its static array holds (fa_bwd_noalloc_max_bytes) */
} fa_status;

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

/* Element strides of one logical [B, N, H, D] tensor (stride of d is 1). */
typedef struct {
  int64_t b, n, h;
} fa_stride3;

typedef struct {
  fa_stride3 q, k, v, o;
} fa_fwd_strides;

typedef struct {
  fa_stride3 q, k, v, o, dout, dq, dk, dv;
} fa_bwd_strides;

/*
 * fa_fwd -- fused attention forward.
 *   q, k, v : inputs, [B, N, H, D] (strided), dtype.
 *   o       : output, [B, N, H, D] (strided), dtype; every element written.
 *   lse     : output, fp32 contiguous [B, H, N]; every element written.
 *   causal  : 0 = full attention, 1 = key j visible to query i iff j <= i.
 *   scale   : multiplies q.k before the softmax; any finite value
 *             (1/sqrt(D) is the formula's choice).
 *   strides : NULL or the element strides of q, k, v, o.
 * o must not alias q, k or v.  Extra device memory: none.
 * Launches with at most two query rows per (batch, head) run a vector-unit
 * kernel that streams K and V through registers and keeps the softmax
 * weights in fp32; larger ones run the tiled matrix-core kernels, which
 * round the weights to dtype for the P.V product.  Both meet the same
 * bound against the exact result.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int D, int causal, float scale, int dtype,
           const fa_fwd_strides* strides, hipStream_t stream);

/*
 * fa_fwd_qk -- fa_fwd with Nq query rows against Nk keys (fa_fwd is the
 * case Nq = Nk = N).
 *   q, o : [B, Nq, H, D];  k, v : [B, Nk, H, D];  lse : [B, H, Nq].
 *   causal = 1 aligns the mask to the last query and key: query i sees key j
 *   iff j <= i + Nk - Nq.  So Nq new queries against an Nk-key history see
 *   what the last Nq rows of the square problem see, and with Nq > Nk the
 *   first Nq - Nk queries see no key: their o row is 0 and lse is -inf (the
 *   logsumexp of an empty set).  The mask, and the exact merge of results
 *   over split key sets (fa_merge), are those of the reading of the pages'
 *   causal (lower-triangular) mask for unequal lengths.
 * Other arguments, errors and memory: as fa_fwd (Nq and Nk both >= 1).
 */
int fa_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Nq, int Nk, int D, int causal, float scale,
              int dtype, const fa_fwd_strides* strides, hipStream_t stream);

/*
 * fa_fwd_split -- fa_fwd_qk with the keys divided among workgroups, for
 * launches whose query side alone cannot fill the device (few heads, short
 * Nq against a long key history, e.g. decoding or small chunks of a long
 * context).  The keys are cut into contiguous ranges of ceil(Nk /
 * num_splits) keys rounded up to a multiple of 128; every range is
 * processed by its own workgroups, which write an fp32 partial (O_r, LSE_r)
 * over that range into the workspace, and a second kernel combines them
 * exactly with the rule of fa_merge (LSE = ln sum_r exp(LSE_r), O =
 * sum_r exp(LSE_r - LSE) O_r), rounding o once.  The result is fa_fwd_qk's
 * up to fp32 rounding of the combination; ranges a query row cannot see
 * (causal) carry no weight.
 *   num_splits      : 1 .. 256; 1 (or a count that leaves one range) is
 *                     fa_fwd_qk and needs no workspace.
 *   workspace       : device buffer of at least
 *                     fa_fwd_split_workspace_bytes(B, H, Nq, D, num_splits)
 *                     bytes, 256-byte aligned; contents undefined on entry
 *                     and on exit.
 * Other arguments and errors: as fa_fwd_qk; num_splits out of range, or a
 * missing or too small workspace when it is needed: FA_ERR_INVALID_ARG.
 */
int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Nq, int Nk, int D, int causal, float scale,
                 int dtype, const fa_fwd_strides* strides, int num_splits,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace of fa_fwd_split: fp32 [num_splits, B, H, Nq, D] partial outputs
 * and [num_splits, B, H, Nq] logsumexps, each part rounded up to 256 bytes.
 * Returns 0 for invalid sizes. */
size_t fa_fwd_split_workspace_bytes(int B, int H, int Nq, int D, int num_splits);

/* A split count for fa_fwd_split.  Nq <= 2 (the vector-unit kernel, one
 * 4-wave workgroup per (batch, head, split)): 1 when B*H >= 256, else
 * ceil(256 / (B*H)) limited to floor(Nk / 1024) and 64.  Larger Nq, with W
 * the waves of the unsplit launch (one per 32 query rows; two at head_dim
 * 128 in its two-key-group forms): 1 when W > 1024 (one wave per SIMD of
 * the device); else S = min(ceil(4096 / W), 64, floor(Nk / 2048)), and
 * where W*S < 1024 instead min(ceil(4096 / W), 64, floor(Nk / 1024),
 * ceil(1024 / W)).  The result is at least 1. */
int fa_fwd_split_count(int B, int H, int Nq, int Nk, int D, int causal);

/*
 * fa_bwd_workspace_bytes -- size of the scratch fa_bwd needs: the row vector
 * Dvec = rowsum(dO o O) [B, H, N] (fp32), the dQ accumulator [B, H, N, D]
 * (int32, fixed point), three maxima per 16-row block [B*H, 3, ceil(N/16)]
 * (fp32), one dQ bound per head [B*H] (fp32), and -- for launches with
 * few key blocks of 256 keys, whose query range is split into S
 * segments -- partial dK and dV sums [S, B, H, N, D] (fp32) each.
 * S = min(8, ceil(512 / key blocks), T) for a causal launch with fewer than
 * 512 key blocks, min(8, ceil(256 / key blocks), T) for a non-causal one
 * with at most 128, else 1 (no partials when S = 1); T is the number of
 * query tiles, ceil(N / 64) at D = 64 and ceil(N / 32) at D = 128.  This size is the causal one, which serves either mask.
 * Every part is rounded up to 256 bytes.  O(N*D) per head; no N*N term.
 * Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int D);

/* Workspace of fa_bwd_qk: as above with Dvec and the dQ accumulator over Nq
 * rows, the maxima over ceil(max(Nq, Nk) / 16) blocks, and the partial sums
 * [S, B, H, Nk, D] with S from the key blocks of Nk and the query tiles of
 * Nq.
 * Like fa_bwd_workspace_bytes, it is the size for a causal launch, which
 * serves either mask. */
size_t fa_bwd_qk_workspace_bytes(int B, int H, int Nq, int Nk, int D);

/* The workspace one mask needs (causal 0 or 1): fa_bwd_qk_workspace_bytes
 * for causal = 1; for causal = 0, the partial dK, dV sums of the non-causal
 * segment count (none above 128 key blocks).  The partial sums are the last
 * part of the layout, so a buffer of this size and one of the causal size
 * are used identically below it.  Returns 0 for invalid sizes or causal. */
size_t fa_bwd_qk_workspace_bytes_for(int B, int H, int Nq, int Nk, int D, int causal);

/*
 * fa_bwd -- attention backward by recomputation.
 *   q, k, v, o, lse : exactly as given to / produced by fa_fwd with the same
 *                     B, H, N, D, causal, scale and dtype.
 *   dout            : gradient of the loss w.r.t. o, [B, N, H, D], dtype.
 *   dq, dk, dv      : outputs, [B, N, H, D] (strided), dtype; overwritten
 *                     (not accumulated into).  They may be views into one
 *                     packed dqkv tensor but must not overlap each other or
 *                     any input.
 *   workspace       : device buffer of at least
 *                     fa_bwd_qk_workspace_bytes_for(B, H, N, N, D, causal)
 *                     bytes (fa_bwd_workspace_bytes(B, H, N, D) serves
 *                     either mask), 256-byte aligned; contents undefined on
 *                     entry and on exit.
 * Three kernels are enqueued on `stream`: the Dvec preprocess (which also
 * clears the dQ accumulator and takes the largest |dO_i|, |K| element
 * and |V_j| per head, |.| the Euclidean norm of a row), the K/V-block-
 * parallel dK/dV kernel that accumulates dQ with 32-bit integer atomics in
 * units of B / 2^30, B = 4 max|K| max|dO_i| max|V_j| per (batch, head) --
 * a bound on any partial sum of dS K -- and the dQ conversion.  Narrow
 * launches (causal below 512 key blocks, non-causal at 128 or fewer) add a
 * fourth, which sums the partial dK, dV of the query segments.  The integer
 * dQ sum is exact, so dq is bitwise reproducible; each key block's
 * contribution is rounded to the nearest unit.  B is
 * raised to at least 2^-96 (the scale 2^30 / B stays finite); heads whose
 * bound is not finite (non-finite inputs) get dq = NaN.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int D, int causal, float scale, int dtype,
           const fa_bwd_strides* strides, void* workspace,
           size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd_stages -- fa_bwd split into its three kernels, for callers that
 * schedule or time them separately.  Arguments are those of fa_bwd; `stages`
 * is a bit mask: FA_STAGE_PREPROCESS (Dvec, the cleared dQ accumulator and
 * the bound maxima, written to the workspace), FA_STAGE_DKDV (dK, dV, and dQ
 * accumulated in the workspace) and FA_STAGE_DQ (dq from the accumulator).  Each stage
 * reads what the previous one left in the same workspace, so the stages must
 * run in this order on one stream with the same workspace; fa_bwd is
 * fa_bwd_stages with all three bits.  stages = 0 or unknown bits:
 * FA_ERR_INVALID_ARG.
 */
#define FA_STAGE_PREPROCESS 1u
#define FA_STAGE_DKDV 2u
#define FA_STAGE_DQ 4u
#define FA_STAGE_ALL 7u
int fa_bwd_stages(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk,
                  void* dv, int B, int H, int N, int D, int causal,
                  float scale, int dtype, const fa_bwd_strides* strides,
                  void* workspace, size_t workspace_bytes, unsigned stages,
                  hipStream_t stream);

/*
 * fa_bwd_qk -- fa_bwd_stages with Nq query rows against Nk keys, for o and
 * lse from fa_fwd_qk with the same arguments.  q, o, dout, dq : [B, Nq, H,
 * D]; k, v, dk, dv : [B, Nk, H, D]; lse : [B, H, Nq]; workspace of at least
 * fa_bwd_qk_workspace_bytes(B, H, Nq, Nk, D) bytes.  Queries that see no
 * key get dq = 0 and add nothing to dk, dv.  Stages, errors and memory: as
 * fa_bwd_stages (FA_STAGE_ALL for the whole backward).
 */
int fa_bwd_qk(const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, void* dq, void* dk, void* dv,
              int B, int H, int Nq, int Nk, int D, int causal, float scale,
              int dtype, const fa_bwd_strides* strides, void* workspace,
              size_t workspace_bytes, unsigned stages, hipStream_t stream);

/*
 * fa_bwd_noalloc -- fa_bwd_qk (all three stages) with no caller workspace,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * scratch is one static device array of fa_bwd_noalloc_max_bytes() bytes
 * (64 MiB) per device, which that device holds from the first call on it
 * until the process ends; the call itself never calls hipMalloc, hipFree or
 * any allocating routine.  On its first call on a device (the device current
 * on the calling thread, which must be the stream's device) it looks up the
 * array's device address once (hipGetSymbolAddress) and keeps it.
 *   Arguments, layouts, results and errors: as fa_bwd_qk with stages =
 *   FA_STAGE_ALL, minus the workspace.  A problem whose
 *   fa_bwd_qk_workspace_bytes(B, H, Nq, Nk, D) exceeds
 *   fa_bwd_noalloc_max_bytes() returns FA_ERR_TOO_LARGE before any HIP call
 *   (roughly B*H*Nq*(D+1)*4 bytes: B=1 H=8 N=8192 D=128 fits, B=1 H=16
 *   N=16384 D=64 does not); a failed address lookup returns FA_ERR_HIP.
 * Every call on one device uses that device's single array.  The kernels
 * write every scratch value before reading it, so what an earlier call left
 * there does not matter; but calls that overlap in time on one device
 * (different streams or host threads) race on it and give wrong results --
 * serialise them.  dq, dk and dv equal those of fa_bwd_qk bit for bit.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int Nq, int Nk, int D, int causal, float scale,
                   int dtype, const fa_bwd_strides* strides, hipStream_t stream);

/* Size in bytes of fa_bwd_noalloc's static scratch array (64 MiB). */
size_t fa_bwd_noalloc_max_bytes(void);

/*
 * fa_merge -- exact combination of P attention results over disjoint key
 * sets of the same queries (for example the chunks of a sequence-sharded or
 * chunked K/V): LSE = ln sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r.
 * This is what keeping the logsumexp allows (hotelren.com FlashAttention-2
 * walkthrough, section 3.1).  Rows that no part covers (all LSE_r = -inf)
 * get o = 0, lse = -inf.
 *   o_parts   : device, P results stacked contiguously, [P, B, N, H, D], dtype.
 *   lse_parts : device, fp32 [P, B, H, N].
 *   o         : output, contiguous [B, N, H, D], dtype (must not overlap the
 *               parts).
 *   lse       : output, fp32 [B, H, N].
 * The weights and sums are fp32; o is rounded once (RNE).  Errors: as
 * fa_fwd (P <= 0: FA_ERR_INVALID_ARG).  Extra device memory: none.
 */
int fa_merge(const void* o_parts, const float* lse_parts, int P, void* o,
             float* lse, int B, int H, int N, int D, int dtype,
             hipStream_t stream);

/*
 * fa_fwd_fp8 -- attention forward with FP8 inputs.  FlashAttention-3 adds
 * FP8 inputs for throughput (FlashAttention IO-awareness article at
 * 0539edu.com, sections "H100的FP8加速能力" and "未来展望"); the pages give
 * no format or scaling rule, and this entry point takes:
 *   q, k, v   : device, OCP FP8 E4M3 codes (1 sign, 4 exponent bits with
 *               bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN),
 *               [B, Nq, H, D] and [B, Nk, H, D], d contiguous.
 *   descale_q, descale_k, descale_v : device, fp32 [B*H] (index b*H + h),
 *               or NULL for 1.  The value of code c is descale * e4m3(c).
 *               Finite; any sign (a negative factor flips the scores).
 *   o         : output, [B, Nq, H, D], out_dtype (FA_BF16 or FA_F16).
 *   lse       : output, fp32 [B, H, Nq], natural log.
 * Result: o = softmax(scale * Q K^T) V over the descaled values, with the
 * softmax weights rounded to E4M3 (round to nearest even) before the
 * product with V and the row normalised by the sum of the rounded weights;
 * both products run on the 8-bit matrix cores with fp32 accumulation.  lse
 * is the logsumexp of the exact scaled scores (fp32 weights).  causal and
 * Nq != Nk: as fa_fwd_qk.  Strides (in elements, i.e. bytes for q, k, v)
 * as fa_fwd_strides or NULL for contiguous; q, k, v strides must be
 * multiples of 16, o strides multiples of 8, all n strides below 2^24.
 * Errors: as fa_fwd_qk; out_dtype other than FA_BF16 / FA_F16:
 * FA_ERR_INVALID_ARG.  Extra device memory: none.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               const float* descale_q, const float* descale_k, const float* descale_v,
               int B, int H, int Nq, int Nk, int D, int causal, float scale,
               int out_dtype, const fa_fwd_strides* strides, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_str(int status);

/* Library version string, e.g. "fa-gfx950 0.3.0" (static string). */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
