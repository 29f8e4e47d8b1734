/*
 * sagesla.h — C ABI of the SageSLA attention forward for AMD Instinct MI355X (gfx950).
 *
 * SageSLA is the attention of TurboDiffusion's video DiT layers: per query block, the top-k most important
 * key blocks are attended with INT8-quantized scores (SageAttention), and the remaining key blocks go to an
 * elu+1 linear-attention branch whose output passes through a D×D projection (SLA).
 * Sources:
 *   [TD-news]  "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn): §三(一) SageAttention2++ items 1–3
 *              (smoothing, per-block quantization, low-bit attention) and §三(二) SLA items 1–3 (top-k selection,
 *              linear branch with projection, select-then-INT8 hybrid);
 *   [TD-guide] "TurboDiffusion技术指南：突破视频生成效率瓶颈的实践方案" (blog.gitcode.com): inference flags
 *              --attention_type sagesla and --sla_topk (fraction of blocks kept).
 *
 * Conventions shared by every entry point
 *  - Tensors are row-major [B][H][N][D] with D contiguous; q, k, v and out are bf16 (raw 16-bit patterns).
 *  - Every data pointer is a device pointer owned by the caller. The library never allocates, frees or
 *    synchronizes device memory; all scratch lives in the caller's workspace.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is the null stream). Outputs are
 *    ready when the stream reaches that point.
 *  - Parameters are validated on the host before any launch; on an error nothing is launched and the status
 *    says why. Exceptions never cross the ABI.
 *  - Two calls that share a workspace or output buffers must not run concurrently.
 *  - Results are deterministic: no floating-point atomics; every reduction has a fixed order.
 *  - Inputs must be finite.
 */
#ifndef SAGESLA_H
#define SAGESLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAGESLA_OK = 0,
  SAGESLA_E_NULL = 1,        /* a required pointer is NULL                                              */
  SAGESLA_E_SHAPE = 2,       /* B, H or N < 1, B*H > 65535, topk outside [0, n_kb], sm_scale < 0 or NaN,
                                norm_eps negative or not finite (with SAGESLA_QK_RMSNORM)                    */
  SAGESLA_E_UNSUPPORTED = 3, /* D != 128, blk_k != 64, blk_q not in {64, 128}, unknown flag bits,
                                N > 2^24 or n_kb > 20480                                                  */
  SAGESLA_E_WORKSPACE = 4,   /* workspace smaller than sagesla_workspace_bytes()                         */
  SAGESLA_E_ALIGN = 5,       /* a pointer is not 16-byte aligned (workspace: 256-byte aligned)           */
  SAGESLA_E_HIP = 6          /* a HIP call or launch failed; sagesla_last_hip_error() holds its code     */
} sagesla_status;

/* stages of sagesla_forward, in launch order (for the optional timing events) */
#define SAGESLA_STAGE_QUANTIZE 0 /* (RMSNorm of Q and K,) K mean, smoothing, INT8 codes, scales, pooled means */
#define SAGESLA_STAGE_SELECT 1   /* block scores and top-k                                          */
#define SAGESLA_STAGE_LINEAR 2   /* linear branch: block states and the remaining state of each query block */
#define SAGESLA_STAGE_ATTN 3     /* block-sparse INT8 attention, then per query block the linear branch's
                                    contraction with phi(Q) and W_p and the output (one kernel) */
#define SAGESLA_NUM_STAGES 4

/* flags */
#define SAGESLA_LINEAR 0x1u         /* run the linear branch on the non-selected blocks (needs w_proj)      */
#define SAGESLA_SMOOTH_K 0x2u       /* subtract the per-channel mean of K over all N tokens before quantizing */
#define SAGESLA_USE_GIVEN_MASK 0x4u /* sagesla_forward reads block_idx instead of selecting (block_idx required) */
#define SAGESLA_QUANT_GROUP32 0x8u  /* one INT8 scale per 32 tokens of Q and of K instead of one per block: the
                                       "thread-level" granularity of [TD-news] §三(一) item 2, each 32×32 tile of
                                       scores with its own pair of scales (q_scale/k_scale then hold n_g values) */
#define SAGESLA_QK_RMSNORM 0x10u    /* first normalize Q and K, per token over all H*D channels of its heads, by
                                       RMSNorm with the weights q_norm_w / k_norm_w ([TD-news] §三(四) item 2,
                                       point 1); every later step sees the normalized values (see sagesla_quantize) */

typedef struct sagesla_params {
  int32_t B, H, N, D;   /* batch, heads, tokens, head dim (D == 128)                                       */
  int32_t blk_q, blk_k; /* query block 64 or 128; key block 64                                             */
  int32_t topk;         /* key blocks kept per query block, 0..n_kb (n_kb = ceil(N / blk_k))               */
  uint32_t flags;       /* SAGESLA_* bits                                                                  */
  float sm_scale;       /* softmax scale on the dequantized scores; 0 means 1/sqrt(D)                      */
  const void* w_proj;   /* bf16 [D][D] row-major projection of the linear branch: out_row += o_l_row · W_p  */
  void* workspace;      /* device scratch of workspace_bytes bytes, 256-byte aligned                        */
  size_t workspace_bytes;
  /* Optional intermediates (device, caller-owned). NULL keeps an intermediate inside the workspace; a
     non-NULL pointer makes the library write it there (and read it back from there in later stages).     */
  int8_t* q_i8;       /* [B][H][N][D]      INT8 codes of Q                                                */
  float* q_scale;     /* [B][H][n_qb]      per query block: fp32(absmax/127), 0 for an all-zero block;
                         [B][H][n_g] per 32 tokens with SAGESLA_QUANT_GROUP32 (n_g = ceil(N / 32))        */
  int8_t* k_i8;       /* [B][H][N][D]      INT8 codes of the smoothed K                                   */
  float* k_scale;     /* [B][H][n_kb]      (or [B][H][n_g] with SAGESLA_QUANT_GROUP32)                      */
  float* k_mean;      /* [B][H][D]         fp32(sum_t K[t][c] / N), zeros without SAGESLA_SMOOTH_K         */
  double* q_pool;     /* [B][H][n_qb][D]   mean of the raw Q rows of each query block                     */
  double* k_pool;     /* [B][H][n_kb][D]   mean of the smoothed K rows of each key block                  */
  int32_t* block_idx; /* [B][H][n_qb][topk] selected key blocks, ascending (input with USE_GIVEN_MASK: distinct) */
  float* o_lin;       /* [B][H][N][D]      linear-branch output after the projection (fp32)               */
  /* Optional timing: NULL, or 2*SAGESLA_NUM_STAGES caller-created hipEvent_t handles (as void*). sagesla_forward
     records events[2s] on `stream` just before stage s and events[2s+1] just after it (both at the same point
     when the stage has nothing to do). The caller owns the events and reads them after synchronizing.       */
  void* const* events;
  /* RMSNorm of Q and K (SAGESLA_QK_RMSNORM): bf16 [H*D] weights, indexed h*D + d (required with the flag), and
     eps (finite, >= 0). q_hat / k_hat: optional exports [B][H][N][D] bf16 of the normalized Q and K. */
  const void* q_norm_w;
  const void* k_norm_w;
  void* q_hat;
  void* k_hat;
  float norm_eps;
  /* sagesla_backward with SAGESLA_QK_RMSNORM (required there, ignored elsewhere): fp32 [H*D] outputs, dL/d of the
     norm weights of Q and of K (summed over every token of every batch entry). */
  float* dq_norm_w;
  float* dk_norm_w;
  /* Optional export (device, caller-owned, 16-byte aligned): [B][H][n_qb][n_kb] fp64, the block scores
     q_pool[I] . k_pool[J] that the top-k ranks ([TD-news] §三(二) item 1; the 1/sqrt(D) factor and a softmax
     over J leave the ranking unchanged and are not applied). Written only when the selection runs
     (0 < topk < n_kb and no SAGESLA_USE_GIVEN_MASK). */
  double* scores;
} sagesla_params;

/* Bytes of workspace the three entry points need for these parameters (all intermediates kept inside).
   Only sizes, block shapes and flags are read (pointers may be NULL). Returns 0 when those are invalid.
   Host only; no device access. */
size_t sagesla_workspace_bytes(const sagesla_params* p);

/* Host-side validation of a parameter block (sizes, flags, w_proj presence and the alignment of every pointer
   it carries; not the tensors passed separately): SAGESLA_OK or the first error found. */
sagesla_status sagesla_validate(const sagesla_params* p);

/* Quantize stage ([TD-news] §三(一) items 1–2).
   Reads q, k (bf16 [B][H][N][D]). With SAGESLA_QK_RMSNORM these are first replaced by their normalized
   values: per (b, token n), S = the sum of x^2 over the H*D channels of q[b][:][n][:] (fp64; exact, and so
   order-independent, when every partial sum is representable), r = fp32(1 / sqrt(S / (H*D) + eps)) (fp64
   division, addition, square root and reciprocal, each correctly rounded, then one rounding to fp32), and
   x_hat = bf16_rne(fp32(bf16_rne(fp32(x * r)) * w[h*D + d])); likewise k with k_norm_w. Everything below then
   applies to q_hat and k_hat (the K mean, codes and pooled means here; the selection, both attention branches
   in sagesla_forward). With SAGESLA_SMOOTH_K, k_mean = fp32(exact column sum / N) per (b, h) and
   K is smoothed to k' = fp32(K - k_mean); otherwise k' = K. Per block of blk_q query rows (blk_k key rows) × D
   channels, the last block holding only the remaining rows: scale = fp32(absmax/127) and
   code = clamp(round-half-even(fp32(x / scale)), -127, 127) for Q and for k'; with SAGESLA_QUANT_GROUP32 the
   same per group of 32 rows (the last group holding the remaining rows). Also writes q_pool/k_pool, the block
   means of raw Q and of k' (fp64). Codes, scales and k_mean are bit-exact functions of the inputs. */
sagesla_status sagesla_quantize(const void* q, const void* k, const sagesla_params* p, void* stream);

/* Select stage ([TD-news] §三(二) item 1; [TD-guide] --sla_topk).
   Needs the pooled means written by sagesla_quantize with the same params and workspace. For every query
   block I, ranks key blocks J by the fp64 score q_pool[I] · k_pool[J] (the /sqrt(D) does not change the
   order), keeps the topk best with exact ties going to the lower J, and writes them ascending to block_idx. */
sagesla_status sagesla_select(const sagesla_params* p, void* stream);

/* Whole forward ([TD-news] §三(二) item 3: select first, then INT8 attention on the selected blocks, linear
   attention on the rest). Runs quantize, select (or reads block_idx with SAGESLA_USE_GIVEN_MASK: each row must
   hold topk distinct key blocks in [0, n_kb), in any order, which the select stage's own lists always do; a row
   that repeats a block is outside this contract, and out-of-range indices are clamped, which can repeat one),
   the linear branch (SAGESLA_LINEAR) and the sparse attention, and writes
   out = bf16_rne(O_s + O_lin):
     O_s[i]  = softmax over the selected keys j of z_ij = (codeQ_i · codeK_j) · scale_q(i) · scale_k(j) · sm_scale,
               where scale_q(i) / scale_k(j) is the scale of the block (or, with SAGESLA_QUANT_GROUP32, of the
               32-row group) holding row i / j, applied to the bf16 value rows (0 when topk == 0);
     O_lin   = O_l · W_p, O_l[i] = phi(q_i) H_m / (phi(q_i) · Z_m), phi = elu + 1 on the raw bf16 q and k,
               H_m / Z_m = the sum over all key blocks of phi(K_J)^T V_J / sum phi(K_J) minus the same sums over
               the selected blocks (0 when every key block is selected). */
sagesla_status sagesla_forward(const void* q, const void* k, const void* v, void* out, const sagesla_params* p,
                               void* stream);

/* SLA backward for a fixed selection (SLA is trainable: [TD-news] §三(二), fine-tuned with the model in §四).
   Computes the gradient of the float forward
     out = O_s + O_lin, O_s = softmax over the listed key blocks of q . k * sm_scale applied to v, O_lin as above,
   with INT8 quantization passed straight through and the K-mean shift dropped (it changes no softmax row), for
   the selection in block_idx (required when topk > 0; each row holds topk distinct key blocks in [0, n_kb), in
   any order, as for SAGESLA_USE_GIVEN_MASK in sagesla_forward). dout: bf16 [B][H][N][D] = dL/d(out). Writes dq, dk, dv: fp32 [B][H][N][D], and with SAGESLA_LINEAR
   dw_proj: fp32 [D][D], dL/dW_p summed over every (b, h) (zeros when every block is selected). Accumulation is
   fp32 in a fixed order (deterministic); every product runs on bf16 MFMA with each operand that is not exactly
   bf16 (P, dS, phi of q and k, the linear branch's states and intermediates) split into bf16 hi + lo pairs; the
   linear branch starts from the forward's remaining state (bf16 hi + lo).
   With SAGESLA_QK_RMSNORM the attention's gradient is taken at the normalized Q and K the forward uses (their
   bf16 roundings pass gradients unchanged, like the quantization) and carried through the norm: dq and dk are then
   the gradients of the raw inputs, and dq_norm_w, dk_norm_w (required) receive those of the norm weights.
   SAGESLA_SMOOTH_K and SAGESLA_QUANT_GROUP32 do not change the result. The workspace must hold
   sagesla_backward_workspace_bytes(p) bytes. */
size_t sagesla_backward_workspace_bytes(const sagesla_params* p);
sagesla_status sagesla_backward(const void* q, const void* k, const void* v, const void* dout, float* dq, float* dk,
                                float* dv, float* dw_proj, const sagesla_params* p, void* stream);

/* The forward for callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
   harnesses that forbid hipMalloc): the same computation and results as sagesla_forward, with the workspace
   taken from a device array of SAGESLA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
   (p->workspace and p->workspace_bytes are ignored). The caller still passes q, k, v, out and any exports.
   Returns SAGESLA_E_WORKSPACE when sagesla_workspace_bytes(p) exceeds that size. Calls no allocating routine;
   the first call on a device looks up the array's address there (with that device current). Every call on one
   GPU shares its array, so calls that overlap on one GPU (other streams, other host threads) race. */
#define SAGESLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sagesla_status sagesla_forward_noalloc(const void* q, const void* k, const void* v, void* out,
                                       const sagesla_params* p, void* stream);

/* Text of a status code (static storage). */
const char* sagesla_status_str(sagesla_status s);

/* hipError_t of the most recent SAGESLA_E_HIP in the calling thread (0 if none; a later success does not clear it).
 *
 * Launches are asynchronous: SAGESLA_E_HIP from an entry point reports a failed launch, and a fault while a kernel
 * runs surfaces at a later synchronizing HIP call. With the environment variable SAGESLA_DEBUG set to a value other
 * than "" or "0" (read once, at the first launch of the process), every entry point synchronizes its stream after
 * each stage's launches and returns SAGESLA_E_HIP for a fault of that stage, naming the stage's launcher on
 * stderr. Debug mode blocks the host after every stage and must not be used while the stream is being captured. */
int sagesla_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SAGESLA_H */
