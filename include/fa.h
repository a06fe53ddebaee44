/*
 * fa.h -- C ABI of an exact scaled-dot-product attention library for AMD
 * MI355X (gfx950).  Forward and backward passes run as hand-written HIP
 * kernels; this header has no HIP, C++ or framework types in it.
 *
 * What is computed (forward).  For every batch b and query head h, with
 * key/value head g = h / (H_q / H_kv):
 *
 *     S  = scale * Q[b,h] K[b,g]^T            (N x N scores; with causal,
 *                                              S[i][j] = -inf for j > i)
 *     P  = row-softmax(S)
 *     O[b,h]   = P V[b,g]
 *     LSE[b,h][i] = ln sum_j exp(S[i][j])     (natural log)
 *
 * Sources: the standard attention walk-through (Steps 1-3) of the page
 * "Flash attention: fast and memory-efficient exact attention with
 * IO-awareness -- a deep dive"; the scale factor from "Optimizing memory
 * usage on GPUs with flash attention mechanisms", section "Mechanics of Flash
 * Attention"; grouped-query / multi-query head sharing and head dims up to
 * 256 from "The Future of AI: How FlashAttention Revolutionizes Deep
 * Learning", section "FlashAttention-2: Enhanced Performance".  The kernels
 * evaluate it block by block with the running-max / running-sum recurrence
 * given in the softmax answer of the FlashAttention interview Q&A
 * (app.wittybyte.ai, "FlashAttention1"); the N x N matrices never reach
 * device memory, and LSE is the per-row statistic kept for the backward
 * pass (deep-dive page, "Intuition" under the softmax mathematics).
 * The causal mask (j > i hidden, diagonal kept) and the natural-log LSE are
 * readings: the pages do not define them.
 *
 * Memory layout.  All tensors are dense, row-major and contiguous:
 *     Q, O, dO, dQ : [B][H_q ][N][d]
 *     K, V, dK, dV : [B][H_kv][N][d]
 *     LSE          : [B][H_q ][N]      always float32
 * Elements of Q, K, V, O, dO, dQ, dK, dV are bfloat16 (FA_BF16) or float32
 * (FA_FP32).  bfloat16 results are rounded to nearest even once, from
 * float32 accumulators.
 *
 * Ownership and execution.  Every pointer argument is a DEVICE pointer owned
 * by the caller; the library never allocates, frees or keeps a pointer after
 * the call returns.  Work is enqueued on ``stream`` (a hipStream_t; NULL is
 * the default stream) and the call returns without synchronising: outputs
 * are valid once the stream reaches that point, and the caller keeps every
 * buffer alive until then.  Outputs must not alias inputs.  Calls are
 * thread-safe (the only shared state is a per-device property cache filled
 * once).
 *
 * Errors.  Arguments are validated on the host before anything is enqueued;
 * on an error nothing is launched and a negative FA_ERR_* code is returned.
 * A failed HIP call returns FA_ERR_HIP; fa_last_hip_error() then gives the
 * hipError_t value (thread-local).  fa_status_str() names a status code.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of Q, K, V, O, dO, dQ, dK, dV (LSE is always float32) */
enum fa_dtype { FA_BF16 = 0, FA_FP32 = 1 };

/* status codes */
enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = -1,        /* a required pointer is NULL                      */
    FA_ERR_SHAPE = -2,       /* B, H_q, H_kv or N out of range, or H_q % H_kv   */
    FA_ERR_HEADDIM = -3,     /* d not in {64, 128, 256}                         */
    FA_ERR_DTYPE = -4,       /* dtype is not an fa_dtype value                  */
    FA_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                */
    FA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required         */
    FA_ERR_UNSUPPORTED = -7, /* valid arguments, no kernel for this combination */
    FA_ERR_HIP = -8,         /* a HIP runtime call failed (fa_last_hip_error)   */
    FA_ERR_ARG = -9          /* causal not 0/1, scale not finite, or a count
                                out of range                                    */
};

/* Largest sequence length and head count accepted (index arithmetic in the
 * kernels is 64-bit for element offsets; these bound the grid). */
#define FA_MAX_N (1 << 22)
#define FA_MAX_HEADS 65535
/* Largest number of key ranges (partial results) of the split forward and
 * of the merge. */
#define FA_MAX_SPLITS 4096
/* Block-sparse attention: positions per block of the block map, and the
 * longest sequence its entry points accept. */
#define FA_SPARSE_BLOCK 128
#define FA_SPARSE_MAX_N 65536
/* Largest B * H_q * N of fa_bwd_noalloc (8 MiB of float32 D_i terms). */
#define FA_NOALLOC_MAX_ROWS (1 << 21)

/*
 * fa_fwd -- forward pass.
 *   Q [B,H_q,N,d], K [B,H_kv,N,d], V [B,H_kv,N,d]   inputs (dtype)
 *   O [B,H_q,N,d]                                    output (dtype)
 *   LSE [B,H_q,N]                                    output (float32), may be
 *                                                    NULL when not wanted
 *   B >= 0, N >= 0 (B == 0 or N == 0: nothing to do, returns FA_OK and
 *   pointers may be NULL), 1 <= H_kv <= H_q <= FA_MAX_HEADS, H_q % H_kv == 0,
 *   N <= FA_MAX_N, d in {64, 128, 256}, causal in {0, 1}, scale finite with
 *   |scale| * log2(e) finite in float (|scale| < 2.35e38; else FA_ERR_ARG).
 *   N needs no relation to any tile size.  All pointers 16-byte aligned.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int B, int H_q, int H_kv, int N, int d, float scale, int causal,
           int dtype, void* stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs for these
 * sizes (0 when there is nothing to do).  The workspace holds the per-row
 * term D_i = sum_c dO[i][c] O[i][c] (float32 [B,H_q,N]), rounded up to 256
 * bytes.  For bf16 with grouped heads (H_q > H_kv) whose dK/dV grid would
 * leave compute units idle, each key/value head's query heads are split
 * over S workgroups (S a power of two dividing H_q / H_kv, chosen from the
 * current device's compute-unit count), and the workspace also holds their
 * float32 partial dK and dV, 2 x S*B*H_kv*N*d*4 bytes (each rounded up to
 * 256), summed in slice order.  Query it with the device that will run the
 * backward current; the same sizes give the same answer on that device.
 */
size_t fa_bwd_workspace_size(int B, int H_q, int H_kv, int N, int d, int dtype);

/*
 * fa_bwd -- backward pass with on-chip recomputation of the scores.
 *   Q, K, V                 the forward inputs
 *   O, LSE                  the forward outputs of fa_fwd with the same
 *                           scale, causal flag and dtype (LSE required here)
 *   dO [B,H_q,N,d]          gradient of the loss with respect to O
 *   dQ [B,H_q,N,d], dK, dV [B,H_kv,N,d]
 *                           outputs, OVERWRITTEN (not accumulated into); for
 *                           grouped heads dK/dV of a key/value head are the
 *                           sums over the query heads of its group
 *   workspace               device buffer of at least
 *                           fa_bwd_workspace_size(...) bytes, 256-byte
 *                           aligned; contents on entry are ignored
 * The backward recomputes P from Q, K and LSE instead of storing it (page
 * "The Future of AI ...", section "Understanding FlashAttention",
 * recomputation).  The gradient formulas are the analytic derivative of the
 * forward definition (the pages print none):
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij = dO_i . O_i,
 *   dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 * Shapes and constraints as fa_fwd; d in {64, 128} for FA_BF16 (d = 256
 * returns FA_ERR_UNSUPPORTED).
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O,
           const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
           void* workspace, size_t workspace_bytes,
           int B, int H_q, int H_kv, int N, int d, float scale, int causal,
           int dtype, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, result and errors as fa_bwd, without the
 * workspace: the D_i term goes to a fixed buffer inside the library (one
 * per device, FA_NOALLOC_MAX_ROWS floats, kept until the process ends).
 * Nothing is allocated or freed by the call.  Sizes with
 * B * H_q * N > FA_NOALLOC_MAX_ROWS return FA_ERR_WORKSPACE (use
 * fa_bwd).  Calls on one device share that buffer: calls that may overlap
 * in time on one device (different streams, or different host threads
 * without ordering) race and give unspecified gradients; calls ordered on
 * one stream are safe.  The buffer's contents are rewritten before use, so
 * nothing carries over between calls.
 */
int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                   int B, int H_q, int H_kv, int N, int d, float scale, int causal,
                   int dtype, void* stream);

/*
 * Local (sliding-window) attention.  The pages name local and sparse
 * attention as a combination with the method (FlashAttention interview Q&A,
 * app.wittybyte.ai "FlashAttention1": sparse attention such as local
 * attention for very long sequences; sparse FlashAttention as a future
 * direction) but define no pattern.  Reading: with the window
 * (window_left, window_right), query i sees key j exactly when
 *     i - window_left <= j <= i + window_right,
 * -1 meaning unbounded on that side: (-1, 0) is fa_fwd's causal mask,
 * (-1, -1) no mask.  Every row sees at least its own key.  Key tiles wholly
 * outside a query block's windows are not visited.
 *
 * fa_fwd_window / fa_bwd_window -- as fa_fwd / fa_bwd with the window in
 * place of the causal flag; window_left, window_right >= -1 (else
 * FA_ERR_ARG).  fa_bwd_window must get O and LSE of fa_fwd_window with the
 * same window.  Same shapes, dtypes and constraints as fa_fwd / fa_bwd.
 */
int fa_fwd_window(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  int B, int H_q, int H_kv, int N, int d, float scale,
                  int window_left, int window_right, int dtype, void* stream);
int fa_bwd_window(const void* Q, const void* K, const void* V, const void* O,
                  const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                  void* workspace, size_t workspace_bytes,
                  int B, int H_q, int H_kv, int N, int d, float scale,
                  int window_left, int window_right, int dtype, void* stream);

/*
 * Block-sparse attention.  The deep-dive page ("Flash attention: fast and
 * memory-efficient exact attention with IO-awareness -- a deep dive") names
 * block-sparse FlashAttention in its closing paragraph, and the interview
 * Q&A (app.wittybyte.ai, "FlashAttention1", scaling answer) suggests sparse
 * patterns for very long sequences; neither defines a layout.  Reading: the
 * sequence is cut into blocks of FA_SPARSE_BLOCK = 128 positions; the map
 *   block_mask  uint8 [nb][nb], nb = ceil(N / 128), DEVICE memory, one map
 *               for every batch entry and head (nonzero = visible)
 * lets query i see key j exactly when block_mask[i / 128][j / 128] != 0,
 * and with causal = 1 also j <= i.  Key tiles of hidden blocks are neither
 * loaded nor computed.  A query row that sees no key gets O = 0 and
 * LSE = -inf and adds nothing to dK / dV; its dQ row is 0.
 *
 * fa_fwd_blocksparse / fa_bwd_blocksparse -- as fa_fwd / fa_bwd plus the
 * map; fa_bwd_blocksparse must get O and LSE of fa_fwd_blocksparse with the
 * same map, scale and causal flag (workspace: fa_bwd_workspace_size).
 * FA_BF16 with d in {64, 128} and N <= FA_SPARSE_MAX_N; other valid
 * combinations return FA_ERR_UNSUPPORTED.  block_mask NULL: FA_ERR_NULL.
 * The host does not read the map (no synchronisation); it must hold nb * nb
 * bytes.
 */
int fa_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                       const unsigned char* block_mask, int B, int H_q, int H_kv, int N, int d,
                       float scale, int causal, int dtype, void* stream);
int fa_bwd_blocksparse(const void* Q, const void* K, const void* V, const void* O,
                       const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                       void* workspace, size_t workspace_bytes, const unsigned char* block_mask,
                       int B, int H_q, int H_kv, int N, int d, float scale, int causal,
                       int dtype, void* stream);

/*
 * Dropout on the attention probabilities.  The deep-dive page ("Flash
 * attention: fast and memory-efficient exact attention with IO-awareness --
 * a deep dive", "Computing and memory basics", quantitative evidence) names
 * dropout with softmax and masking as the steps that dominate unfused
 * attention; it gives no formula or generator.  Reading (inverted dropout on
 * P, with a counter-based generator so that the backward regenerates the
 * forward's mask instead of storing it):
 *   O = (P o Z) V / (1 - p8),   LSE as without dropout,
 *   dV = (P o Z)^T dO / (1 - p8),  dP = (dO V^T) o Z / (1 - p8),
 *   dS = P o (dP - D) with D_i = dO_i . O_i,  dQ, dK as fa_bwd.
 * The mask: t8 = round(dropout_p * 256) (half to even), p8 = t8 / 256; the
 * 4 x 4 block of queries 4a..4a+3 and keys 4c..4c+3 of batch b and query
 * head h takes the four 32-bit words of Philox-4x32-10 (J. K. Salmon et al.,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011) with
 *   key (seed & 0xFFFFFFFF, seed >> 32), counter (c, a, b * H_q + h, offset);
 * word i % 4 belongs to query i, its byte j % 4 (bits 8 (j % 4) .. +7) to key
 * j, and Z_ij = 1 when that byte >= t8.
 *
 * fa_fwd_dropout / fa_bwd_dropout -- as fa_fwd / fa_bwd plus dropout_p
 * (0 <= dropout_p, rounding to t8 <= 255, else FA_ERR_ARG; t8 = 0 is plain
 * attention), seed and offset.  fa_bwd_dropout must get O and LSE of
 * fa_fwd_dropout with the same dropout_p, seed, offset, scale and causal
 * flag.  FA_BF16 with d in {64, 128}; other valid combinations return
 * FA_ERR_UNSUPPORTED.
 */
int fa_fwd_dropout(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int H_q, int H_kv, int N, int d, float scale, int causal,
                   float dropout_p, unsigned long long seed, unsigned int offset,
                   int dtype, void* stream);
int fa_bwd_dropout(const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                   void* workspace, size_t workspace_bytes,
                   int B, int H_q, int H_kv, int N, int d, float scale, int causal,
                   float dropout_p, unsigned long long seed, unsigned int offset,
                   int dtype, void* stream);

/*
 * Packed variable-length batches.  The interview Q&A page (app.wittybyte.ai,
 * "FlashAttention1", scaling-challenges answer) names uneven work across the
 * GPU's cores for variable sequence lengths and gives no layout.  Reading:
 * the batch's sequences are packed back to back, per head, with no padding:
 *   Q, O      [H_q, total, d]     K, V   [H_kv, total, d]
 *   LSE       float32 [H_q, total]   (fa_fwd_varlen: may be NULL)
 *   cu_seqlens  int32 [batch + 1], DEVICE memory: cu[0] = 0, non-decreasing,
 *               cu[batch] = total; sequence b is rows cu[b] .. cu[b+1]-1 of
 *               every head
 *   max_seqlen  >= every cu[b+1] - cu[b], <= FA_MAX_N (sizes the grid)
 * Each sequence is attended to on its own, exactly as one batch entry of
 * fa_fwd / fa_bwd (causal: within the sequence); no query sees a key of
 * another sequence.  An empty sequence is allowed.  dQ is shaped as Q, dK and
 * dV as K; the backward workspace holds H_q * total floats
 * (fa_bwd_varlen_workspace_size).
 * The host cannot read cu_seqlens, so it is not checked: the kernels clamp
 * each offset into [0, total] and each length to max_seqlen, which keeps
 * every access inside the buffers above, but offsets that break the rules
 * give unspecified values (rows past max_seqlen of a longer sequence, and
 * rows outside every sequence, are not written).
 * batch == 0, total == 0 or max_seqlen == 0: nothing to do (FA_OK).  Other
 * constraints (heads, d, dtype, alignment, d = 256 backward) as fa_fwd /
 * fa_bwd; cu_seqlens must be 4-byte aligned; total < 0 is FA_ERR_SHAPE.
 */
int fa_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  const int* cu_seqlens, int batch, int total, int max_seqlen,
                  int H_q, int H_kv, int d, float scale, int causal, int dtype, void* stream);
/* Bytes of device workspace fa_bwd_varlen needs; 0 when total <= 0 or the
 * arguments are invalid. */
size_t fa_bwd_varlen_workspace_size(int total, int H_q, int H_kv, int d, int dtype);
int fa_bwd_varlen(const void* Q, const void* K, const void* V, const void* O,
                  const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                  void* workspace, size_t workspace_bytes, const int* cu_seqlens,
                  int batch, int total, int max_seqlen, int H_q, int H_kv, int d,
                  float scale, int causal, int dtype, void* stream);

/*
 * Split key/value forward: N_q queries against N_k keys, the keys cut into
 * ranges whose partial results are merged -- for decoding steps and other
 * inputs with few queries per head (N_q much smaller than N_k) or few
 * (batch, head) units, where one workgroup per query block would leave the
 * GPU idle.
 *
 * Partial results over disjoint blocks of keys combine exactly: a block
 * keeps its maximum and sum of exponentials, and blocks combine by
 * rescaling to the larger maximum (FlashAttention interview Q&A,
 * app.wittybyte.ai "FlashAttention1", softmax answer; the same page names
 * combining partial results of different blocks and incremental attention
 * among what the method enables).  With a partial kept as
 * (O_p = its own softmax-weighted V, LSE_p = ln of its sum of exponentials):
 *     LSE = ln sum_p exp(LSE_p),      O = sum_p exp(LSE_p - LSE) O_p.
 *
 * Result: the same attention as fa_fwd, generalised to N_q != N_k:
 *     Q [B,H_q,N_q,d], K, V [B,H_kv,N_k,d], O [B,H_q,N_q,d], LSE [B,H_q,N_q]
 * With causal = 1 the queries are the LAST N_q positions of the key
 * sequence: key j is hidden from query i when j > i + N_k - N_q (a reading;
 * the pages define no mask).  N_q = N_k gives fa_fwd's mask; N_q = 1 sees
 * every key.  A query that sees no key (N_q > N_k, causal) gets O = 0 and
 * LSE = -inf.
 */

/* Number of key ranges fa_fwd_split uses: num_splits if > 0, else a default
 * that gives every SIMD of the GPU work; 0 when there is nothing to do or
 * the arguments are invalid. */
int fa_fwd_split_parts(int B, int H_q, int H_kv, int N_q, int N_k, int d, int num_splits);

/* Bytes of device workspace fa_fwd_split needs (the float32 partials:
 * parts x B*H_q*N_q x (d + 1) values, each array 256-byte aligned); 0 when
 * there is nothing to do or the arguments are invalid. */
size_t fa_fwd_split_workspace_size(int B, int H_q, int H_kv, int N_q, int N_k, int d, int num_splits, int dtype);

/*
 * fa_fwd_split -- split key/value forward, then the merge, on ``stream``.
 *   Q, K, V, O, LSE    as above; LSE may be NULL; all 16-byte aligned
 *   num_splits         key ranges (0: fa_fwd_split_parts default), at most
 *                      FA_MAX_SPLITS; ranges past N_k are empty (no cost
 *                      but their partial, which merges as nothing)
 *   workspace          at least fa_fwd_split_workspace_size(...) bytes,
 *                      256-byte aligned; contents on entry are ignored
 *   B >= 0, N_q >= 0 (B == 0 or N_q == 0: nothing to do, FA_OK), N_k >= 1,
 *   N_q, N_k <= FA_MAX_N, heads as fa_fwd, causal in {0, 1}, scale as fa_fwd.
 *   dtype FA_BF16 and d in {64, 128}; other valid combinations return
 *   FA_ERR_UNSUPPORTED.
 */
int fa_fwd_split(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int B, int H_q, int H_kv, int N_q, int N_k, int d, float scale, int causal,
                 int num_splits, void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * fa_lse_merge -- merge partial results (the combine step of fa_fwd_split,
 * also usable for partials computed elsewhere, e.g. on other devices).
 *   O_parts   float32 [num_parts][rows][d]   each part's output, normalised
 *                                            by its own sum of exponentials
 *   LSE_parts float32 [num_parts][rows]      each part's LSE (natural log;
 *                                            -inf: the part saw no key)
 *   O         [rows][d] of dtype (FA_BF16 or FA_FP32)    output
 *   LSE       float32 [rows]                 output, may be NULL
 *   1 <= num_parts <= FA_MAX_SPLITS, rows >= 0 (0: nothing to do),
 *   d in {64, 128, 256}; pointers 16-byte aligned.  A row whose parts are
 *   all -inf gets O = 0, LSE = -inf.
 */
int fa_lse_merge(const float* O_parts, const float* LSE_parts, int num_parts, long long rows, int d,
                 void* O, float* LSE, int dtype, void* stream);

/* Name of a status code ("FA_OK", "FA_ERR_SHAPE", ...); never NULL. */
const char* fa_status_str(int status);

/* hipError_t value behind the last FA_ERR_HIP returned on this thread
 * (0 when none). */
int fa_last_hip_error(void);

/* Library ABI version (major * 100 + minor). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
