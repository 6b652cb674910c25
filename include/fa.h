/*
 * fa.h - exact, IO-aware attention on AMD Instinct MI355X (gfx950).
 *
 * Computes O = softmax(scale * Q K^T [masked]) V without ever writing the N x N
 * score (S) or probability (P) matrices to device memory, and its gradients,
 * which recompute P from the saved per-row logsumexp.
 *
 * Sources (three web pages on FlashAttention):
 *   - lecture summary on FlashAttention v1 (spark.aweffr.cn), section 2.1: the
 *     attention formula softmax(Q K^T / sqrt(d_k)) V; section 3.2: the one-pass
 *     online softmax; section 3.3: the tiled forward; part 4.2: the backward
 *     recomputes S and P from the saved statistics.
 *   - FlashAttention-2 overview (jishu.shishitao.com), "main operations": the
 *     backward needs only the row logsumexp; the forward gives each worker one
 *     block of query rows; the backward gives each worker one block of key
 *     columns and merges dQ by atomic addition (here dQ has a pass of its own
 *     instead, see fa_bwd); block-sparse attention skips zero blocks
 *     ("Block-Sparse FlashAttention").
 *
 * Conventions shared by every entry point:
 *   Layout     Q, K, V, O, dO, dQ, dK, dV are [B, H, N, d] bfloat16, contiguous,
 *              d fastest. lse is [B, H, N] float32 (natural-log logsumexp of the
 *              scaled, masked scores of each query row).
 *   Memory     every data pointer is a DEVICE pointer owned by the caller; the
 *              library allocates nothing; its only global state is the
 *              fixed device array of fa_bwd_noalloc (and its cached address).
 *              Inputs are read-only; outputs must not overlap any input.
 *   Alignment  data pointers must be 16-byte aligned.
 *   Limits     B, H, N >= 0 (a zero extent is a no-op that returns FA_OK);
 *              d in {64, 128}; scale finite and > 0; B*H*N*d < 2^40;
 *              N <= 2^31 - 1025 (B*H <= 2^31 - 1 follows);
 *              4*B*H*ceil(N / 256)*256 <= 2^32 - 1, so that no launch asks
 *              for 2^32 work-items or more (a dispatch counts them in 32 bits).
 *              N need not be a multiple of any tile size. With a block mask,
 *              ceil(N / 128) <= 16384 (N <= 2^21).
 *   Streams    `stream` is a hipStream_t passed as void* (NULL = default
 *              stream). Every call only enqueues work and returns; results are
 *              ready after the caller synchronises the stream. Device faults
 *              surface at that synchronisation.
 *   Errors     argument checks run on the host before anything is enqueued and
 *              return a negative fa_status; nothing is written then. A failed
 *              kernel launch returns FA_ERR_HIP.
 *   Determinism every output is bitwise reproducible run to run (no atomics).
 */
#ifndef EXACT_IO_AWARE_FA_H
#define EXACT_IO_AWARE_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a required pointer is NULL                            */
  FA_ERR_SHAPE = -2,     /* B/H/N negative, d unsupported, or sizes overflow       */
  FA_ERR_MASK = -3,      /* unknown mask kind, block != 128, NULL grid, N > 2^21  */
  FA_ERR_ALIGN = -4,     /* a data pointer is not 16-byte aligned                  */
  FA_ERR_WORKSPACE = -5, /* backward workspace missing or too small                */
  FA_ERR_HIP = -6,       /* the HIP runtime reported an error at launch            */
  FA_ERR_SCALE = -7,     /* scale is not finite and > 0                            */
  FA_ERR_ALIAS = -8,     /* an output range overlaps an input range                */
  FA_ERR_SCRATCH = -9    /* problem too large for fa_bwd_noalloc's fixed scratch   */
} fa_status;

/* Mask kinds (bit flags; 0 = every key visible to every query). */
#define FA_MASK_CAUSAL 1 /* query i sees key j iff j <= i                                     */
#define FA_MASK_BLOCK 2  /* query i sees key j iff blocks[i / 128][j / 128] != 0              */

/*
 * Mask description. Block-sparse attention (FlashAttention-2 overview, section
 * "Block-Sparse FlashAttention") keeps or drops whole blocks of the score
 * matrix; blocks whose entry is 0 are skipped entirely and contribute exactly
 * zero to O and to every gradient. Both flags may be combined (logical AND).
 */
typedef struct fa_mask {
  int32_t kind;           /* OR of FA_MASK_* flags                                       */
  int32_t block;          /* block edge in rows/keys; must be 128 when FA_MASK_BLOCK is set */
  const uint8_t* blocks;  /* DEVICE pointer, uint8 [nb][nb] row-major, nb = ceil(N / 128); */
                          /* nonzero = keep. Read-only. Ignored unless FA_MASK_BLOCK.       */
  int64_t bh_stride;      /* elements between the grids of consecutive (b, h); 0 = one grid */
                          /* shared by every (b, h), else grid of (b, h) at blocks + (b*H+h)*bh_stride */
} fa_mask_t;

/*
 * Forward: O = softmax(scale * Q K^T, masked) V and lse = row logsumexp.
 * Tiled with the online softmax (lecture summary, section 3.2; FlashAttention-2
 * overview, forward pass): one workgroup per (b, h, block of query rows), a
 * running max and denominator per row kept on chip, normalisation deferred to
 * the end. A row with no visible key gets O = 0 and lse = -inf.
 *   q, k, v : inputs [B, H, N, d] bf16
 *   o       : output [B, H, N, d] bf16 (round-to-nearest-even)
 *   lse     : output [B, H, N] float32, natural log
 *   mask    : NULL = no mask
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, const fa_mask_t* mask, void* stream);

/*
 * Bytes of device workspace fa_bwd needs, written to *bytes (pure host
 * arithmetic). The workspace holds two per-row float32 arrays [B, H, Np]
 * (Np = N rounded up to a multiple of 128), each 256-byte aligned: the row
 * terms D_i = dO_i . O_i and LSE_i log2(e) (+inf for rows past N and rows that
 * see no key). That is about 8 bytes per query row.
 */
int fa_bwd_workspace_size(int B, int H, int N, int d, size_t* bytes);

/*
 * Backward: dQ, dK, dV of L given dO = dL/dO, recomputing P tile by tile from
 * q, k and the forward's lse (lecture summary, part 4.2). dK and dV come from
 * one workgroup per block of key columns (FlashAttention-2 overview, backward
 * pass); dQ, the only quantity those workgroups share, comes from its own pass
 * over blocks of query rows instead of an atomic merge, so every output is
 * bitwise reproducible.
 *   q, k, v, o, dout : inputs [B, H, N, d] bf16 (o from fa_fwd with the same arguments)
 *   lse              : input [B, H, N] float32 from fa_fwd
 *   dq, dk, dv       : outputs [B, H, N, d] bf16
 *   workspace        : DEVICE buffer of at least fa_bwd_workspace_size() bytes,
 *                      owned by the caller; its contents on entry do not matter
 *                      and are overwritten.
 * Enqueues the three stages below, in order.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, const fa_mask_t* mask,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The three stages of fa_bwd, exposed so a caller can time or schedule them
 * separately; calling them in order on one stream, with one workspace, equals
 * fa_bwd (dkdv and dq only read the workspace, so they may also run
 * concurrently once fa_bwd_preprocess has finished).
 *   fa_bwd_preprocess : D_i = sum_c dO_ic O_ic and LSE_i log2(e), from o, dout
 *                       and lse, into the workspace.
 *   fa_bwd_dkdv       : dK, dV (bf16), from q, k, v, dout and the workspace.
 *   fa_bwd_dq         : dQ (bf16), from q, k, v, dout and the workspace.
 * Argument meanings and checks are those of fa_bwd; the two gradient stages
 * take the row statistics from the workspace only, so scale and mask must be
 * those the gradients are wanted for (the preprocess needs neither).
 */
int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int H, int N,
                      int d, void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                int B, int H, int N, int d, float scale, const fa_mask_t* mask,
                void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
              int B, int H, int N, int d, float scale, const fa_mask_t* mask,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward in the loop order of the lecture summary's algorithm overview
 * (section 3.3; the first FlashAttention): O, l, m are kept in device memory
 * (the workspace, float32), the outer loop walks the K/V blocks and the inner
 * loop every Q block, reading and writing back O_i, l_i, m_i at each step with
 * the normalised online-softmax recurrence of section 3.2; one workgroup per
 * (b, h). Same result as fa_fwd (O bf16, lse natural log, causal = 0 or 1; no
 * block mask); it exists to measure the IO of that order against fa_fwd's
 * (query blocks outer, FlashAttention-2 overview), not for speed.
 *   workspace : DEVICE buffer of at least fa_fwd_kv_outer_workspace_size()
 *               bytes (O float32 [B, H, N, d], then m, l float32 [B, H, N],
 *               each part 256-byte aligned), contents irrelevant on entry
 * Arguments, limits and errors otherwise as fa_fwd.
 */
int fa_fwd_kv_outer_workspace_size(int B, int H, int N, int d, size_t* bytes);
int fa_fwd_kv_outer(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decoding against a key/value cache. The pages name inference with a KV cache
 * and FlashDecoding (lecture summary, remark after section 3.1, conclusion)
 * without defining them; what is computed is attention of the Nq newest
 * queries of each (b, h) over its Nk cached keys, query i sitting at position
 * Nk - Nq + i:
 *   O_i = sum_j softmax_j(scale q_i . k_j) v_j over the visible keys j,
 *   lse_i = ln sum_j e^(scale q_i . k_j)  (natural log),
 * where every key is visible, or with causal = 1 only keys j <= Nk - Nq + i
 * (aligned at the bottom right; the top-left rule of fa_fwd when Nq = Nk). A
 * query that sees no key gets O = 0 and lse = -inf. The keys are split into
 * chunks processed in parallel, each by the tiled online softmax of fa_fwd; a
 * second kernel merges the chunks' (max, denominator, output) states.
 *   q      : [B, H, Nq, d] bf16        k, v : [B, H, Nk, d] bf16 (the cache)
 *   o      : output [B, H, Nq, d] bf16  lse  : output [B, H, Nq] float32
 *   causal : 0 or 1 (other values: FA_ERR_MASK)
 *   workspace : DEVICE buffer of at least fa_decode_workspace_size() bytes,
 *               caller-owned, contents irrelevant on entry, overwritten
 * Limits: 0 <= Nq <= 32, 0 <= Nk <= 2^31 - 1025 (k and v may be NULL when Nk = 0),
 * d in {64, 128}, B*H*(Nq+Nk)*d < 2^40, B*H*Nq*d <= 2^32 - 1 and
 * 64*(B*H + 1024) <= 2^32 - 1 (work-items of the merge and the key split).
 * Errors and streams as above; outputs
 * and workspace must not overlap each other or any input.
 */
int fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d, size_t* bytes);
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Nq, int Nk, int d, float scale, int causal,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Row softmax with the online normalizer ("why attention is slow" page, section
 * on the online normalizer, attributed there to NVIDIA, 2018): for every row r,
 *   y[r][c] = e^(x[r][c] - m_r) / sum_c' e^(x[r][c'] - m_r),  m_r = max_c x[r][c],
 * with m_r and the denominator found in one pass over the row (the running
 * denominator rescaled whenever the running maximum grows) and y written in a
 * second. Entries equal to -inf get 0; a row with no finite entry is all 0.
 * Inputs holding NaN or +inf give unspecified results.
 *   x : input [rows, cols] float32, row-major, DEVICE pointer, read-only
 *   y : output [rows, cols] float32, DEVICE pointer; y == x (in place) is
 *       allowed, any other overlap is FA_ERR_ALIAS
 *   rows, cols : 0 .. 2^31 - 1 each, rows * cols < 2^40 (either 0: no-op
 *                returning FA_OK); otherwise FA_ERR_SHAPE. Matrices of more
 *                than 2^21 rows are processed as several launches of at most
 *                2^21 rows each, enqueued in row order on `stream`.
 * x and y must be 4-byte aligned; rows that are 16-byte aligned (cols a
 * multiple of 4, x and y 16-byte aligned) take the vectorised kernels.
 * Asynchronous on `stream` like every entry point.
 */
int fa_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, void* stream);

/*
 * fa_bwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, results and kernels as fa_bwd, without the workspace: the per-row
 * workspace lives in a fixed 16 MiB device array of the library (one copy per
 * GPU, kept until the process ends), so B * H * ceil(N / 128) * 128 must be at
 * most 2^21 rows, else FA_ERR_SCRATCH before anything is enqueued. The call
 * itself allocates nothing (its first call on a device looks the array's
 * address up once). Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (several streams or host threads) race and must be
 * serialised by the caller. The array needs no initialisation between calls.
 * The GPU is the one `stream` belongs to (the current device for NULL).
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, const fa_mask_t* mask, void* stream);

/* Static description of a status code; never NULL. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_FA_H */
