/*
 * fa.h - C ABI of an exact-attention (FlashAttention) forward and backward
 * library for AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the page "把 FlashAttention 搬上昇腾：Triton-Ascend
 * CV Pipeline 优化实战" (BiumBiu, 2026-08-30), cited as [FA-Ascend]:
 *
 *   forward  ([FA-Ascend] §一):  S = Q K^T * scale,  P = softmax(S),  O = P V
 *   backward ([FA-Ascend] §二):  Delta = rowsum(O * dO); P recomputed from the
 *            saved row statistic; dP = dO V^T; dS = scale * P * (dP - Delta);
 *            dQ = dS K; dK = dS^T Q; dV = P^T dO.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors Q, K, V, O, dO, dQ, dK, dV are dense, contiguous, row-major
 *   (Z, H, N, D) arrays: Z batch, H heads, N sequence length (queries and keys
 *   alike), D head dimension.  lse is contiguous (Z, H, N) float32 and the
 *   backward row statistics are contiguous (2, Z, H, N) float32.
 * - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *   never allocates, frees or retains device memory.  Pointers must be 16-byte
 *   aligned.  Outputs must not alias inputs.
 * - dtype is FA_DTYPE_F16 or FA_DTYPE_BF16 and applies to q, k, v, dout, dq,
 *   dk, dv.  o_dtype is either dtype or FA_DTYPE_F32 and applies to o.
 * - D must be 64, 128 or 256 ([FA-Ascend] §七 treats exactly these head dims).
 *   N may be any value >= 1 (a ragged last tile is masked); Z*H*N == 0 is a
 *   valid empty problem and returns FA_OK without launching anything (its
 *   pointers are not checked and may be NULL).  (N + 256) * D * 4 must stay
 *   below 2^31 (32-bit offsets within one head).
 * - causal (0 or 1) selects the causal mask: key j is visible to query i iff
 *   j <= i ([FA-Ascend] §八, lower triangle including the diagonal).
 * - scale must be finite and > 0 (normally 1/sqrt(D)).
 * - Every call enqueues its kernels on `stream` (0 = the default stream) and
 *   returns without synchronising.  The return value reports argument and
 *   launch errors only; a device fault shows at the caller's next
 *   synchronisation.  Setting the environment variable FA_DEBUG_SYNC=1 makes
 *   each call synchronise its stream and report errors it finds there.
 * - Argument checks happen before any HIP call: a call that returns
 *   FA_ERR_INVALID_ARGUMENT or FA_ERR_UNSUPPORTED has touched no GPU state.
 * - Return values are fa_status codes.  fa_last_error() gives a
 *   human-readable detail of the last failure on the calling thread.
 * - No C++ exception crosses this interface and the library writes nothing to
 *   stdout or stderr.  All entry points are thread-safe.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_dtype {
  FA_DTYPE_F16 = 0,
  FA_DTYPE_BF16 = 1,
  FA_DTYPE_F32 = 2
} fa_dtype;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad enum, negative size, small workspace */
  FA_ERR_UNSUPPORTED = 2,      /* valid arguments outside what the kernels implement (e.g. D=96) */
  FA_ERR_HIP = 3               /* a HIP runtime call or kernel launch failed */
} fa_status;

/* Library version: major*10000 + minor*100 + patch. */
int fa_version(void);

/* Static string naming a status code ("FA_OK", ...); never NULL. */
const char* fa_status_string(int status);

/* Detail of the last error on the calling thread ("" if none); valid until
 * the next call into the library on the same thread. */
const char* fa_last_error(void);

/*
 * Forward pass, [FA-Ascend] §一.
 *   q, k, v : (Z,H,N,D) dtype, read only.
 *   o       : (Z,H,N,D) o_dtype, written: O = softmax(Q K^T * scale) V.
 *   lse     : (Z,H,N) float32, written: natural-log log-sum-exp of each score
 *             row, lse_i = ln(sum_j exp(S_ij)), the row statistic the backward
 *             needs to recompute P ([FA-Ascend] §二 "recompute_softmax").
 * One kernel: the Q tile stays in registers, K/V tiles stream through LDS,
 * the softmax is the online (running max / running sum) form of §一, and
 * neither S nor P is ever written to memory.
 */
int fa_fwd(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype,
           const void* q, const void* k, const void* v, void* o, float* lse,
           float scale, int causal, hipStream_t stream);

/* Bytes of device workspace fa_bwd needs: 2*Z*H*N*sizeof(float) (the row
 * statistics written by fa_bwd_preprocess). */
size_t fa_bwd_workspace_bytes(int64_t Z, int64_t H, int64_t N, int64_t D);

/*
 * Backward pass, [FA-Ascend] §二.
 *   q, k, v, o, lse : as produced for/by fa_fwd with the same scale, causal,
 *                     dtype and o_dtype (lse must be passed unchanged).
 *   dout            : (Z,H,N,D) dtype, the incoming gradient dO.
 *   dq, dk, dv      : (Z,H,N,D) dtype, written (overwritten, not accumulated).
 *   workspace       : device buffer of at least fa_bwd_workspace_bytes();
 *                     holds the row statistics between the stages; contents
 *                     on return are those of fa_bwd_preprocess's `stats`.
 * Runs fa_bwd_dq_and_stats, then fa_bwd_dkdv on `stream`.  The result is
 * bitwise that of fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq run one by one.
 */
int fa_bwd(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype,
           const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           float scale, int causal, void* workspace, size_t workspace_bytes,
           hipStream_t stream);

/*
 * fa_bwd without the workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The row statistics live in a fixed array of the
 * library's own device memory (2 * FA_BWD_NOALLOC_MAX_ROWS float32 = 32 MiB on
 * every GPU the library runs on, held until the process ends), so the call
 * allocates and frees nothing.
 *   Limit: Z*H*N <= FA_BWD_NOALLOC_MAX_ROWS query rows; larger problems return
 *   FA_ERR_UNSUPPORTED before any work is enqueued.
 * Arguments, results (bitwise) and other errors are those of fa_bwd.  All
 * calls on one GPU share that GPU's array, which keeps the last call's
 * statistics: calls that overlap on one GPU (on other streams or from other
 * threads) race, and the caller must serialise them.
 */
#define FA_BWD_NOALLOC_MAX_ROWS ((int64_t)1 << 22)
int fa_bwd_noalloc(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype, int o_dtype,
                   const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   float scale, int causal, hipStream_t stream);

/*
 * Stage 1 of the backward: the per-row statistics of the gradient stages.
 *   o     : (Z,H,N,D) o_dtype;  dout : (Z,H,N,D) dtype;
 *   lse   : (Z,H,N) float32 from fa_fwd (read);
 *   stats : (2,Z,H,N) float32 (written): stats[0] = Delta, with
 *           Delta[z,h,i] = sum_d O[z,h,i,d] * dO[z,h,i,d] accumulated in
 *           float32 ([FA-Ascend] §二, first line), and stats[1] = lse * log2(e),
 *           the log-sum-exp in the exp2 units in which P is recomputed.
 */
int fa_bwd_preprocess(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype,
                      int o_dtype, const void* o, const void* dout,
                      const float* lse, float* stats, hipStream_t stream);

/*
 * Stage 2: dK and dV.  A persistent grid of `num_programs` workgroups (0 =
 * one per resident slot on the device: compute units x workgroups per CU)
 * walks a static schedule of (head, key-tile) units; each workgroup owns whole
 * key tiles, recomputes P from lse for every query tile, and writes each dK/dV
 * tile exactly once: no atomics and no N*N scratch ([FA-Ascend] §二 three
 * principles, §五 persistent programs).  stats comes from fa_bwd_preprocess.
 * The result does not depend on num_programs (bitwise).
 */
int fa_bwd_dkdv(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype,
                const void* q, const void* k, const void* v, const void* dout,
                const float* stats, void* dk, void* dv, float scale, int causal,
                int num_programs, hipStream_t stream);

/*
 * Stage 3: dQ.  One workgroup per (head, query tile) owns its dQ tile and
 * writes it exactly once ([FA-Ascend] §二: a query tile can finish dQ by
 * itself).  stats comes from fa_bwd_preprocess.
 */
int fa_bwd_dq(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype,
              const void* q, const void* k, const void* v, const void* dout,
              const float* stats, void* dq, float scale, int causal,
              hipStream_t stream);

/*
 * dQ, dK and dV in one pass: the persistent-program form of [FA-Ascend] §五.
 * A grid of `num_programs` workgroups (0 = one per resident slot on the
 * device) claims heads with a fixed stride; a program computes everything of
 * its heads, walking the key tiles in order with dK/dV of the key tile in
 * registers and adding each query tile's dQ contribution to an fp32 partial
 * of the head kept in `workspace`; the key tile holding a query tile's last
 * visible key writes its finished dQ rows instead.  Five matrix products per
 * (query tile, key tile), against seven for fa_bwd_dkdv + fa_bwd_dq.  Each
 * dQ, dK and dV element has one writer; no atomics; the scratch is O(N*D) per
 * head, never N*N ([FA-Ascend] §二).
 *   q, k, v, dout   : (Z,H,N,D) dtype (read);  stats : (2,Z,H,N) float32
 *                     from fa_bwd_preprocess (read);
 *   dq, dk, dv      : (Z,H,N,D) dtype (written once);
 *   workspace       : device buffer of at least
 *                     fa_bwd_fused_workspace_bytes(Z, H, N, D) bytes
 *                     (Z*H*ceil(N/32)*32*D float32: the heads' dQ partials;
 *                     contents on return are unspecified).
 * The result does not depend on num_programs (bitwise) and equals the
 * two-pass result to rounding (dQ's fp32 summation order differs).
 * Plain heads and dense batches only.  Errors as for fa_bwd_dkdv.
 */
size_t fa_bwd_fused_workspace_bytes(int64_t Z, int64_t H, int64_t N, int64_t D);
int fa_bwd_fused(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype,
                 const void* q, const void* k, const void* v, const void* dout,
                 const float* stats, void* dq, void* dk, void* dv, float scale,
                 int causal, int num_programs, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/*
 * dQ together with the row statistics ([FA-Ascend] §二): the dQ pass computes
 * Delta for its own query rows from o and dout (with the summation order of
 * fa_bwd_preprocess, so the values are bitwise the same) and lse * log2(e)
 * from lse, uses them, and writes both to `stats` ((2,Z,H,N) float32, the
 * layout fa_bwd_preprocess writes) for a following fa_bwd_dkdv.  This saves
 * the separate pass over O and dO.  Arguments as in fa_bwd.
 */
int fa_bwd_dq_and_stats(int64_t Z, int64_t H, int64_t N, int64_t D, int dtype,
                        int o_dtype, const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse,
                        float* stats, void* dq, float scale, int causal,
                        hipStream_t stream);

/*
 * Grouped key/value heads (GQA; MQA when Hkv = 1).  The page "从算子到
 * Serving：昇腾推理评测链路实践" (BiumBiu), section "GQA Paged Attention",
 * cited as [Serving-Ascend], lets H query heads share Hkv key/value heads, H a
 * whole multiple of Hkv: query head h attends with key/value head h / G,
 * G = H / Hkv.  The operation per query head is that of fa_fwd / fa_bwd; the
 * gradients of a shared key/value head are the sums over its G query heads.
 *   q, o, dout, dq : (Z,H,N,D);  k, v, dk, dv : (Z,Hkv,N,D);  lse : (Z,H,N).
 *   workspace      : fa_bwd_workspace_bytes(Z, H, N, D) (query heads).
 * Other arguments, the result and the errors are those of fa_fwd and fa_bwd;
 * in addition FA_ERR_INVALID_ARGUMENT if Hkv <= 0 (with H > 0) or H is not a
 * multiple of Hkv, and FA_ERR_UNSUPPORTED if G * (N + 256) * D * 2 reaches
 * 2^31 (one group is indexed with 32-bit offsets).  With Hkv = H these are
 * fa_fwd and fa_bwd, bitwise.  The G query heads of one key/value head run on
 * one XCD and share its K and V through that XCD's L2; dK / dV are written
 * once per key tile by the workgroup that walks all G query heads of it (no
 * atomics).
 */
int fa_fwd_gqa(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype,
               int o_dtype, const void* q, const void* k, const void* v, void* o,
               float* lse, float scale, int causal, hipStream_t stream);
int fa_bwd_gqa(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype,
               int o_dtype, const void* q, const void* k, const void* v,
               const void* o, const void* dout, const float* lse, void* dq,
               void* dk, void* dv, float scale, int causal, void* workspace,
               size_t workspace_bytes, hipStream_t stream);

/*
 * The two stages fa_bwd_gqa runs, for callers that schedule them (or time
 * them) one by one: fa_bwd_dq_and_stats and fa_bwd_dkdv with Hkv key/value
 * heads, arguments and shapes as above (stats: (2,Z,H,N) over query heads).
 * fa_bwd_dkdv_gqa's persistent workgroups own (key/value head, key tile)
 * units and walk the query tiles of all G query heads of their head.
 */
int fa_bwd_dq_and_stats_gqa(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D,
                            int dtype, int o_dtype, const void* q, const void* k,
                            const void* v, const void* o, const void* dout,
                            const float* lse, float* stats, void* dq, float scale,
                            int causal, hipStream_t stream);
int fa_bwd_dkdv_gqa(int64_t Z, int64_t H, int64_t Hkv, int64_t N, int64_t D, int dtype,
                    const void* q, const void* k, const void* v, const void* dout,
                    const float* stats, void* dk, void* dv, float scale, int causal,
                    int num_programs, hipStream_t stream);

/*
 * Variable-length batches.  [Serving-Ascend] (the page named above, sections
 * "GQA Paged Attention" and the integration discussion before it) has the
 * sequences of one batch differ in length (context_lens), with tokens past a
 * sequence's end taking no part.  Here the B sequences are packed one after
 * another along the token axis, head-major:
 *   q, o, dout, dq : (H, T, D);  k, v, dk, dv : (Hkv, T, D);  lse : (H, T);
 *   cu_seqlens     : DEVICE int32[B+1], token offsets: sequence b is tokens
 *                    cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head
 *                    (0 = cu_seqlens[0] <= ... <= cu_seqlens[B] = T; empty
 *                    sequences allowed); read by the kernels, never written;
 *   max_seqlen     : at least the longest sequence: it sizes the grids.
 *                    With a smaller value some tiles of a longer sequence
 *                    get no workgroup (not only its last ones: with the
 *                    causal mask query tiles are dealt in pairs from both
 *                    ends, so interior tiles are the ones left out); their
 *                    outputs are left unwritten and the results of such a
 *                    call are unspecified;
 *   workspace      : fa_bwd_workspace_bytes(1, H, T, D) bytes (stats are
 *                    (2, H, T) for the stage forms).
 * Each sequence is its own attention problem (causal within itself when
 * causal = 1) with the grouping of fa_fwd_gqa (Hkv = H for plain heads).
 * Offsets outside [0, T] or decreasing are clamped into range by the kernels,
 * so no offsets array makes them access memory outside the tensors; the
 * results for such an array are unspecified.  Errors as for fa_fwd_gqa /
 * fa_bwd_gqa, plus FA_ERR_INVALID_ARGUMENT for a NULL or misaligned
 * cu_seqlens or T < 0, and FA_ERR_UNSUPPORTED when G * (T + 256) * D * 2 or
 * (T + 256) * D * 4 reaches 2^31.  B*H*T == 0 is an empty problem.
 * The dK/dV stage of a packed batch runs one workgroup per (sequence
 * key/value head, key tile), first key tiles first, instead of the
 * persistent schedule (whose static dealing does not know the lengths):
 * fa_bwd_dkdv_varlen ignores num_programs.
 */
int fa_fwd_varlen(int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t max_seqlen,
                  int64_t D, int dtype, int o_dtype, const int32_t* cu_seqlens,
                  const void* q, const void* k, const void* v, void* o, float* lse,
                  float scale, int causal, hipStream_t stream);
int fa_bwd_varlen(int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t max_seqlen,
                  int64_t D, int dtype, int o_dtype, const int32_t* cu_seqlens,
                  const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  float scale, int causal, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);
int fa_bwd_dq_and_stats_varlen(int64_t B, int64_t H, int64_t Hkv, int64_t T,
                               int64_t max_seqlen, int64_t D, int dtype, int o_dtype,
                               const int32_t* cu_seqlens, const void* q, const void* k,
                               const void* v, const void* o, const void* dout,
                               const float* lse, float* stats, void* dq, float scale,
                               int causal, hipStream_t stream);
int fa_bwd_dkdv_varlen(int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t max_seqlen,
                       int64_t D, int dtype, const int32_t* cu_seqlens, const void* q,
                       const void* k, const void* v, const void* dout,
                       const float* stats, void* dk, void* dv, float scale, int causal,
                       int num_programs, hipStream_t stream);

/*
 * Paged KV cache ([Serving-Ascend], sections "ReshapeAndCache" and "GQA Paged
 * Attention").  One page is one physical block of one key/value head:
 *   k_cache : (num_blocks, Hkv, D/8, block_size, 8) dtype, the page's keys in
 *             16-byte chunks of 8 channels, chunk-major: channel d of the
 *             token at offset o is element [block][head][d/8][o][d%8];
 *   v_cache : (num_blocks, Hkv, D, block_size) dtype, the page's values
 *             transposed (one row of block_size values per channel d).
 * block_size is a multiple of 16 in [16, 1024].
 *
 * fa_reshape_and_cache: writes new tokens into the cache.
 *   key, value   : (num_tokens, Hkv, D) dtype, read;
 *   slot_mapping : DEVICE int64[num_tokens]; token i goes to block
 *                  slot / block_size at offset slot % block_size; a negative
 *                  slot skips the token (as on the page), and so does a slot
 *                  past the cache (slot >= num_blocks * block_size).  Slots of
 *                  one call must be distinct (two tokens on one slot leave
 *                  either one there).
 *   k_cache, v_cache : written at the tokens' slots only.
 *
 * fa_paged_decode: attention of one query token per sequence over its cached
 * context.
 *   q            : (B, H, D) dtype; query head h uses key/value head
 *                  h / (H / Hkv);
 *   block_tables : DEVICE int32 (B, max_blocks_per_seq): token t of sequence
 *                  b is in physical block block_tables[b][t / block_size] at
 *                  offset t % block_size;
 *   context_lens : DEVICE int32[B], tokens of each context (clamped to
 *                  [0, max_blocks_per_seq * block_size]); every token of the
 *                  context is visible; the rest of the last block is masked;
 *   max_context_len : host bound on the context lengths, used only to size
 *                  the split of long contexts (and the workspace); longer
 *                  contexts are still processed whole;
 *   o            : (B, H, D) o_dtype (dtype or FA_DTYPE_F32), written;
 *   lse          : (B, H) float32 natural-log log-sum-exp of each score row,
 *                  written, or NULL;
 *   workspace    : fa_paged_decode_workspace_bytes(B, H, Hkv, D,
 *                  max_context_len) bytes of device memory (0 bytes: NULL is
 *                  fine), 16-byte aligned.
 * A block-table entry outside [0, num_blocks) makes the tokens of that block
 * take no part (they are not read).  A context of 0 tokens gives O = 0 and
 * lse = -inf.  Long contexts are split over several workgroups per (sequence,
 * key/value head) whose partial (O, lse) pairs a second kernel combines.
 */
int fa_reshape_and_cache(int64_t num_tokens, int64_t Hkv, int64_t D, int64_t block_size,
                         int64_t num_blocks, int dtype, const void* key, const void* value,
                         const int64_t* slot_mapping, void* k_cache, void* v_cache,
                         hipStream_t stream);
size_t fa_paged_decode_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t D,
                                       int64_t max_context_len);
int fa_paged_decode(int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t block_size,
                    int64_t num_blocks, int64_t max_blocks_per_seq, int64_t max_context_len,
                    int dtype, int o_dtype, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_tables,
                    const int32_t* context_lens, void* o, float* lse, float scale,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Query-aware page selection and attention over the kept pages
 * ([Serving-Ascend], section "Quest Sparse Attention": score the pages of a
 * long context cheaply, keep the Top-K, run exact attention over their
 * tokens only).  The scoring rule is the published Quest one: a page keeps
 * the channel-wise minimum and maximum of its valid keys, and its score for a
 * query q is sum_d max(q_d * min_d, q_d * max_d), an upper bound of q . k
 * over the page.  A key/value head keeps one set of pages for its G query
 * heads, scored by the sum of their scores; ties go to the lower
 * page; kept pages are listed in ascending order.  Caches, block tables and
 * context lengths as for fa_paged_decode; contexts of at most 4096 pages
 * (max_blocks_per_seq <= 4096).
 *
 * fa_quest_page_minmax: kmeta (num_blocks, Hkv, 2, D) dtype, written for the
 *   physical blocks of every context: [.., 0, :] = minimum, [.., 1, :] =
 *   maximum over the page's tokens inside the context (exact).  A physical
 *   block shared by two contexts gets the metadata of either.
 * fa_quest_select: selected (B, Hkv, topk) int32, n_selected (B, Hkv) int32,
 *   written: the kept logical pages of each (sequence, key/value head), min(topk,
 *   pages of the context) of them, ascending; entries past n_selected are
 *   left unwritten (with topk == 0, selected may be NULL; so in
 *   fa_paged_decode_sparse, whose outputs are then O = 0 and lse = -inf).
 * fa_paged_decode_sparse: fa_paged_decode over the tokens of the kept pages
 *   (selected / n_selected as written by fa_quest_select, or any ascending
 *   lists of logical pages); the last page of a context is cut at the
 *   context's end.  workspace: fa_paged_decode_workspace_bytes(B, H, Hkv, D,
 *   topk * block_size) bytes.  Pages outside the context, and counts outside
 *   [0, topk], are clamped or skipped, never read out of bounds.
 */
int fa_quest_page_minmax(int64_t B, int64_t Hkv, int64_t D, int64_t block_size,
                         int64_t num_blocks, int64_t max_blocks_per_seq, int dtype,
                         const void* k_cache, const int32_t* block_tables,
                         const int32_t* context_lens, void* kmeta, hipStream_t stream);
int fa_quest_select(int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t block_size,
                    int64_t num_blocks, int64_t max_blocks_per_seq, int64_t topk, int dtype,
                    const void* q, const void* kmeta, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t* selected, int32_t* n_selected,
                    hipStream_t stream);
int fa_paged_decode_sparse(int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t block_size,
                           int64_t num_blocks, int64_t max_blocks_per_seq, int64_t topk,
                           int dtype, int o_dtype, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, const int32_t* selected,
                           const int32_t* n_selected, void* o, float* lse, float scale,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode attention over one or two KV sources normalised together (the page
 * "在 4 张 A100 上部署 DeepSeek-V4-Flash-0731" (BiumBiu), section 7.5: one
 * sparse attention kernel serves a single source (the sliding-window pool)
 * or two sources (sliding-window and compressed pools, section 7.3) whose
 * pages form one logical set under a single softmax denominator).
 *
 * A source is a paged cache in the layouts above with its own block table,
 * context lengths and block size; it contributes every token of each
 * context (n_selected == NULL) or the tokens of its kept logical pages
 * (n_selected != NULL: as for fa_paged_decode_sparse, the last page of a
 * context cut at the context's end).  For query head h of sequence b the
 * attended set is the concatenation of the sources' tokens for key/value
 * head h / (H / Hkv): O = softmax(scale q K^T) V and lse = ln sum exp over
 * that set.  Every source has the same Hkv, D and dtype; q, o, lse as for
 * fa_paged_decode.  The struct is read on the host during the call only.
 *   max_context_len : dense source: host bound on its context lengths (sizes
 *                     its split only, as for fa_paged_decode); ignored for a
 *                     sparse source (topk * block_size is used);
 *   selected        : (B, Hkv, topk) int32 ascending kept pages, or NULL
 *                     (only with topk == 0) for a sparse source; must be
 *                     NULL for a dense one.
 * n_sources is 1 or 2.  workspace: fa_paged_decode_sources_workspace_bytes
 * of the same arguments (0 bytes: NULL is fine), 16-byte aligned.  A query
 * head with no token in any source gets O = 0 and lse = -inf.  Every split of
 * every source writes a partial (O, lse) pair and one combine merges them, so
 * the sources share one maximum and one denominator.
 */
typedef struct fa_kv_source {
  const void* k_cache;          /* (num_blocks, Hkv, D/8, block_size, 8) dtype */
  const void* v_cache;          /* (num_blocks, Hkv, D, block_size) dtype */
  const int32_t* block_tables;  /* DEVICE (B, max_blocks_per_seq) */
  const int32_t* context_lens;  /* DEVICE (B) */
  int64_t block_size;           /* multiple of 16 in [16, 1024] */
  int64_t num_blocks;
  int64_t max_blocks_per_seq;
  int64_t max_context_len;
  const int32_t* selected;      /* DEVICE (B, Hkv, topk) or NULL */
  const int32_t* n_selected;    /* DEVICE (B, Hkv), or NULL for a dense source */
  int64_t topk;
  const int32_t* row_lens;      /* DEVICE (B, Tq): tokens each query row sees, or NULL (all) */
} fa_kv_source;
size_t fa_paged_decode_sources_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t D,
                                               int n_sources, const fa_kv_source* sources);
int fa_paged_decode_sources(int64_t B, int64_t H, int64_t Hkv, int64_t D, int dtype,
                            int o_dtype, const void* q, int n_sources,
                            const fa_kv_source* sources, void* o, float* lse, float scale,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Several query tokens per sequence over the same sources (section 7.5 of the
 * page above: prefill and decode share the kernel because the causal
 * constraint is expanded into per-row lengths).  q is (B, Tq, H, D); o is
 * (B, Tq, H, D) o_dtype and lse (B, Tq, H) float32 or NULL.  A source's
 * row_lens (DEVICE int32 (B, Tq), or NULL) gives how many of its tokens --
 * the first ones of its context, or of its kept pages' tokens in page order --
 * query token t of sequence b sees (clamped to [0, what the source holds]);
 * NULL: all of them.  For a chunk of the last Tq tokens of a context of n
 * cached tokens, row_lens[b][t] = n - Tq + t + 1 is causal attention.  A
 * query row that sees no token gets O = 0 and lse = -inf.  Tq = 1 is
 * fa_paged_decode_sources.  workspace: fa_paged_attention_sources_workspace_bytes
 * of the same arguments.
 */
size_t fa_paged_attention_sources_workspace_bytes(int64_t B, int64_t Tq, int64_t H, int64_t Hkv,
                                                  int64_t D, int n_sources,
                                                  const fa_kv_source* sources);
int fa_paged_attention_sources(int64_t B, int64_t Tq, int64_t H, int64_t Hkv, int64_t D,
                               int dtype, int o_dtype, const void* q, int n_sources,
                               const fa_kv_source* sources, void* o, float* lse, float scale,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Device facts used for launch sizing, for the current device: compute
 * units, and the persistent grid fa_bwd_dkdv uses for (D, dtype) when
 * num_programs is 0.  Either output pointer may be NULL.
 */
int fa_device_info(int64_t D, int dtype, int* compute_units, int* dkdv_programs);

/*
 * Host-only planning helpers (no HIP call, no device needed).
 *
 * fa_dkdv_schedule: replays the static schedule of fa_bwd_dkdv with
 * `num_programs` programs.  units_per_program[p] receives the number of
 * (head, key tile) units program p owns and qtiles_per_program[p] the number
 * of query tiles it visits; both arrays hold num_programs entries (either may
 * be NULL).  *n_units receives the total unit count.  [FA-Ascend] §五 deals
 * heads to a fixed number of programs with a fixed stride; without the causal
 * mask and with one key tile per head this reproduces that dealing.
 *
 * fa_fwd_tile_pairs: number of (query tile, key tile) pairs fa_fwd visits for
 * a sequence of N at head dim D, and the total number of pairs, so that the
 * work saved by the shortened causal loop ([FA-Ascend] §八) can be checked.
 */
int fa_dkdv_schedule(int64_t Z, int64_t H, int64_t N, int64_t D, int causal, int num_programs,
                     int64_t* units_per_program, int64_t* qtiles_per_program, int64_t* n_units);
int fa_fwd_tile_pairs(int64_t N, int64_t D, int causal, int64_t* visited, int64_t* total);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
