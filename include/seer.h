/*
 * seer.h -- C-ABI of the MI355X (gfx950) block-sparse attention prefill library.
 *
 * The calls follow the statement of the problem in the SeerAttention pages:
 * soft block scores are turned into per-query-block KV-block lists by
 * threshold or TopK (model card "SeerAttention-Llama-3.1-8B-AttnGates", method
 * summary), a block-sparse flash-attention kernel then visits only the listed
 * KV blocks (rebuttal "SeerAttention: Learning Intrinsic Sparse Attention in
 * Your LLMs", "Weakness 5 (Pseudo code of Inference Kernel)"), and a dense
 * flash-attention pass emits the 2D max-pooled attention map used as the gate's
 * training target (reproducibility summary of "SeerAttention: Self-distilled
 * Attention Gating for Efficient Long-context Prefilling", Pseudocode row,
 * Figure 8).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Block size is 64 tokens (same summary, Experiment Setup row).
 * - Tensors are dense, contiguous, row-major:
 *     Q, O  : bf16 [B, Hq,  T, D]      K, V : bf16 [B, Hkv, T, D]
 *   following the [Batch, Head, Seq, Dim] layout the rebuttal uses
 *   ("Weakness 3 (The meaning of "max and min pooling on K matrix" is not clear)").
 *   Q, K, V and O must be 16-byte aligned.
 * - nQB = ceil(T / 64).  T need not be a multiple of 64: the last block is
 *   short, as if padded (rebuttal, "Weakness 4 (Rounding Issue when Seq not
 *   evenly divided by B)").
 * - Attention is causal with Tq = Tk = T: query position r sees key c iff c <= r.
 * - GQA: query head h reads KV head h / (Hq / Hkv).
 * - Every pointer argument named "device" is device memory owned by the caller.
 *   The library never allocates or frees memory and may be called from several
 *   host threads at once.  It keeps no buffer and no global mutable state,
 *   with one exception: seer_sparse_prefill_noalloc's static scratch array and
 *   the per-device address of it that the library caches (calls of that entry
 *   point that overlap on one GPU race on the array).
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Every call only enqueues work on it and returns without synchronising.
 * - Errors: argument errors are detected on the host before anything is
 *   enqueued and return a non-zero seer_status_t; nothing is written then.
 *   A failed kernel launch returns SEER_ERR_HIP.  No C++ exception crosses
 *   this interface.
 */
#ifndef SEER_H_
#define SEER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SEER_BLOCK 64
/* Longest row seer_build_mask accepts: 4096 blocks = 262144 tokens. */
#define SEER_MAX_QUERY_BLOCKS 4096

typedef enum {
  SEER_OK = 0,
  SEER_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned tensor, bad scalar */
  SEER_ERR_UNSUPPORTED = 2, /* head dim other than 64 or 128, sizes beyond int range */
  SEER_ERR_CAPACITY = 3,    /* max_k too small for the TopK budget or the forced blocks */
  SEER_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the *_workspace_size() */
  SEER_ERR_HIP = 5          /* the HIP runtime refused a launch */
} seer_status_t;

typedef enum { SEER_MASK_THRESHOLD = 0, SEER_MASK_TOPK = 1 } seer_mask_mode_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* seer_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int seer_version(void);

/*
 * Number of KV blocks the TopK rule keeps for the last (largest) query block,
 * i.e. the smallest max_k seer_build_mask accepts in TopK mode:
 *   k_i = min(i + 1, max(|F_i|, ceil(density * (i + 1)))) at i = nQB - 1,
 * with the product and ceiling in IEEE double and F_i the forced blocks
 * (diagonal, plus block 0 when keep_sink).  TopK is per row (rebuttal,
 * "Weakness 2 (Memory complexity)") and its size is a user knob ("Weakness 1
 * (How to choose sparsity?)").  Host only.  Returns -1 for nQB < 0 or a
 * density outside (0, 1].
 */
int seer_topk_budget(int nQB, double density, int keep_sink);

/*
 * Block-mask construction: soft block scores -> compact per-row KV-block lists.
 *
 * scores  device fp32 [B, H, nQB, nKB]; row (b,h,i) reads only entries j <= i.
 *         nKB >= nQB is the row stride.
 * mode    SEER_MASK_TOPK: row i keeps its forced blocks plus the best-ranked
 *         other causal blocks, k_i in total (see seer_topk_budget); `density`
 *         must lie in (0, 1], `threshold` is ignored.
 *         SEER_MASK_THRESHOLD: row i keeps its forced blocks plus every other
 *         causal block whose fp32 score is >= (float)threshold (NaN never
 *         passes); `threshold` must be finite, `density` is ignored.  When the
 *         list would exceed max_k it keeps the forced blocks plus the
 *         best-ranked passing blocks.
 *         Forced blocks: the diagonal i, plus block 0 if keep_sink != 0.
 *         Ranking: score descending, ties to the lower block index, NaN lowest.
 * kv_idx  device int32 out [B, H, nQB, max_k]: row (b,h,i) holds its selected
 *         blocks in strictly ascending order, then -1 up to max_k.
 * kv_cnt  device int32 out [B, H, nQB]: list lengths (always <= max_k).
 * nQB     <= SEER_MAX_QUERY_BLOCKS, else SEER_ERR_UNSUPPORTED.
 * max_k   TopK: >= seer_topk_budget(nQB, density, keep_sink);
 *         threshold: >= 2 if keep_sink and nQB > 1, else >= 1.
 *         Otherwise SEER_ERR_CAPACITY.
 * The result is fully determined by the inputs (bit-reproducible).
 */
int seer_build_mask(const float* scores, int B, int H, int nQB, int nKB, int mode,
                    float threshold, double density, int keep_sink, int32_t* kv_idx,
                    int32_t* kv_cnt, int max_k, void* stream);

/*
 * seer_build_mask that also reports, for every row, how many blocks the rule
 * selects before any cut to max_k (the capacity signal of threshold mode).
 *
 * kv_need device int32 out [B, H, nQB], non-null:
 *         TopK mode: the row's k_i (equal to kv_cnt, since max_k is at least
 *         seer_topk_budget);
 *         threshold mode: the forced blocks plus every other causal block with
 *         score >= (float)threshold.  kv_need > max_k means the row was cut to
 *         its forced blocks plus the max_k - |forced| best-ranked passing
 *         blocks (kv_cnt = max_k): the list differs from what the threshold
 *         selects, and seer_validate_lists reports it as SEER_LIST_CAPACITY.
 * Lists, counts, arguments and errors are exactly those of seer_build_mask
 * (model card "SeerAttention-Llama-3.1-8B-AttnGates", method summary:
 * threshold or TopK on the soft block scores; the budget is a user knob,
 * rebuttal "Weakness 1 (How to choose sparsity?)").
 */
int seer_build_mask_need(const float* scores, int B, int H, int nQB, int nKB, int mode,
                         float threshold, double density, int keep_sink, int32_t* kv_idx,
                         int32_t* kv_cnt, int32_t* kv_need, int max_k, void* stream);

/* Flag bits written by seer_validate_lists (OR-ed per row and over all rows). */
#define SEER_LIST_BAD_COUNT 1 /* kv_cnt < 0 or > max_k (the calls read it clamped to [0, max_k]) */
#define SEER_LIST_BAD_ENTRY 2 /* a counted entry outside [0, r] (the calls skip it) */
#define SEER_LIST_REPEAT 4    /* a block counted twice in one row (it would be accumulated twice) */
#define SEER_LIST_UNSORTED 8  /* counted entries not strictly ascending (allowed; never written
                                 by seer_build_mask) */
#define SEER_LIST_CAPACITY 16 /* kv_need > max_k: a threshold row was cut to max_k */

/*
 * Checks block lists in the [Seq/Block, TopK] layout of the rebuttal
 * "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs", "Weakness 2
 * (Memory complexity)" against what the sparse prefill requires: row r (of nB
 * rows per head) may list blocks 0..r, each at most once, among its first
 * min(max(kv_cnt, 0), max_k) entries.
 *
 * kv_idx    device int32 [B, H, nB, max_k]; kv_cnt device int32 [B, H, nB].
 * kv_need   device int32 [B, H, nB] as written by seer_build_mask_need, or NULL
 *           (then SEER_LIST_CAPACITY is never set).
 * row_flags device int32 out [B, H, nB] (the row's flag bits), or NULL.
 * flags     device int32 out, one element: the OR of every row's flags (the
 *           call clears it first, on the stream).
 * Repeats are found in any order for rows r < 8192; in longer rows only when
 * the repeated entries are adjacent.  Asynchronous on `stream`: read `flags`
 * after the stream has completed (seer_list_flags_status turns them into a
 * status).  Errors: SEER_ERR_INVALID_ARG for negative sizes, max_k < 1 or a
 * NULL kv_idx / kv_cnt / flags; SEER_ERR_UNSUPPORTED if B*H*nB exceeds int range.
 */
int seer_validate_lists(const int32_t* kv_idx, const int32_t* kv_cnt, const int32_t* kv_need,
                        int B, int H, int nB, int max_k, int32_t* row_flags, int32_t* flags,
                        void* stream);

/* Host only: the status a set of list flags amounts to -- SEER_ERR_CAPACITY if
 * a row was cut (SEER_LIST_CAPACITY), else SEER_ERR_INVALID_ARG if a block is
 * repeated (SEER_LIST_REPEAT, the one violation that changes results), else
 * SEER_OK (counts and entries outside the rules are clamped and skipped by the
 * calls, and any order is accepted). */
int seer_list_flags_status(int flags);

/* Bytes of device workspace seer_sparse_prefill needs (work list of the
 * load-balancing schedule).  Returns 0 for invalid sizes. */
size_t seer_sparse_prefill_workspace_size(int B, int Hq, int Hkv, int T);

/*
 * Block-sparse causal flash-attention prefill (rebuttal, "Weakness 5 (Pseudo
 * code of Inference Kernel)"): query block i of head h attends only to the KV
 * blocks listed in kv_idx[b,h,i,0:min(kv_cnt,max_k)]; K and V of a step come
 * from the same block.  Equivalent to logits sm_scale*<q_r,k_c> set to -inf on
 * every unlisted block, then softmax and P.V.
 *
 * q, k, v  device bf16, layouts above; D in {64, 128}; Hq % Hkv == 0.
 * sm_scale finite and > 0 (pass 1/sqrt(D) for the usual scaling).
 * kv_idx   device int32 [B, Hq, nQB, max_k], kv_cnt device int32 [B, Hq, nQB]
 *          (as written by seer_build_mask).  Entries outside [0, i] are
 *          skipped, list order does not matter, a list must not repeat a block.
 *          A row with no valid entry produces O = 0.
 * o        device bf16 out [B, Hq, T, D], rounded to nearest even.
 * workspace device, >= seer_sparse_prefill_workspace_size(B, Hq, Hkv, T) bytes,
 *          256-byte aligned; overwritten.
 */
int seer_sparse_prefill(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                        int T, int D, float sm_scale, const int32_t* kv_idx,
                        const int32_t* kv_cnt, int max_k, void* o, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * seer_sparse_prefill with lists of `block`-token blocks, block in {64, 128}
 * (else SEER_ERR_UNSUPPORTED); the rebuttal's "Question 3 (Block Size
 * Experiments)" evaluates block sizes 32, 64 and 128.  kv_idx is
 * [B, Hq, nB, max_k] and kv_cnt [B, Hq, nB] with nB = ceil(T / block), both
 * counting blocks of `block` tokens (e.g. seer_build_mask run on
 * [B, Hq, nB, nB] block scores); query block i of `block` rows attends to the
 * keys of its listed blocks, causally.  Everything else, the workspace
 * included, is as for seer_sparse_prefill, which is this call with block 64.
 */
int seer_sparse_prefill_block(const void* q, const void* k, const void* v, int B, int Hq,
                              int Hkv, int T, int D, float sm_scale, int block,
                              const int32_t* kv_idx, const int32_t* kv_cnt, int max_k, void* o,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace seer_pooled_attn_map needs: the stored per-row
 * block maxima r_ij (fp32, 64 per causal (i, j) tile).  0 for invalid sizes. */
/*
 * seer_sparse_prefill for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments minus the workspace, and the same kernels and results.  The
 * schedule's work list lives in a static device array of the library instead,
 * sized for B * Hq * nQB <= 262144 items (4 MiB; one copy per GPU, held until
 * the process ends); larger problems return SEER_ERR_WORKSPACE before any
 * launch.  Its device address is looked up on the first call made with a
 * device current (the device of `stream`), so make that device current.  The
 * call allocates nothing.  Calls that overlap on one GPU (other streams, other
 * host threads) share the array and race: serialise them.
 */
int seer_sparse_prefill_noalloc(const void* q, const void* k, const void* v, int B, int Hq,
                                int Hkv, int T, int D, float sm_scale, const int32_t* kv_idx,
                                const int32_t* kv_cnt, int max_k, void* o, void* stream);

size_t seer_pooled_attn_map_workspace_size(int B, int Hq, int T);

/*
 * Dense causal flash attention that also emits the 2D max-pooled attention
 * map (reproducibility summary, Pseudocode row, Figure 8): a first pass stores
 * the row maxima r_ij of every tile while it accumulates O, m_i and l_i; a
 * second pass rescales them as exp(r_ij - m_i) / l_i and takes the max over
 * the tile's rows.
 *
 * q, k, v, D, sm_scale as for seer_sparse_prefill.
 * o     device bf16 out [B, Hq, T, D].
 * amap  device fp32 out [B, Hq, nQB, nQB]: amap[b,h,i,j] = largest softmax
 *       probability inside the (i, j) tile for j <= i, 0 for j > i.  Not
 *       row-normalised.
 * workspace device, >= seer_pooled_attn_map_workspace_size(B, Hq, T) bytes,
 *       256-byte aligned; overwritten.
 */
int seer_pooled_attn_map(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                         int T, int D, float sm_scale, void* o, float* amap, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Bytes of device workspace seer_attn_gate_scores needs: the pooled Q and K
 * (fp32 [B,Hq,nQB,D] and [B,Hkv,nQB,2D], sized for D = 128), the projected,
 * rotated Q~ [B,Hq,nQB,Dg] and K~ [B,Hkv,nQB,Dg] (fp32), and each row's
 * (max, sum of exponentials) per 64-block tile of keys (fp32 pairs).  0 for
 * invalid sizes. */
size_t seer_attn_gate_workspace_size(int B, int Hq, int Hkv, int T, int Dg);

/*
 * AttnGate soft block scores, the input of seer_build_mask.  The gate pools
 * along the sequence per 64-token block -- Q by average, K by max and by min,
 * the two K poolings concatenated along the hidden dimension -- before its
 * linear layers (rebuttal "SeerAttention: Learning Intrinsic Sparse Attention
 * in Your LLMs", Weakness 3 and "Question 1 (Theoretical or Intuitive
 * Explanation for Pooling Selection)"), pools the Q and K from before the
 * model's RoPE and applies its own block RoPE ("Q1 More about in AttnGate's
 * RoPE"), and outputs a softmax per row ("Question 2: (Row-Normalization of
 * Max-Pooled Attention Map)").  With Qp_i = mean of Q's rows in block i and
 * Kp_j = [max | min] of K's rows in block j:
 *   Q~_i = rope(Qp_i Wq[h], i),  K~_j = rope(Kp_j Wk[g], j),  g = h / (Hq / Hkv)
 *   scores[b,h,i,j] = softmax over j' <= i of scale <Q~_i, K~_j'>   (j <= i), 0 (j > i)
 * rope is the rotate-half rotary embedding over Dg dims, frequencies
 * rope_base^(-2t/Dg), at the block index.  A short last block pools the rows
 * it has (torch pooling with ceil_mode, "Weakness 4 (Rounding Issue ...)").
 *
 * q, k     device bf16 [B,Hq,T,D] and [B,Hkv,T,D] (before the model's RoPE),
 *          16-byte aligned; D in {64, 128}; Hq % Hkv == 0.
 * wq, wk   device fp32 [Hq, D, Dg] and [Hkv, 2D, Dg] (row-major, no bias),
 *          16-byte aligned.
 * Dg       32, 64 or 128.
 * scale    finite and > 0 (1/sqrt(Dg) is the usual choice); rope_base finite
 *          and > 1 (10000 is the usual choice).
 * scores   device fp32 out [B, Hq, nQB, nQB].
 * workspace device, >= seer_attn_gate_workspace_size(B, Hq, Hkv, T, Dg) bytes,
 *          256-byte aligned; overwritten.
 * Arithmetic is fp32 (the linear layers and Q~K~^T on the fp32 matrix cores;
 * RoPE angles formed and reduced mod 2 pi in fp64, then fp32 sin/cos); results
 * are bit-reproducible.
 */
int seer_attn_gate_scores(const void* q, const void* k, int B, int Hq, int Hkv, int T, int D,
                          const float* wq, const float* wk, int Dg, float scale, float rope_base,
                          float* scores, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace seer_attn_gate_mask needs: that of
 * seer_attn_gate_scores, plus B * Hq * nQB * nQB fp32 for the logits when no
 * scores buffer is given (with_scores == 0).  0 for invalid sizes. */
size_t seer_attn_gate_mask_workspace_size(int B, int Hq, int Hkv, int T, int Dg,
                                          int with_scores);

/* Bytes of device workspace for seer_attn_gate_mask without a scores buffer
 * when the logits are produced and selected in passes of pass_tiles tile rows
 * (64 query blocks each) instead of all at once: that of seer_attn_gate_scores
 * plus B * Hq * min(nQB, 64 pass_tiles) * nQB fp32, so the logits take memory
 * linear in T for a fixed pass.  This is the tiling the rebuttal "SeerAttention:
 * Learning Intrinsic Sparse Attention in Your LLMs" suggests for the gate when
 * its quadratic output is too large ("Weakness 2 (Memory complexity)"): the
 * gate is computed tile by tile like FlashAttention and each row is selected
 * as soon as its tiles are done (a whole row fits on chip, so no local TopK
 * and merge are needed).  0 for invalid sizes or pass_tiles < 1. */
size_t seer_attn_gate_mask_pass_workspace_size(int B, int Hq, int Hkv, int T, int Dg,
                                               int pass_tiles);

/*
 * AttnGate scores and the block mask in one call: the gate's scores, as
 * seer_attn_gate_scores defines them, go straight into the per-row threshold
 * or TopK of seer_build_mask (the gate's soft scores are what the mask is
 * built from: model card "SeerAttention-Llama-3.1-8B-AttnGates", method
 * summary).  The lists are those seer_build_mask(scores, B, Hq, nQB, nQB,
 * mode, threshold, density, keep_sink, ...) returns for the scores
 * seer_attn_gate_scores returns, bit for bit; the last kernel normalises each
 * score row in registers and selects from it there, so the score map is
 * neither written twice nor read back (and not written at all when scores is
 * NULL).
 *
 * q, k, wq, wk, Dg, scale, rope_base: as seer_attn_gate_scores.
 * mode, threshold, density, keep_sink, kv_idx, kv_cnt, max_k: as
 *          seer_build_mask with nQB = nKB = ceil(T / 64); nQB <=
 *          SEER_MAX_QUERY_BLOCKS (else SEER_ERR_UNSUPPORTED); the same
 *          capacity rules (SEER_ERR_CAPACITY).
 * scores   device fp32 out [B, Hq, nQB, nQB] (the scores, as
 *          seer_attn_gate_scores writes them), or NULL.
 * workspace device, 256-byte aligned, overwritten.  With scores: >=
 *          seer_attn_gate_mask_workspace_size(B, Hq, Hkv, T, Dg, 1) bytes.
 *          Without: >= seer_attn_gate_mask_pass_workspace_size(B, Hq, Hkv, T,
 *          Dg, 1) bytes; the call then runs as many tile rows per pass as the
 *          workspace holds (one pass from
 *          seer_attn_gate_mask_workspace_size(..., 0) bytes on).  The lists do
 *          not depend on the number of passes.  Too small: SEER_ERR_WORKSPACE.
 */
int seer_attn_gate_mask(const void* q, const void* k, int B, int Hq, int Hkv, int T, int D,
                        const float* wq, const float* wk, int Dg, float scale, float rope_base,
                        int mode, float threshold, double density, int keep_sink,
                        int32_t* kv_idx, int32_t* kv_cnt, int max_k, float* scores,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Row-normalised distillation target and its MSE against gate scores.  The
 * max-pooled map is normalised per row so that, like the gate's softmax
 * output, each row sums to 1 (rebuttal "SeerAttention: Learning Intrinsic
 * Sparse Attention in Your LLMs", "Question 2: (Row-Normalization of
 * Max-Pooled Attention Map)"); the gate learns it with an MSE loss (same
 * rebuttal, "Question 2 (Currently use MSE loss, how about e2e LM loss?)").
 *
 * amap    device fp32 [B, H, nQB, nQB], e.g. from seer_pooled_attn_map; only
 *         entries j <= i are read.
 * gate    device fp32 [B, H, nQB, nQB] gate scores, or NULL (target only);
 *         only entries j <= i are read.
 * target  device fp32 out [B, H, nQB, nQB]: amap[b,h,i,j] / sum_{j'<=i}
 *         amap[b,h,i,j'] for j <= i (0 if that sum is 0), 0 for j > i.  May be
 *         the same buffer as amap (normalised in place).
 * row_sse device fp32 out [B, H, nQB] or NULL: sum over j <= i of
 *         (gate - target)^2.  Written only when gate is given.
 * loss    device fp32 out [1] or NULL: the mean of (gate - target)^2 over all
 *         B * H * nQB * (nQB + 1) / 2 causal entries, summed in a fixed order.
 *         Requires gate and row_sse (else SEER_ERR_INVALID_ARG).
 * Sums are fp32 per row (fixed order, bit-reproducible) and fp64 for the loss.
 */
int seer_pooled_target_mse(const float* amap, const float* gate, int B, int H, int nQB,
                           float* target, float* row_sse, float* loss, void* stream);

/*
 * Decode (one new token per sequence over a KV cache)
 * ---------------------------------------------------
 * The abstract of "SeerAttention-R: Sparse Attention Adaptation for Long
 * Reasoning" carries the learned block sparsity over to auto-regressive
 * decoding, with a token budget (4K tokens) and sparse-attention blocks of 64
 * or 128 tokens.  Conventions of the two decode calls:
 * - The cache is K, V : bf16 [B, Hkv, Tmax, D] (16-byte aligned); sequence b
 *   holds kv_len[b] tokens at positions 0 .. kv_len[b] - 1, the last of them
 *   being the new token, whose query is q[b] : bf16 [B, Hq, D].  kv_len is
 *   device int32 [B]; values are clamped to [0, Tmax] (no access outside the
 *   cache); a sequence with 0 tokens outputs zeros.
 * - Blocks are `block` tokens, block in {64, 128}; sequence b has
 *   nb = ceil(kv_len[b] / block) of them, the last one possibly short.
 * - Lists have one row per list head: list_heads = Hq (each query head its own
 *   list) or list_heads = Hkv (the G = Hq / Hkv query heads of a KV group share
 *   one list); query head h reads list head h or h / G.
 */

/*
 * Decode block lists: scores fp32 [B, H, nKB] (row stride nKB; row (b, h)
 * reads entries j < nb) -> kv_idx int32 [B, H, max_k] (ascending, -1 padded),
 * kv_cnt int32 [B, H].  The rule is the prefill row rule for the new token:
 * forced blocks are nb - 1 (holds the token) and block 0 if keep_sink; TopK
 * keeps min(nb, max(|forced|, k_blocks)) blocks (k_blocks = token budget /
 * block, >= 1); threshold keeps the forced blocks and every block whose fp32
 * score >= (float)threshold, the best-ranked ones first if max_k is short.
 * Ranking, ties and NaN as for seer_build_mask.  nb is capped at nKB.
 * nKB <= SEER_MAX_QUERY_BLOCKS (else SEER_ERR_UNSUPPORTED).
 * max_k   TopK: >= min(nKB, max(k_blocks, 2 if keep_sink else 1));
 *         threshold: >= 2 if keep_sink and nKB > 1, else >= 1.
 *         Otherwise SEER_ERR_CAPACITY.
 */
int seer_build_mask_decode(const float* scores, const int32_t* kv_len, int B, int H, int nKB,
                           int block, int mode, float threshold, int k_blocks, int keep_sink,
                           int32_t* kv_idx, int32_t* kv_cnt, int max_k, void* stream);

/* Bytes of device workspace seer_attn_gate_decode_keys needs for all blocks:
 * the pooled cache K [B,Hkv,nKB,2D] fp32, nKB = ceil(Tmax / block).  0 for
 * invalid sizes. */
size_t seer_attn_gate_decode_keys_workspace_size(int B, int Hkv, int Tmax, int D, int block);

/*
 * Per-token AttnGate of decoding.  The abstract of "SeerAttention-R: Sparse
 * Attention Adaptation for Long Reasoning" keeps the gate for decoding but
 * drops its query pooling; read here as: the K side is seer_attn_gate_scores's
 * (block [max | min] pooling of the cached K over the sequence's tokens, a
 * short last block pooling the tokens it has, the same linear layer and block
 * RoPE at the block index j), the new token's q goes through the same Q layer
 * unpooled and is rotated at its own block index nb - 1 (nb = ceil(kv_len[b] /
 * block)), and
 *   scores[b,h,j] = softmax over j' < nb of scale <Q~_{b,h}, K~_{b,g,j'}>
 * for j < nb, 0 for j >= nb (a zero row when kv_len[b] = 0).  The gate keys
 * K~ depend on the cache only, so a decoder keeps them and refreshes just the
 * block each new token joins: two calls.
 *
 * seer_attn_gate_decode_keys: k_gate [B, Hkv, nKB, Dg] fp32 (in/out) gets K~_j
 *   for every block j < nb of each sequence, or with last_block_only for block
 *   nb - 1 only (the rows of other blocks are left as they are).
 * seer_attn_gate_decode_scores: the scores of the tokens q from k_gate.
 *
 * q        device bf16 [B, Hq, D], the new tokens (before the model's RoPE).
 * k_cache  device bf16 [B, Hkv, Tmax, D] (before the model's RoPE), 16-byte
 *          aligned; kv_len device int32 [B], clamped to [0, Tmax]; positions
 *          >= kv_len[b] are never read.
 * wq, wk, Dg, scale, rope_base: as seer_attn_gate_scores (wk and k_gate
 *          16-byte aligned).
 * block    64 or 128 (the list block of seer_build_mask_decode); nKB =
 *          ceil(Tmax / block) <= SEER_MAX_QUERY_BLOCKS.
 * scores   device fp32 out [B, Hq, nKB], the input of seer_build_mask_decode.
 * workspace (keys over all blocks only; may be NULL with last_block_only)
 *          device, >= seer_attn_gate_decode_keys_workspace_size(B, Hkv, Tmax,
 *          D, block) bytes, 256-byte aligned; overwritten.
 * Arithmetic is fp32 (all-block keys on the fp32 matrix cores, single rows on
 * the VALU, RoPE angles reduced in fp64); results are bit-reproducible.
 */
int seer_attn_gate_decode_keys(const void* k_cache, const int32_t* kv_len, int B, int Hkv,
                               int Tmax, int D, const float* wk, int Dg, float rope_base,
                               int block, int last_block_only, float* k_gate, void* workspace,
                               size_t workspace_bytes, void* stream);
int seer_attn_gate_decode_scores(const void* q, const float* k_gate, const int32_t* kv_len,
                                 int B, int Hq, int Hkv, int Tmax, int D, const float* wq,
                                 int Dg, float scale, float rope_base, int block, float* scores,
                                 void* stream);

/*
 * seer_attn_gate_decode_scores and seer_build_mask_decode in one pass: each
 * (sequence, query head) computes its score row as the scores call does and
 * selects its blocks from it on chip with the decode rule of
 * seer_build_mask_decode (H = Hq, nKB = ceil(Tmax / block)), so kv_idx and
 * kv_cnt equal the two-call result bit for bit and the scores need not go
 * through memory.  scores may be NULL; if given it receives the same row as
 * the scores call.  Arguments and errors are those of the two calls; in
 * addition B * Hq * max_k must fit in int32 (else SEER_ERR_UNSUPPORTED).
 */
int seer_attn_gate_decode_mask(const void* q, const float* k_gate, const int32_t* kv_len, int B,
                               int Hq, int Hkv, int Tmax, int D, const float* wq, int Dg,
                               float scale, float rope_base, int block, int mode,
                               float threshold, int k_blocks, int keep_sink, int32_t* kv_idx,
                               int32_t* kv_cnt, int max_k, float* scores, void* stream);

/* Bytes of device workspace seer_sparse_decode needs (the union of a KV
 * group's per-head lists, and one partial softmax state per chunk of blocks
 * and query head).  0 for invalid sizes. */
size_t seer_sparse_decode_workspace_size(int B, int Hq, int Hkv, int Tmax, int D,
                                         int list_heads, int max_k, int block);

/*
 * Block-sparse decode attention: for each sequence b and query head h,
 *   o[b,h] = softmax over the allowed keys c of sm_scale <q[b,h], k[b,g,c]>,
 *            times v[b,g,c],   g = h / G,
 * where c is allowed iff c < kv_len[b] and block c / block is listed in
 * kv_idx[b, lh, 0:min(kv_cnt[b, lh], max_k)] (lh the list head of h).  The
 * same definition as seer_sparse_prefill's for the last query row
 * (rebuttal "SeerAttention: Learning Intrinsic Sparse Attention in Your
 * LLMs", "Weakness 5 (Pseudo code of Inference Kernel)").
 *
 * q        device bf16 [B, Hq, D]; k_cache, v_cache device bf16 [B, Hkv, Tmax, D];
 *          D in {64, 128}; Hq % Hkv == 0 and G = Hq / Hkv <= 8; Tmax >= 1 and
 *          ceil(Tmax / block) <= 32768.
 * kv_len   device int32 [B] (see above).
 * kv_idx   device int32 [B, list_heads, max_k], kv_cnt device int32
 *          [B, list_heads]; list_heads in {Hq, Hkv}.  Entries outside [0, nb)
 *          are skipped, order does not matter, a list must not repeat a block.
 *          A head with no valid entry outputs zeros.
 * o        device bf16 out [B, Hq, D], rounded to nearest even.
 * workspace device, >= seer_sparse_decode_workspace_size(...) bytes, 256-byte
 *          aligned; overwritten.
 * Each selected block is read once per KV group.  Results are bit-reproducible.
 */
int seer_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* kv_len, int B, int Hq, int Hkv, int Tmax, int D,
                       float sm_scale, int block, const int32_t* kv_idx, const int32_t* kv_cnt,
                       int list_heads, int max_k, void* o, void* workspace,
                       size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SEER_H_ */
