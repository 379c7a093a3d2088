/*
 * amtk.h - C ABI of the attention-mass top-k oracle library (libamtk.so) for
 * long-context causal prefill of full/GQA attention layers on gfx950.
 *
 * Method: "How Much Dense Attention is Necessary? Oracle-Guided Sparse
 * Prefill for Full/GQA Layers in Hybrid Long-Context Models" (arXiv
 * 2606.07703). Citations below name two pages about it:
 *   [Abstract] the authors' abstract (searcharxiv.org page);
 *   [TB x.y]   the gist.science page, "Technischer Bericht", section x.y.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are DEVICE pointers owned by the caller, row-major, contiguous,
 *    16-byte aligned. Q is [n][hq][d], K and V are [n][hkv][d] (token major:
 *    one token's keys for all KV heads are hkv*d contiguous elements).
 *    Q, K, V share one element type (amtk_attn_desc.dtype).
 *  - Query head h reads KV head h / (hq/hkv) (contiguous GQA groups).
 *  - Row i attends to keys j <= i (causal prefill).
 *  - Logits are scale * <Q[i,h], K[j,g]>; scale <= 0 selects 1/sqrt(d).
 *  - Every call validates its arguments on the host first and launches
 *    nothing when a check fails. Work is enqueued asynchronously on `stream`
 *    (a hipStream_t; NULL = the null stream). The library never allocates,
 *    frees or synchronises; it keeps no mutable global state, so calls on
 *    different streams with disjoint outputs and workspaces may overlap.
 *  - Every element of every output is written (-1 / 0 padding included).
 *  - Return value: AMTK_OK or a negative AMTK_E_* code (see amtk_strerror).
 */
#ifndef AMTK_H
#define AMTK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AMTK_OK 0
#define AMTK_E_INVALID (-1)     /* null pointer, bad size, inconsistent arguments */
#define AMTK_E_UNSUPPORTED (-2) /* well-formed but outside what the kernels cover */
#define AMTK_E_WORKSPACE (-3)   /* workspace smaller than the *_workspace query says */
#define AMTK_E_HIP (-4)         /* a HIP launch failed; see amtk_last_hip_error */

#define AMTK_BF16 0
#define AMTK_F32 1

/* One GQA attention layer in prefill. */
typedef struct {
  int64_t n;      /* tokens (rows), 1 <= n < 2^31 */
  int32_t hq;     /* query heads */
  int32_t hkv;    /* KV heads; hq % hkv == 0 */
  int32_t d;      /* head dim: 64 or 128 */
  int32_t dtype;  /* AMTK_BF16 or AMTK_F32 (arithmetic is fp32 either way) */
  int32_t causal; /* must be 1: the method is defined for causal prefill */
  float scale;    /* softmax temperature on the logits; <= 0 means 1/sqrt(d) */
} amtk_attn_desc;

/* Support granularity and budget ([TB 2.1]: budget k and support granularity;
 * [TB 2.2]: k stays adjustable at inference). */
typedef struct {
  int32_t k;             /* budget, in key_block units, 1 <= k <= 8192 */
  int32_t key_block;     /* 1 = token support, 64 = aligned 64-token key blocks */
  int32_t query_block;   /* queries sharing one support (b_sel): 1 (per query) or
                            64 (with key_block = 1), see topk_support */
  int32_t candidate_cap; /* candidates kept per row by the streaming filter;
                            0 = automatic; values above 65000 are clamped.
                            Rows that exceed it are recomputed densely, so
                            any value >= 1 gives the same result. */
} amtk_support_desc;

/* Bytes of device workspace topk_support / oracle_prefill need for these
 * shapes (written to *bytes). Returns AMTK_OK or a validation error. */
int amtk_topk_workspace(const amtk_attn_desc* attn, const amtk_support_desc* sup, size_t* bytes);

/* The same figure as a plain return value: the workspace bytes of
 * topk_support / oracle_prefill for these shapes, or 0 when the descriptors
 * are invalid or unsupported (amtk_topk_workspace reports which). */
size_t amtk_workspace_bytes(const amtk_attn_desc* attn, const amtk_support_desc* sup);

/*
 * topk_support - the attention-mass top-k oracle's support selection.
 * [TB 2.1], [Abstract]: for every query row i the per-head causal softmax
 * p_h(i,j) = exp(s_h(i,j) - LSE_h(i)) is averaged over all hq heads,
 * P_i(j) = (1/hq) sum_h p_h(i,j), and the top-k units of P_i are kept.
 * key_block = 64 ranks aligned key blocks by M_i(b) = sum of P_i(j) over the
 * block's keys j <= i. Units are ranked by mass descending, then id ascending.
 * A row with at most k visible units keeps all of them.
 *
 * Two passes over the causal score matrix (per-head LSE, then mass + streaming
 * threshold filter) and an exact select; the n x n mass is never stored.
 *
 * query_block = 64 ([TB 2.1]: a selection-block-shared support, one support
 * set for a block of 64 consecutive queries): the block scores key j by the
 * mean over its rows of P_i(j), keys after row i counting 0 for that row, and
 * its top-k keys among those its last row sees are written into the index
 * row of every query of the block (mass = the block score). sparse_attn then
 * skips, for each row, the shared keys after it. The last block holds the
 * remaining rows. Pass 2 then writes the column sums of P over each 32-row
 * tile into the workspace ((n+31)/32 x n floats) instead of filtering.
 *
 * q, k      : inputs as described above.
 * idx       : OUT [n][k] int32, row i's selected unit ids (token ids, or key
 *             block ids when key_block = 64) ascending, then -1 padding.
 * count     : OUT [n] int32, number of selected units = min(k, visible units)
 *             (query_block = 64: the keys the block's last row sees).
 * mass      : OUT [n][k] fp32 mass of each selected unit (0 padding), or NULL.
 * lse       : OUT [hq][n] fp32 per-head dense log-sum-exp (natural log), or NULL.
 * ws        : device workspace of ws_bytes >= amtk_topk_workspace(); its
 *             contents on entry are ignored; it is owned by the caller and
 *             must not be shared by calls that run concurrently.
 */
int topk_support(const amtk_attn_desc* attn, const amtk_support_desc* sup, const void* q,
                 const void* k, int32_t* idx, int32_t* count, float* mass, float* lse, void* ws,
                 size_t ws_bytes, void* stream);

/*
 * topk_support_stage - one stage of topk_support, for callers that time or
 * schedule the stages separately. Calling stages 1, 2, 3 in that order on
 * one stream with the same arguments and workspace is exactly topk_support:
 *   stage 1: per-head dense log-sum-exp pass (writes lse, or the workspace's
 *            copy when lse is NULL);
 *   stage 2: head-averaged mass pass with the streaming top-k filter
 *            (candidate pool in the workspace);
 *   stage 3: exact select from the pool (rows whose pool overflowed are
 *            recomputed densely), writes idx, count and mass.
 * Stages 2 and 3 read what the earlier stages left in ws (and lse).
 */
int topk_support_stage(const amtk_attn_desc* attn, const amtk_support_desc* sup, int32_t stage,
                       const void* q, const void* k, int32_t* idx, int32_t* count, float* mass,
                       float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * sparse_attn - attention recomputed on each row's support only.
 * [TB 2.1], [TB 2.2], [Abstract]: O_i[h] = sum_{j in S_i}
 * softmax_{S_i}(s_h(i,j)) V[j, g(h)], the softmax renormalised over S_i.
 * S_i is given by idx/count in the layout topk_support writes:
 * key_block = 1: idx[i][0..count[i]) are token ids; key_block = 64: they are
 * key block ids, expanded to tokens b*64 .. b*64+63 and clipped to j <= i.
 * Negative ids and tokens j > i are skipped; count[i] is clamped to
 * [0, max_units]. A row with an empty support gets O = 0 and LSE = -inf.
 * The ids of a row may come in any order; they are expected to be distinct
 * (topk_support writes them so), a repeated id counting once per entry.
 *
 * idx       : [n][max_units] int32 (device); count: [n] int32 (device).
 * o         : OUT [n][hq][d] fp32.
 * lse_sparse: OUT [hq][n] fp32 log-sum-exp over the support, or NULL.
 */
int sparse_attn(const amtk_attn_desc* attn, int32_t key_block, int32_t max_units, const void* q,
                const void* k, const void* v, const int32_t* idx, const int32_t* count, float* o,
                float* lse_sparse, void* stream);

/* Scratch bytes of sparse_attn_windowed for this layer shape. */
int amtk_sparse_attn_workspace(const amtk_attn_desc* attn, size_t* bytes);

/*
 * sparse_attn_windowed - sparse_attn computed in key windows: the same
 * result (up to fp32 rounding order) with better cache reuse at long n.
 * [TB 2.1], [TB 2.2], [Abstract], as sparse_attn. The supports are walked
 * in windows of at least 8192 consecutive key tokens, one launch per
 * window; each launch attends every row over its ids in that window and
 * merges the partial softmax into o (o stays normalised; the running LSE
 * lives in lse_sparse when given, else in ws). Rows whose ids are ascending
 * (as topk_support writes them) are split this way; a row whose ids are not
 * ascending is attended whole in the first window. Where the windowed form
 * does not apply (other shapes than bf16, d = 128, hq / hkv in {1, 2, 4, 8}
 * with n * hkv * 256 < 2^32; n of one window) the call is sparse_attn.
 *
 * Arguments as sparse_attn, plus ws: device scratch of ws_bytes >=
 * amtk_sparse_attn_workspace bytes, 256-byte aligned, owned by the caller
 * (AMTK_E_WORKSPACE if smaller). Its contents on return are unspecified.
 */
int sparse_attn_windowed(const amtk_attn_desc* attn, int32_t key_block, int32_t max_units,
                         const void* q, const void* k, const void* v, const int32_t* idx,
                         const int32_t* count, float* o, float* lse_sparse, void* ws,
                         size_t ws_bytes, void* stream);

/* Bytes of the static device scratch array of sparse_attn_windowed_static
 * (one copy per GPU, held until the process ends). */
#define AMTK_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * sparse_attn_windowed_static - sparse_attn_windowed for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It takes no workspace: the windowed
 * gather's scratch (window starts of every row, and the running LSE when
 * lse_sparse is NULL) lives in a static device array of
 * AMTK_STATIC_SCRATCH_BYTES on each GPU. The call allocates and frees
 * nothing; the result is exactly that of sparse_attn_windowed (same kernels).
 * Arguments and validation as sparse_attn_windowed, without ws / ws_bytes.
 * The array of the CURRENT device (hipGetDevice) is used, so the current
 * device must be the device of `stream`; its address is resolved at the
 * first call on each device.
 * Limit: the layer's scratch, amtk_sparse_attn_workspace() = n * 4 * (key
 * windows + 1) + hq * n * 4 bytes (rounded to 256), must fit the array:
 * n up to about 160K tokens at hq = 32. Larger layers return
 * AMTK_E_WORKSPACE before anything is launched.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs clearing: every word a call reads, the call
 * writes first). Calls that overlap on one GPU (other streams, other host
 * threads) race on the array and must be serialised by the caller.
 */
int sparse_attn_windowed_static(const amtk_attn_desc* attn, int32_t key_block,
                                int32_t max_units, const void* q, const void* k, const void* v,
                                const int32_t* idx, const int32_t* count, float* o,
                                float* lse_sparse, void* stream);

/*
 * sparse_attn_blocks - attention of each selection block's queries on the
 * block's shared support, the keys gathered once per block.
 * [TB 2.1]: with selection-block-shared granularity one support set serves
 * a block of query_block consecutive queries; each query i then attends
 * over the shared keys j <= i, softmax renormalised over them.
 * Block t holds rows t*query_block .. min((t+1)*query_block, n) - 1; its
 * support is idx[t*query_block][0..count[t*query_block]) (token ids, or
 * key-block ids expanded to their 64 tokens when key_block = 64; any order,
 * distinct), i.e. the first row of the block in the [n][max_units] layout
 * topk_support / indexer_topk write with sup->query_block = query_block. The
 * other rows' entries are not read. Per row, negative ids, tokens >= n and
 * tokens > i are skipped; a row left with no key gets O = 0 and LSE = -inf.
 * The result equals sparse_attn (same key_block) when every row of a block
 * holds the block's support.
 * query_block = 64. bf16, d = 128, hkv = 8, hq = 32 runs the block tile
 * kernel (the block's keys gathered once); every other shape sparse_attn
 * takes runs its per-row gather, each row reading its block's first index
 * row (same result, keys gathered per row); anything else returns
 * AMTK_E_UNSUPPORTED.
 *
 * idx       : [n][max_units] int32 (device); count: [n] int32 (device).
 * o         : OUT [n][hq][d] fp32.
 * lse_sparse: OUT [hq][n] fp32 log-sum-exp over each row's keys, or NULL.
 */
int sparse_attn_blocks(const amtk_attn_desc* attn, int32_t key_block, int32_t query_block,
                       int32_t max_units, const void* q, const void* k, const void* v,
                       const int32_t* idx, const int32_t* count, float* o, float* lse_sparse,
                       void* stream);

/*
 * oracle_prefill - topk_support followed by sparse_attn on the same stream:
 * the oracle's full per-layer step (dense mass -> top-k support -> sparse
 * recompute with the original Q/K/V), [TB 2.1], [Abstract].
 * Arguments as in the two calls above; idx and count are required outputs.
 * With sup->query_block = 64 the sparse step is sparse_attn_blocks where it
 * supports the shape, else sparse_attn on the per-row copies. With
 * query_block = 1 it is sparse_attn_windowed, its scratch taken from the
 * candidate pool of ws (free once the supports are selected) when the pool
 * is large enough, else sparse_attn.
 */
int oracle_prefill(const amtk_attn_desc* attn, const amtk_support_desc* sup, const void* q,
                   const void* k, const void* v, float* o, int32_t* idx, int32_t* count,
                   float* mass, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of indexer_topk for these shapes. */
int amtk_indexer_workspace(int64_t n, int32_t d_idx, int32_t dtype,
                           const amtk_support_desc* sup, size_t* bytes);

/*
 * indexer_topk - head-collapsed indexer scoring and top-k.
 * [TB 2.2], [Abstract]: one shared score per key replaces per-head scores,
 * s(i,j) = scale * <q_idx[i], k_idx[j]>; P_idx = causal softmax over j <= i;
 * units are tokens (key_block = 1) or aligned 64-token key blocks ranked by
 * their summed P_idx (key_block = 64); the top-k units feed sparse_attn.
 *
 * q_idx, k_idx: [n][d_idx] device tensors, d_idx = 64 or 128.
 * scale <= 0 selects 1/sqrt(d_idx).
 * idx/count/mass/ws as in topk_support.
 * sup->query_block = 64 ([TB 2.1] selection blocks, realised with the
 * indexer): one support per block of 64 queries; a unit scores the mean over
 * the block's rows of their P_idx on its keys up to the row, the top-k units
 * among those the last row sees go into the index row of every query of the
 * block (mass = the block score). key_block = 64 runs one kernel per block
 * (bf16, d_idx = 64, k <= 1024, at most 2048 key blocks); key_block = 1 the
 * column-sum path of topk_support.
 */
int indexer_topk(int64_t n, int32_t d_idx, int32_t dtype, float scale,
                 const amtk_support_desc* sup, const void* q_idx, const void* k_idx,
                 int32_t* idx, int32_t* count, float* mass, void* ws, size_t ws_bytes,
                 void* stream);

/*
 * indexer_prefill - the indexer-driven sparse prefill of one layer: the
 * indexer's support from (q_idx, k_idx), then attention of (q, k, v) on it.
 * [TB 2.2] (indexer inference: score, select top-k, recompute attention on
 * the chosen tokens); [TB 2.3], [Abstract] (runtime realisation: selection
 * blocks and kernel fusion).
 * sup->query_block = 1: the per-query realisation, indexer_topk then
 * sparse_attn (key_block as given).
 * sup->query_block = 64, key_block = 64: the fused realisation. After the
 * indexer's LSE pass one kernel per block of 64 queries scores the key
 * blocks, selects the shared top-k and attends over them for every KV head
 * (bf16, d = 128, hkv = 8, hq = 32, d_idx = 64, k <= 1024). With other
 * backbone head layouts, or key_block = 1, the same support is formed by
 * indexer_topk (query_block 64, written to every row of a block) and
 * attended by sparse_attn row by row.
 * q_idx, k_idx: [n][d_idx], the layer's dtype. idx_scale <= 0: 1/sqrt(d_idx).
 * o: OUT [n][hq][d] fp32; idx/count/mass: OUT, the support as indexer_topk
 * writes it (mass may be NULL). ws: ws_bytes >= amtk_indexer_workspace(n,
 * d_idx, dtype, sup).
 */
int indexer_prefill(const amtk_attn_desc* attn, int32_t d_idx, float idx_scale,
                    const amtk_support_desc* sup, const void* q, const void* k, const void* v,
                    const void* q_idx, const void* k_idx, float* o, int32_t* idx, int32_t* count,
                    float* mass, void* ws, size_t ws_bytes, void* stream);

/*
 * captured_mass - per row, the head-averaged dense attention mass that a
 * support keeps: captured[i] = sum_{j in S_i} P_i(j)
 *                            = (1/hq) sum_h exp(lse_support[h][i] - lse_dense[h][i]).
 * [TB 2.3]: the layer-level analogue of the oracle, indexer and realization
 * gaps (how much of the dense mass the oracle's, an indexer's or a shared
 * block support keeps).
 * lse_dense  : [hq][n] fp32 dense per-head LSE (topk_support's lse output).
 * lse_support: [hq][n] fp32 LSE over the support (lse_sparse of sparse_attn
 *              or sparse_attn_blocks on that support); -inf (an empty
 *              support) counts 0.
 * captured   : OUT [n] fp32.
 */
int captured_mass(int64_t n, int32_t hq, const float* lse_dense, const float* lse_support,
                  float* captured, void* stream);

/*
 * support_overlap - per row, the number of ids two supports share
 * (overlap / count_a is the recall of support a by support b).
 * [TB 2.3]: the indexer gap compares an indexer's support with the oracle's.
 * idx_a [n][max_a], count_a [n]; idx_b [n][max_b], count_b [n]: the ids of
 * each row ascend within its count (as topk_support and indexer_topk write
 * them); counts are clamped to [0, max]; both supports use the same units
 * (tokens, or key blocks). Negative ids never match.
 * overlap: OUT [n] int32.
 */
int support_overlap(int64_t n, int32_t max_a, const int32_t* idx_a, const int32_t* count_a,
                    int32_t max_b, const int32_t* idx_b, const int32_t* count_b,
                    int32_t* overlap, void* stream);

/* Bytes of device workspace kl_distill needs for these shapes. */
int amtk_kl_workspace(const amtk_attn_desc* attn, int32_t d_idx, size_t* bytes);

/*
 * kl_distill - KL-distillation loss of the head-collapsed indexer against the
 * oracle's dense head-averaged attention mass, and its gradients.
 * [TB 2.2]: the indexer is trained by KL divergence from the dense
 * attention-mass distribution, the backbone frozen. Teacher P_i = head-averaged
 * mass of (q, k) over keys j <= i; student Q_i = causal softmax over j <= i of
 * t_ij = idx_scale * <q_idx[i], k_idx[j]> (idx_scale <= 0: 1/sqrt(d_idx)).
 *   kl_row[i] = sum_j P_ij (log P_ij - log Q_ij)     (P_ij = 0 terms count 0)
 *   loss      = (1/n) sum_i kl_row[i]
 *   dq_idx[i] = dloss/dq_idx[i] = (idx_scale/n) sum_j (Q_ij - P_ij) k_idx[j]
 *   dk_idx[j] = dloss/dk_idx[j] = (idx_scale/n) sum_{i>=j} (Q_ij - P_ij) q_idx[i]
 * No n x n matrix, and no array of that size, is stored: the workspace is
 * O(n * (hq + hkv * d_idx)) floats (the dense LSE, the student LSE and the
 * key gradient's per-KV-group shares) plus, for 32/8 heads, a copy of K. Both gradients are deterministic
 * (fixed summation order).
 * q, k      : as for topk_support; bf16, d = 128, 4 query heads per KV head
 *             and 1, 2, 4 or 8 KV heads (hq = 4 * hkv); anything else returns
 *             AMTK_E_UNSUPPORTED.
 * q_idx     : [n][d_idx] bf16 (device), k_idx: [n][d_idx] bf16; d_idx = 64.
 * kl_row    : OUT [n] fp32.   loss: OUT [1] fp32, or NULL.
 * dq_idx    : OUT [n][d_idx] fp32.   dk_idx: OUT [n][d_idx] fp32.
 * ws        : device workspace of ws_bytes >= amtk_kl_workspace()
 *             (n * (hq + 1 + hkv * d_idx) * 4 bytes, with 8 KV heads x 4
 *             query heads plus a copy of K in MFMA operand order for the
 *             teacher's LSE pass, plus alignment: 138 MB at n = 32768 with
 *             32/8 heads).
 */
int kl_distill(const amtk_attn_desc* attn, int32_t d_idx, float idx_scale, const void* q,
               const void* k, const void* q_idx, const void* k_idx, float* kl_row, float* loss,
               float* dq_idx, float* dk_idx, void* ws, size_t ws_bytes, void* stream);

/* Message for an AMTK_* code. Never NULL. */
const char* amtk_strerror(int code);

/* The hipError_t of the most recent AMTK_E_HIP returned on this thread. */
int amtk_last_hip_error(void);

/*
 * amtk_pool_stats - diagnostics of the last topk_support / indexer_topk run
 * that used workspace `ws` (same descriptors). Copies the per-row candidate
 * counts back and reports the largest count, the number of rows whose pool
 * overflowed the capacity (recomputed densely), and the capacity itself.
 * SYNCHRONOUS: waits for `stream`. For tests and tuning only.
 * AMTK_E_UNSUPPORTED for query_block = 64 (no candidate pools are kept).
 */
int amtk_pool_stats(const amtk_attn_desc* attn, const amtk_support_desc* sup, const void* ws,
                    size_t ws_bytes, int64_t* max_candidates, int64_t* overflow_rows,
                    int64_t* capacity, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AMTK_H */
