// Internal launchers behind the C-ABI (not exported). Every launcher assumes
// its arguments were validated by the API layer and only enqueues work on
// `stream`; none allocates, frees or synchronises.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "amtk.h"

namespace amtk {

enum ElemType { kBF16 = 0, kF32 = 1 };

struct LayerShape {
  int n;        // tokens
  int hq;       // query heads
  int hkv;      // KV heads
  int d;        // head dim
  int dtype;    // ElemType
  float scale;  // softmax temperature on the logits
};

// Candidate pool produced by pass 2 and consumed by the select kernels.
struct CandidatePool {
  uint2* cand;      // [n][cap] (mass bits, unit id)
  int* count;       // [n] candidates seen (may exceed cap: overflow)
  int* bin;         // [n] final threshold bin (diagnostic)
  int* ovf_count;   // [1] rows whose pool overflowed
  int* ovf_list;    // [n] their row ids
  float* scratch;   // [slots][units_max] dense rows for the overflow path
  void* kops;       // key tiles in MFMA operand order (pass2_key_operand_bytes)
  int cap;          // capacity per row
  int slots;        // overflow rows processed concurrently
  bool kops_ready = false;   // kops already holds this call's keys (written by pass 1)
};

constexpr int kMaxBudget = 8192;      // largest k the select kernel sorts in LDS
constexpr size_t kLdsBytesPerCu = 160 * 1024;   // LDS of one gfx950 CU (one workgroup's maximum)
constexpr int kMaxQRow = 8192;        // largest Hq*d held in LDS by the overflow path
constexpr int kFallbackSlots = 128;   // concurrent overflow rows

// Bytes of pass 2's copy of the keys in MFMA operand order (8 KV heads, bf16,
// d = 128, one support per query; 0 for other shapes, which stage key tiles
// through LDS instead).
size_t pass2_key_operand_bytes(const LayerShape& s, int key_block);

// Per-head causal row log-sum-exp, lse[h][i] (natural log). Also zeroes
// pool.ovf_count for the pass that follows.
hipError_t launch_pass1_lse(const LayerShape& s, const void* q, const void* k, float* lse,
                            int* zero_counter, hipStream_t stream);
// The same for bf16, d = 128, 1, 2, 4 or 8 KV heads and 2 or 4 query heads
// per KV head with a workspace of pass1_key_operand_bytes(s) at kops: the
// keys are copied there in MFMA operand order, and pass 1 reads them
// straight into registers. Other shapes (or kops == nullptr) run
// launch_pass1_lse.
hipError_t launch_pass1_lse_kops(const LayerShape& s, const void* q, const void* k, float* lse,
                                 int* zero_counter, void* kops, hipStream_t stream);
// Whether launch_pass1_lse_kops takes the direct path (and so writes kops),
// and the bytes of kops it then needs.
bool pass1_writes_kops(const LayerShape& s);
size_t pass1_key_operand_bytes(const LayerShape& s);
// The pass-1 kernel of launch_pass1_lse_kops alone (kops already written).
hipError_t launch_pass1_direct(const LayerShape& s, const void* q, const void* kops, float* lse,
                               int* zero_counter, hipStream_t stream);

// Head-averaged mass, streaming threshold filter, candidate compaction.
hipError_t launch_pass2_filter(const LayerShape& s, int key_block, int budget, const void* q,
                               const void* k, const float* lse, const CandidatePool& pool,
                               hipStream_t stream);

// Selection blocks of consecutive queries: column sums of the head-averaged
// mass over each 32-row tile, colsum[tile][j] (keys j up to the tile's last
// row), in place of the per-row filter.
hipError_t launch_pass2_colsum(const LayerShape& s, const void* q, const void* k, const float* lse,
                               float* colsum, hipStream_t stream);

// The shared top-k of each selection block of bsel rows (a multiple of 32)
// from those column sums, written into the index row of every query of the
// block (ascending ids, -1 padding), with the block scores as masses.
hipError_t launch_block_topk(const LayerShape& s, int bsel, int budget, const float* colsum,
                             int32_t* idx, int32_t* count, float* mass, hipStream_t stream);

// Exact top-k from each row's candidates (rows whose pool did not overflow),
// then the dense recompute + select for rows that did.
hipError_t launch_select(const LayerShape& s, int key_block, int budget, const void* q,
                         const void* k, const float* lse, const CandidatePool& pool, int32_t* idx,
                         int32_t* count, float* mass, hipStream_t stream);

// Attention on each row's support (token ids or key blocks), fp32 output.
hipError_t launch_sparse_attn(const LayerShape& s, int key_block, int max_units, const void* q,
                              const void* k, const void* v, const int32_t* idx,
                              const int32_t* count, float* o, float* lse_sparse,
                              hipStream_t stream);
// The same for selection blocks of query_block (a power of two) consecutive
// rows: every row reads the ids and count of its block's first row and
// skips the ids after itself. One pass, any shape sparse_attn takes.
hipError_t launch_sparse_attn_block_rows(const LayerShape& s, int key_block, int query_block,
                                         int max_units, const void* q, const void* k,
                                         const void* v, const int32_t* idx,
                                         const int32_t* count, float* o, float* lse_sparse,
                                         hipStream_t stream);
// The same in key windows (one launch per window, partial softmax merged
// into o); scratch of sparse_windowed_scratch_bytes. Falls back to
// launch_sparse_attn where the windowed form does not apply.
size_t sparse_windowed_scratch_bytes(const LayerShape& s);
hipError_t launch_sparse_attn_windowed(const LayerShape& s, int key_block, int max_units,
                                       const void* q, const void* k, const void* v,
                                       const int32_t* idx, const int32_t* count, float* o,
                                       float* lse_sparse, void* scratch, size_t scratch_bytes,
                                       hipStream_t stream);

// Attention of each selection block's queries on the block's shared
// support: the ids and count of the block's first row serve all of its rows,
// each row skipping the ids after it. bf16, d = 128, 8 KV heads x 4 query
// heads, blocks of 64 queries (shared_attn_shape_supported).
hipError_t launch_shared_attn(const LayerShape& s, int key_block, int query_block, int max_units,
                              const void* q, const void* k, const void* v, const int32_t* idx,
                              const int32_t* count, float* o, float* lse_sparse,
                              hipStream_t stream);
bool shared_attn_shape_supported(const LayerShape& s, int query_block);

// The indexer's support shared by each block of 64 queries (key blocks of
// 64): scores and top-k in one kernel per block, given the indexer's row LSE
// lse_idx [n]. With attn (q, k, v, o, lse_sparse) the same kernel then runs
// the block's attention on the shared keys for every KV head (the fused
// realisation); attn = nullptr selects only.
bool indexer_shared_supported(int n, int d_idx, int dtype, int key_block, int query_block,
                              int budget);
hipError_t launch_indexer_shared(int n, int key_block, int budget, float idx_scale,
                                 const void* q_idx, const void* k_idx, const float* lse_idx,
                                 int32_t* idx, int32_t* count, float* mass,
                                 const LayerShape* attn, const void* q, const void* k,
                                 const void* v, float* o, float* lse_sparse, hipStream_t stream);

// Diagnostics: captured[i] = (1/hq) sum_h exp(lse_support[h][i] - lse_dense[h][i])
// (-inf support LSE counts 0); overlap[i] = ids shared by two supports whose
// ids ascend within their counts.
hipError_t launch_captured_mass(int n, int hq, const float* lse_dense, const float* lse_support,
                                float* captured, hipStream_t stream);
hipError_t launch_support_overlap(int n, int max_a, const int32_t* idx_a, const int32_t* count_a,
                                  int max_b, const int32_t* idx_b, const int32_t* count_b,
                                  int32_t* overlap, hipStream_t stream);

// KL distillation of the indexer (q_idx, k_idx: [n][d_idx] bf16) against the
// head-averaged mass of (q, k): per-row KL, the mean loss (if loss is not
// null) and the gradients of the mean loss, given the dense per-head LSE
// lse [hq][n] and the student's LSE lse_t [n]. dk_part: kl_partial_bytes(n, hkv)
// of scratch (the key gradient's per-KV-group shares, hkv x n x d_idx
// floats). bf16, d = 128, 4 query heads per KV head, 1, 2, 4 or 8 KV heads,
// d_idx = 64.
bool kl_shape_supported(const LayerShape& s, int d_idx);
size_t kl_partial_bytes(int n, int hkv);
hipError_t launch_kl_distill(const LayerShape& s, int d_idx, float idx_scale, const void* q,
                             const void* k, const void* q_idx, const void* k_idx,
                             const float* lse, const float* lse_t, float* kl_row, float* loss,
                             float* dq, float* dk, float* dk_part, hipStream_t stream);

// Host-side helpers of the entry points (api.hip): the layer descriptor's
// validation (AMTK_OK or an AMTK_E_* code, *s filled on success), and the
// bookkeeping of a failed HIP call (keeps e for amtk_last_hip_error on this
// thread, returns AMTK_E_HIP).
int validate_attn(const amtk_attn_desc* a, LayerShape* s);
int record_hip_error(hipError_t e);

bool pass_shape_supported(const LayerShape& s);
bool sparse_shape_supported(const LayerShape& s);

}  // namespace amtk
