// C-ABI entry points of libamtk.so (declared in include/amtk.h).
//
// Host-side only: validates descriptors and pointers, carves the caller's
// workspace, and enqueues the kernels on the caller's stream. Nothing here
// allocates device memory or synchronises (except amtk_pool_stats, which is
// documented as a synchronous diagnostic).
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "amtk.h"
#include "kernels.h"

using amtk::CandidatePool;
using amtk::LayerShape;

namespace {

thread_local int g_last_hip = 0;

// Candidate pool capacity per row is kept below 2^16 - 32: the pass-2 filter
// counts candidates per mass bin in 16-bit LDS counters.
constexpr int kMaxCap = 65000;

// Rows per selection block when a support is shared by consecutive queries.
constexpr int kQueryBlock = 64;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return AMTK_E_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

int check_attn(const amtk_attn_desc* a, LayerShape* s) {
  if (!a) return AMTK_E_INVALID;
  if (a->n < 1 || a->n >= (int64_t)1 << 31) return AMTK_E_INVALID;
  if (a->hq < 1 || a->hkv < 1 || a->d < 1) return AMTK_E_INVALID;
  if (a->hq % a->hkv) return AMTK_E_INVALID;
  if (a->dtype != AMTK_BF16 && a->dtype != AMTK_F32) return AMTK_E_INVALID;
  if (std::isnan(a->scale) || std::isinf(a->scale)) return AMTK_E_INVALID;
  if (a->causal != 1) return AMTK_E_UNSUPPORTED;
  if (a->d != 64 && a->d != 128) return AMTK_E_UNSUPPORTED;
  s->n = (int)a->n;
  s->hq = a->hq;
  s->hkv = a->hkv;
  s->d = a->d;
  s->dtype = a->dtype;
  s->scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)a->d);
  return AMTK_OK;
}

int check_support(const amtk_support_desc* sp) {
  if (!sp) return AMTK_E_INVALID;
  if (sp->k < 1 || sp->candidate_cap < 0) return AMTK_E_INVALID;
  if (sp->k > amtk::kMaxBudget) return AMTK_E_UNSUPPORTED;
  if (sp->key_block != 1 && sp->key_block != 64) return AMTK_E_UNSUPPORTED;
  if (sp->query_block != 1 && sp->query_block != kQueryBlock) return AMTK_E_UNSUPPORTED;
  return AMTK_OK;
}

struct Layout {
  size_t cand, count, bin, lse, ovf_count, ovf_list, scratch, colsum, kops, kops_bytes, total;
  int cap, units_max;
};

Layout layout(const LayerShape& s, const amtk_support_desc& sp) {
  Layout L;
  const size_t n = (size_t)s.n;
  if (sp.query_block != 1) {   // selection blocks: LSE and the tiles' column sums
    L = Layout{};
    L.units_max = s.n;
    size_t off = 0;
    L.lse = off;     off = round_up(off + (size_t)s.hq * n * sizeof(float));
    L.ovf_count = off; off = round_up(off + sizeof(int));
    // column sums per 32-row tile (token units only; key blocks are scored
    // per selection block without them)
    const size_t cs = sp.key_block == 1 ? (n + 31) / 32 * n * sizeof(float) : 0;
    L.colsum = off;  off = round_up(off + cs);
    // pass 1 reads the keys from a copy in MFMA operand order where it can
    L.kops_bytes = sp.key_block == 1 ? amtk::pass1_key_operand_bytes(s) : 0;
    L.kops = off;    off = round_up(off + L.kops_bytes);
    L.total = off;
    return L;
  }
  L.units_max = sp.key_block == 1 ? s.n : (s.n - 1) / sp.key_block + 1;
  int cap = sp.candidate_cap > 0 ? sp.candidate_cap
                                 : (8 * sp.k > 4096 ? 8 * sp.k : 4096);
  if (cap > L.units_max) cap = L.units_max;
  if (cap > kMaxCap) cap = kMaxCap;
  L.cap = cap;
  size_t off = 0;
  L.cand = off;       off = round_up(off + n * (size_t)cap * sizeof(uint2));
  L.count = off;      off = round_up(off + n * sizeof(int));
  L.bin = off;        off = round_up(off + n * sizeof(int));
  L.lse = off;        off = round_up(off + (size_t)s.hq * n * sizeof(float));
  L.ovf_count = off;  off = round_up(off + sizeof(int));
  L.ovf_list = off;   off = round_up(off + n * sizeof(int));
  L.scratch = off;    off = round_up(off + (size_t)amtk::kFallbackSlots * L.units_max * sizeof(float));
  // the keys in MFMA operand order: pass 1's copy, which pass 2 also reads
  // with 8 KV heads and token units (the same layout)
  L.kops_bytes = std::max(amtk::pass1_key_operand_bytes(s),
                          amtk::pass2_key_operand_bytes(s, sp.key_block));
  L.kops = off;       off = round_up(off + L.kops_bytes);
  L.colsum = 0;
  L.total = off;
  return L;
}

CandidatePool pool_of(void* ws, const Layout& L) {
  unsigned char* b = static_cast<unsigned char*>(ws);
  CandidatePool p;
  p.cand = reinterpret_cast<uint2*>(b + L.cand);
  p.count = reinterpret_cast<int*>(b + L.count);
  p.bin = reinterpret_cast<int*>(b + L.bin);
  p.ovf_count = reinterpret_cast<int*>(b + L.ovf_count);
  p.ovf_list = reinterpret_cast<int*>(b + L.ovf_list);
  p.scratch = reinterpret_cast<float*>(b + L.scratch);
  p.kops = L.kops_bytes ? b + L.kops : nullptr;
  p.cap = L.cap;
  p.slots = amtk::kFallbackSlots;
  return p;
}

// Shared body of topk_support, topk_support_stage and indexer_topk
// (validated descriptors). stage 0 runs all three stages.
int run_topk(const LayerShape& s, const amtk_support_desc& sp, int stage, const void* q,
             const void* k, int32_t* idx, int32_t* count, float* mass, float* lse, void* ws,
             size_t ws_bytes, hipStream_t stream) {
  if (!amtk::pass_shape_supported(s)) return AMTK_E_UNSUPPORTED;
  if (sp.query_block != 1 && sp.key_block != 1 && (s.hq != 1 || s.hkv != 1))
    return AMTK_E_UNSUPPORTED;   // shared key blocks: the indexer's kernel only
  if (stage < 0 || stage > 3) return AMTK_E_INVALID;
  if (!q || !k || !ws || ((stage == 0 || stage == 3) && (!idx || !count))) return AMTK_E_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(idx, 4) || !aligned(count, 4) ||
      !aligned(ws, 256) || (mass && !aligned(mass, 4)) || (lse && !aligned(lse, 4)))
    return AMTK_E_INVALID;
  const Layout L = layout(s, sp);
  if (ws_bytes < L.total) return AMTK_E_WORKSPACE;
  float* lse_buf = lse ? lse : reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + L.lse);
  hipError_t e = hipSuccess;
  if (sp.query_block != 1 && sp.key_block != 1) {
    // key blocks shared by a selection block: the indexer's per-block kernel
    // (one head of d_idx, as indexer_topk passes it)
    if (s.hq != 1 || s.hkv != 1 ||
        !amtk::indexer_shared_supported(s.n, s.d, s.dtype, sp.key_block, sp.query_block, sp.k))
      return AMTK_E_UNSUPPORTED;
    int* zero = reinterpret_cast<int*>(static_cast<unsigned char*>(ws) + L.ovf_count);
    if (stage == 0 || stage == 1) e = amtk::launch_pass1_lse(s, q, k, lse_buf, zero, stream);
    if (e == hipSuccess && (stage == 0 || stage == 3))
      e = amtk::launch_indexer_shared(s.n, sp.key_block, sp.k, s.scale, q, k, lse_buf, idx, count,
                                      mass, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                      stream);
    return e == hipSuccess ? AMTK_OK : hip_fail(e);
  }
  if (sp.query_block != 1) {   // one support per selection block of consecutive queries
    float* colsum = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + L.colsum);
    int* zero = reinterpret_cast<int*>(static_cast<unsigned char*>(ws) + L.ovf_count);
    void* kops = L.kops_bytes ? static_cast<unsigned char*>(ws) + L.kops : nullptr;
    if (stage == 0 || stage == 1) e = amtk::launch_pass1_lse_kops(s, q, k, lse_buf, zero, kops, stream);
    if (e == hipSuccess && (stage == 0 || stage == 2))
      e = amtk::launch_pass2_colsum(s, q, k, lse_buf, colsum, stream);
    if (e == hipSuccess && (stage == 0 || stage == 3))
      e = amtk::launch_block_topk(s, sp.query_block, sp.k, colsum, idx, count, mass, stream);
    return e == hipSuccess ? AMTK_OK : hip_fail(e);
  }
  CandidatePool pool = pool_of(ws, L);
  // a whole call: pass 2 reads the keys pass 1 copied into operand order
  pool.kops_ready = stage == 0 && pool.kops && amtk::pass1_writes_kops(s) &&
                    amtk::pass2_key_operand_bytes(s, sp.key_block) != 0;
  if (stage == 0 || stage == 1) {
    e = amtk::launch_pass1_lse_kops(s, q, k, lse_buf, pool.ovf_count, pool.kops, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (stage == 0 || stage == 2) {
    e = amtk::launch_pass2_filter(s, sp.key_block, sp.k, q, k, lse_buf, pool, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (stage == 0 || stage == 3) {
    e = amtk::launch_select(s, sp.key_block, sp.k, q, k, lse_buf, pool, idx, count, mass, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return AMTK_OK;
}

int indexer_shape(int64_t n, int32_t d_idx, int32_t dtype, float scale, LayerShape* s) {
  amtk_attn_desc a;
  a.n = n;
  a.hq = 1;
  a.hkv = 1;
  a.d = d_idx;
  a.dtype = dtype;
  a.causal = 1;
  a.scale = scale;
  return check_attn(&a, s);
}

}  // namespace

namespace amtk {
int validate_attn(const amtk_attn_desc* a, LayerShape* s) { return check_attn(a, s); }
int record_hip_error(hipError_t e) { return hip_fail(e); }
}  // namespace amtk

#pragma GCC visibility push(default)
extern "C" {

int amtk_topk_workspace(const amtk_attn_desc* attn, const amtk_support_desc* sup, size_t* bytes) {
  LayerShape s;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if ((rc = check_support(sup))) return rc;
  if (!bytes) return AMTK_E_INVALID;
  if (!amtk::pass_shape_supported(s)) return AMTK_E_UNSUPPORTED;
  *bytes = layout(s, *sup).total;
  return AMTK_OK;
}

size_t amtk_workspace_bytes(const amtk_attn_desc* attn, const amtk_support_desc* sup) {
  size_t b = 0;
  return amtk_topk_workspace(attn, sup, &b) == AMTK_OK ? b : 0;
}

int topk_support(const amtk_attn_desc* attn, const amtk_support_desc* sup, const void* q,
                 const void* k, int32_t* idx, int32_t* count, float* mass, float* lse, void* ws,
                 size_t ws_bytes, void* stream) {
  LayerShape s;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if ((rc = check_support(sup))) return rc;
  return run_topk(s, *sup, 0, q, k, idx, count, mass, lse, ws, ws_bytes,
                  static_cast<hipStream_t>(stream));
}

int topk_support_stage(const amtk_attn_desc* attn, const amtk_support_desc* sup, int32_t stage,
                       const void* q, const void* k, int32_t* idx, int32_t* count, float* mass,
                       float* lse, void* ws, size_t ws_bytes, void* stream) {
  LayerShape s;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if ((rc = check_support(sup))) return rc;
  if (stage < 1 || stage > 3) return AMTK_E_INVALID;
  return run_topk(s, *sup, stage, q, k, idx, count, mass, lse, ws, ws_bytes,
                  static_cast<hipStream_t>(stream));
}

int sparse_attn(const amtk_attn_desc* attn, int32_t key_block, int32_t max_units, const void* q,
                const void* k, const void* v, const int32_t* idx, const int32_t* count, float* o,
                float* lse_sparse, void* stream) {
  LayerShape s;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if (max_units < 1) return AMTK_E_INVALID;
  if (key_block != 1 && key_block != 64) return AMTK_E_UNSUPPORTED;
  if (!amtk::sparse_shape_supported(s)) return AMTK_E_UNSUPPORTED;
  if (!q || !k || !v || !idx || !count || !o) return AMTK_E_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(idx, 4) ||
      !aligned(count, 4) || !aligned(o, 16) || (lse_sparse && !aligned(lse_sparse, 4)))
    return AMTK_E_INVALID;
  hipError_t e = amtk::launch_sparse_attn(s, key_block, max_units, q, k, v, idx, count, o,
                                          lse_sparse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return AMTK_OK;
}

int amtk_sparse_attn_workspace(const amtk_attn_desc* attn, size_t* bytes) {
  LayerShape s;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if (!bytes) return AMTK_E_INVALID;
  *bytes = amtk::sparse_windowed_scratch_bytes(s);
  return AMTK_OK;
}

int sparse_attn_windowed(const amtk_attn_desc* attn, int32_t key_block, int32_t max_units,
                         const void* q, const void* k, const void* v, const int32_t* idx,
                         const int32_t* count, float* o, float* lse_sparse, void* ws,
                         size_t ws_bytes, void* stream) {
  LayerShape s;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if (max_units < 1) return AMTK_E_INVALID;
  if (key_block != 1 && key_block != 64) return AMTK_E_UNSUPPORTED;
  if (!amtk::sparse_shape_supported(s)) return AMTK_E_UNSUPPORTED;
  if (!q || !k || !v || !idx || !count || !o || !ws) return AMTK_E_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(idx, 4) ||
      !aligned(count, 4) || !aligned(o, 16) || (lse_sparse && !aligned(lse_sparse, 4)) ||
      !aligned(ws, 256))
    return AMTK_E_INVALID;
  if (ws_bytes < amtk::sparse_windowed_scratch_bytes(s)) return AMTK_E_WORKSPACE;
  hipError_t e = amtk::launch_sparse_attn_windowed(s, key_block, max_units, q, k, v, idx, count, o,
                                                   lse_sparse, ws, ws_bytes,
                                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return AMTK_OK;
}

int sparse_attn_blocks(const amtk_attn_desc* attn, int32_t key_block, int32_t query_block,
                       int32_t max_units, const void* q, const void* k, const void* v,
                       const int32_t* idx, const int32_t* count, float* o, float* lse_sparse,
                       void* stream) {
  LayerShape s;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if (max_units < 1) return AMTK_E_INVALID;
  if (key_block != 1 && key_block != 64) return AMTK_E_UNSUPPORTED;
  if (query_block != kQueryBlock) return AMTK_E_UNSUPPORTED;
  // the block tile kernel where it covers the shape, else the per-row
  // gather with every row reading its block's first index row
  const bool tile = amtk::shared_attn_shape_supported(s, query_block);
  if (!tile && !amtk::sparse_shape_supported(s)) return AMTK_E_UNSUPPORTED;
  if (!q || !k || !v || !idx || !count || !o) return AMTK_E_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(idx, 4) ||
      !aligned(count, 4) || !aligned(o, 16) || (lse_sparse && !aligned(lse_sparse, 4)))
    return AMTK_E_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = tile ? amtk::launch_shared_attn(s, key_block, query_block, max_units, q, k, v, idx,
                                                 count, o, lse_sparse, st)
                      : amtk::launch_sparse_attn_block_rows(s, key_block, query_block, max_units, q,
                                                            k, v, idx, count, o, lse_sparse, st);
  if (e != hipSuccess) return hip_fail(e);
  return AMTK_OK;
}

int oracle_prefill(const amtk_attn_desc* attn, const amtk_support_desc* sup, const void* q,
                   const void* k, const void* v, float* o, int32_t* idx, int32_t* count,
                   float* mass, float* lse, void* ws, size_t ws_bytes, void* stream) {
  LayerShape s;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if ((rc = check_support(sup))) return rc;
  if (!amtk::sparse_shape_supported(s)) return AMTK_E_UNSUPPORTED;
  if (!v || !o) return AMTK_E_INVALID;
  if (!aligned(v, 16) || !aligned(o, 16)) return AMTK_E_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = run_topk(s, *sup, 0, q, k, idx, count, mass, lse, ws, ws_bytes, st);
  if (rc) return rc;
  // selection blocks: one gather per block where the tile kernel covers the
  // shape; every row also holds its block's support, so the per-row kernel
  // gives the same result elsewhere
  hipError_t e;
  if (sup->query_block != 1) {
    e = amtk::shared_attn_shape_supported(s, sup->query_block)
            ? amtk::launch_shared_attn(s, sup->key_block, sup->query_block, sup->k, q, k, v, idx,
                                       count, o, nullptr, st)
            : amtk::launch_sparse_attn(s, sup->key_block, sup->k, q, k, v, idx, count, o, nullptr, st);
  } else {
    // the candidate pool is free once the supports are selected: the
    // windowed gather's scratch (it falls back to one pass if too small)
    const Layout L = layout(s, *sup);
    e = amtk::launch_sparse_attn_windowed(s, sup->key_block, sup->k, q, k, v, idx, count, o,
                                          nullptr, static_cast<unsigned char*>(ws) + L.cand,
                                          L.count - L.cand, st);
  }
  if (e != hipSuccess) return hip_fail(e);
  return AMTK_OK;
}

int amtk_indexer_workspace(int64_t n, int32_t d_idx, int32_t dtype,
                           const amtk_support_desc* sup, size_t* bytes) {
  LayerShape s;
  int rc = indexer_shape(n, d_idx, dtype, 0.f, &s);
  if (rc) return rc;
  if ((rc = check_support(sup))) return rc;
  if (!bytes) return AMTK_E_INVALID;
  *bytes = layout(s, *sup).total;
  return AMTK_OK;
}

int indexer_topk(int64_t n, int32_t d_idx, int32_t dtype, float scale,
                 const amtk_support_desc* sup, const void* q_idx, const void* k_idx,
                 int32_t* idx, int32_t* count, float* mass, void* ws, size_t ws_bytes,
                 void* stream) {
  LayerShape s;
  int rc = indexer_shape(n, d_idx, dtype, scale, &s);
  if (rc) return rc;
  if ((rc = check_support(sup))) return rc;
  return run_topk(s, *sup, 0, q_idx, k_idx, idx, count, mass, nullptr, ws, ws_bytes,
                  static_cast<hipStream_t>(stream));
}

int captured_mass(int64_t n, int32_t hq, const float* lse_dense, const float* lse_support,
                  float* captured, void* stream) {
  if (n < 1 || n > INT32_MAX || hq < 1) return AMTK_E_INVALID;
  if (!lse_dense || !lse_support || !captured) return AMTK_E_INVALID;
  if (!aligned(lse_dense, 4) || !aligned(lse_support, 4) || !aligned(captured, 4))
    return AMTK_E_INVALID;
  hipError_t e = amtk::launch_captured_mass((int)n, hq, lse_dense, lse_support, captured,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return AMTK_OK;
}

int support_overlap(int64_t n, int32_t max_a, const int32_t* idx_a, const int32_t* count_a,
                    int32_t max_b, const int32_t* idx_b, const int32_t* count_b,
                    int32_t* overlap, void* stream) {
  if (n < 1 || n > INT32_MAX || max_a < 1 || max_b < 1) return AMTK_E_INVALID;
  if (!idx_a || !count_a || !idx_b || !count_b || !overlap) return AMTK_E_INVALID;
  if (!aligned(idx_a, 4) || !aligned(count_a, 4) || !aligned(idx_b, 4) || !aligned(count_b, 4) ||
      !aligned(overlap, 4))
    return AMTK_E_INVALID;
  hipError_t e = amtk::launch_support_overlap((int)n, max_a, idx_a, count_a, max_b, idx_b,
                                              count_b, overlap, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return AMTK_OK;
}

namespace {

struct KlLayout {
  size_t lse, lse_t, zero, part, kops, kops_bytes, total;
};

KlLayout kl_layout(const LayerShape& s) {
  KlLayout L;
  size_t off = 0;
  L.lse = off;    off = round_up(off + (size_t)s.hq * s.n * sizeof(float));
  L.lse_t = off;  off = round_up(off + (size_t)s.n * sizeof(float));
  L.zero = off;   off = round_up(off + sizeof(int));
  L.part = off;   off = round_up(off + amtk::kl_partial_bytes(s.n, s.hkv));
  // the teacher's LSE pass reads the keys from a copy in MFMA operand order
  // where it can
  L.kops_bytes = amtk::pass1_key_operand_bytes(s);
  L.kops = off;   off = round_up(off + L.kops_bytes);
  L.total = off;
  return L;
}

int kl_check(const amtk_attn_desc* attn, int32_t d_idx, LayerShape* s, LayerShape* si) {
  int rc = check_attn(attn, s);
  if (rc) return rc;
  if (d_idx < 1) return AMTK_E_INVALID;
  if (!amtk::kl_shape_supported(*s, d_idx)) return AMTK_E_UNSUPPORTED;
  *si = *s;
  si->hq = 1;
  si->hkv = 1;
  si->d = d_idx;
  return AMTK_OK;
}

}  // namespace

int amtk_kl_workspace(const amtk_attn_desc* attn, int32_t d_idx, size_t* bytes) {
  LayerShape s, si;
  int rc = kl_check(attn, d_idx, &s, &si);
  if (rc) return rc;
  if (!bytes) return AMTK_E_INVALID;
  *bytes = kl_layout(s).total;
  return AMTK_OK;
}

int kl_distill(const amtk_attn_desc* attn, int32_t d_idx, float idx_scale, const void* q,
               const void* k, const void* q_idx, const void* k_idx, float* kl_row, float* loss,
               float* dq_idx, float* dk_idx, void* ws, size_t ws_bytes, void* stream) {
  LayerShape s, si;
  int rc = kl_check(attn, d_idx, &s, &si);
  if (rc) return rc;
  if (std::isnan(idx_scale) || std::isinf(idx_scale)) return AMTK_E_INVALID;
  if (!q || !k || !q_idx || !k_idx || !kl_row || !dq_idx || !dk_idx || !ws) return AMTK_E_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_idx, 16) || !aligned(k_idx, 16) ||
      !aligned(kl_row, 4) || !aligned(dq_idx, 16) || !aligned(dk_idx, 16) || !aligned(ws, 256) ||
      (loss && !aligned(loss, 4)))
    return AMTK_E_INVALID;
  const KlLayout L = kl_layout(s);
  if (ws_bytes < L.total) return AMTK_E_WORKSPACE;
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* lse = reinterpret_cast<float*>(w + L.lse);
  float* lse_t = reinterpret_cast<float*>(w + L.lse_t);
  int* zero = reinterpret_cast<int*>(w + L.zero);
  si.scale = idx_scale > 0.f ? idx_scale : 1.0f / std::sqrt((float)d_idx);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* kops = L.kops_bytes ? w + L.kops : nullptr;
  hipError_t e = amtk::launch_pass1_lse_kops(s, q, k, lse, zero, kops, st);
  if (e == hipSuccess) e = amtk::launch_pass1_lse(si, q_idx, k_idx, lse_t, zero, st);
  if (e == hipSuccess)
    e = amtk::launch_kl_distill(s, d_idx, si.scale, q, k, q_idx, k_idx, lse, lse_t, kl_row, loss,
                                dq_idx, dk_idx, reinterpret_cast<float*>(w + L.part), st);
  if (e != hipSuccess) return hip_fail(e);
  return AMTK_OK;
}

int indexer_prefill(const amtk_attn_desc* attn, int32_t d_idx, float idx_scale,
                    const amtk_support_desc* sup, const void* q, const void* k, const void* v,
                    const void* q_idx, const void* k_idx, float* o, int32_t* idx, int32_t* count,
                    float* mass, void* ws, size_t ws_bytes, void* stream) {
  LayerShape s, si;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if ((rc = indexer_shape(s.n, d_idx, s.dtype, idx_scale, &si))) return rc;
  if ((rc = check_support(sup))) return rc;
  if (!amtk::sparse_shape_supported(s)) return AMTK_E_UNSUPPORTED;
  // both realisations read the backbone q, k, v and write o, idx, count
  if (!q || !k || !v || !o || !idx || !count) return AMTK_E_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return AMTK_E_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (sup->query_block == 1) {   // per-query realisation: indexer_topk, then sparse_attn
    rc = run_topk(si, *sup, 0, q_idx, k_idx, idx, count, mass, nullptr, ws, ws_bytes, st);
    if (rc) return rc;
    // the indexer's candidate pool is free now: the windowed gather's
    // scratch (one pass if it is too small)
    const Layout L = layout(si, *sup);
    hipError_t e = amtk::launch_sparse_attn_windowed(s, sup->key_block, sup->k, q, k, v, idx, count,
                                                     o, nullptr,
                                                     static_cast<unsigned char*>(ws) + L.cand,
                                                     L.count - L.cand, st);
    return e == hipSuccess ? AMTK_OK : hip_fail(e);
  }
  // fused realisation: the indexer's LSE pass, then one kernel per block of
  // queries that scores, selects and attends. Where that kernel does not
  // cover the shapes (token units, other backbone head layouts), the same
  // result in two steps: the block support (indexer_topk, written to
  // every row of the block), then the per-row gather.
  if (sup->key_block == 1 || !amtk::shared_attn_shape_supported(s, sup->query_block) ||
      !amtk::indexer_shared_supported(si.n, si.d, si.dtype, sup->key_block, sup->query_block, sup->k)) {
    rc = run_topk(si, *sup, 0, q_idx, k_idx, idx, count, mass, nullptr, ws, ws_bytes, st);
    if (rc) return rc;
    hipError_t e = amtk::launch_sparse_attn(s, sup->key_block, sup->k, q, k, v, idx, count, o,
                                            nullptr, st);
    return e == hipSuccess ? AMTK_OK : hip_fail(e);
  }
  if (!q_idx || !k_idx || !ws) return AMTK_E_INVALID;
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(idx, 4) || !aligned(count, 4) || !aligned(ws, 256) || (mass && !aligned(mass, 4)))
    return AMTK_E_INVALID;
  const Layout L = layout(si, *sup);
  if (ws_bytes < L.total) return AMTK_E_WORKSPACE;
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* lse_idx = reinterpret_cast<float*>(w + L.lse);
  hipError_t e = amtk::launch_pass1_lse(si, q_idx, k_idx, lse_idx,
                                        reinterpret_cast<int*>(w + L.ovf_count), st);
  if (e == hipSuccess)
    e = amtk::launch_indexer_shared(si.n, sup->key_block, sup->k, si.scale, q_idx, k_idx, lse_idx,
                                    idx, count, mass, &s, q, k, v, o, nullptr, st);
  return e == hipSuccess ? AMTK_OK : hip_fail(e);
}

const char* amtk_strerror(int code) {
  switch (code) {
    case AMTK_OK: return "success";
    case AMTK_E_INVALID: return "invalid argument (null pointer, size, alignment or inconsistent shapes)";
    case AMTK_E_UNSUPPORTED: return "unsupported configuration (dtype, head_dim, group size, budget, granularity or non-causal)";
    case AMTK_E_WORKSPACE: return "workspace too small";
    case AMTK_E_HIP: return "HIP launch failed (see amtk_last_hip_error)";
  }
  return "unknown error code";
}

int amtk_last_hip_error(void) { return g_last_hip; }

int amtk_pool_stats(const amtk_attn_desc* attn, const amtk_support_desc* sup, const void* ws,
                    size_t ws_bytes, int64_t* max_candidates, int64_t* overflow_rows,
                    int64_t* capacity, void* stream) {
  LayerShape s;
  int rc = check_attn(attn, &s);
  if (rc) return rc;
  if ((rc = check_support(sup))) return rc;
  if (!ws || !max_candidates || !overflow_rows || !capacity) return AMTK_E_INVALID;
  if (sup->query_block != 1) return AMTK_E_UNSUPPORTED;   // selection blocks keep no pools
  const Layout L = layout(s, *sup);
  if (ws_bytes < L.total) return AMTK_E_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<int> counts((size_t)s.n);
  int ovf = 0;
  const unsigned char* b = static_cast<const unsigned char*>(ws);
  hipError_t e = hipMemcpyAsync(counts.data(), b + L.count, counts.size() * sizeof(int),
                                hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(&ovf, b + L.ovf_count, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e);
  int64_t mx = 0;
  for (int c : counts) mx = c > mx ? c : mx;
  *max_candidates = mx;
  *overflow_rows = ovf;
  *capacity = L.cap;
  return AMTK_OK;
}

}  // extern "C"
#pragma GCC visibility pop
