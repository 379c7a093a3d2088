// Exact per-row top-k selection (units ranked by mass descending, then by
// unit id ascending), output sorted by unit id.
//
// Method: gist.science page on arXiv 2606.07703, "Technischer Bericht"
// section 2.1: the support is the top-k units of the head-averaged mass
// under budget k. Rows with at most k visible units keep all of them; equal
// masses go to the smaller unit id (a fixed, deterministic order).
//
// Two kernels:
//   * select_pool_kernel: one workgroup per row picks the top-k from the
//     row's candidate pool (pass 2 output). It first keeps the entries at or
//     above the row's final bound bin (a superset of the top-k, since every
//     top-k unit lies in a bin >= the final bound) and copies them to LDS
//     with wave-ballot compaction. A radix select on the fp32 mass bits then
//     runs in LDS, starting at the highest bit where the kept values differ
//     (8-bit digits, LDS histograms); an exact-value tie at the boundary is
//     broken by a second radix select on the unit id. The winners are
//     compacted and bitonic-sorted by id in LDS. Rows with more survivors
//     than the LDS holds select straight from the pool in global memory.
//   * dense_row_kernel: rows whose pool overflowed are recomputed from Q/K
//     and pass 1's LSE into a dense per-row mass array (one row per
//     workgroup, persistent over the overflow list), then selected the same
//     way. It is exact for any input, including massive ties.
#include "device_common.h"
#include "kernels.h"

namespace amtk {

constexpr int kSelThreads = 256;
constexpr int kSelLds = 4096;   // candidates held in LDS by the fast path

struct SelectSmem {
  unsigned hist[256];
  int scal[8];
  // fast path: [0] kept masses, [1] kept ids, [2] winner ids, [3] winner masses;
  // global path: winner ids in [0..1] and masses in [2..3] (kMaxBudget each)
  unsigned buf[4][kSelLds];
};
static_assert(2 * kSelLds >= kMaxBudget, "winner buffers must hold the largest budget");

// Pool entries: (mass bits, unit id) pairs.
struct PoolView {
  const uint2* p;
  __device__ __forceinline__ unsigned val(int t) const { return p[t].x; }
  __device__ __forceinline__ unsigned id(int t) const { return p[t].y; }
};
// Dense rows: mass of unit t at position t.
struct DenseView {
  const float* p;
  __device__ __forceinline__ unsigned val(int t) const { return __float_as_uint(p[t]); }
  __device__ __forceinline__ unsigned id(int t) const { return (unsigned)t; }
};
// Candidates staged in LDS.
struct LdsView {
  const unsigned* v;
  const unsigned* i;
  __device__ __forceinline__ unsigned val(int t) const { return v[t]; }
  __device__ __forceinline__ unsigned id(int t) const { return i[t]; }
};

// Finds, among elements with pred(t), the `need`-th largest of key(t) (a
// 32-bit unsigned key), by 8-bit radix rounds from the top. Returns the key
// value; *above is the number of such elements with a strictly larger key
// and *equal the number with exactly that key. All threads return the same.
// Digits are 8 bits from bit position top_shift down to 0; bits above
// top_shift + 8 must be common to all keys (they are taken from `common`).
template <class KeyFn, class PredFn>
__device__ unsigned radix_kth_largest(int nc, int need, KeyFn key, PredFn pred, SelectSmem& sm,
                                      int* above, int* equal, int top_shift = 24,
                                      unsigned common = 0u) {
  const int tid = threadIdx.x;
  unsigned pmask = top_shift + 8 >= 32 ? 0u : ~((1u << (top_shift + 8)) - 1u);
  unsigned prefix = common & pmask;
  int higher = 0;
  int eq = 0;
  for (int shift = top_shift; shift >= 0; shift -= 8) {
    sm.hist[tid] = 0u;
    __syncthreads();
    for (int t = tid; t < nc; t += kSelThreads) {
      if (!pred(t)) continue;
      const unsigned v = key(t);
      if ((v & pmask) == prefix) atomicAdd(&sm.hist[(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane L holds bins 4L..4L+3; suffix sums over lanes find the digit
      const unsigned h0 = sm.hist[4 * tid], h1 = sm.hist[4 * tid + 1];
      const unsigned h2 = sm.hist[4 * tid + 2], h3 = sm.hist[4 * tid + 3];
      const int lsum = (int)(h0 + h1 + h2 + h3);
      int incl = lsum;   // sum over lanes >= tid
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(incl, off, 64);
        if (tid + off < 64) incl += o;
      }
      const int excl = incl - lsum;   // sum over lanes > tid
      const int want = need - higher;
      if (excl < want && incl >= want) {
        // digit lies in this lane's 4 bins, scanned from the top
        int acc = excl;
        int d = 4 * tid + 3;
        const unsigned hv[4] = {h0, h1, h2, h3};
        for (int b = 3; b >= 0; --b) {
          if (acc + (int)hv[b] >= want) {
            d = 4 * tid + b;
            break;
          }
          acc += (int)hv[b];
        }
        sm.scal[0] = d;
        sm.scal[1] = acc;              // count in bins above d (this round)
        sm.scal[2] = (int)hv[d - 4 * tid];
      }
    }
    __syncthreads();
    const int d = sm.scal[0];
    higher += sm.scal[1];
    eq = sm.scal[2];
    prefix |= (unsigned)d << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  *above = higher;
  *equal = eq;
  return prefix;
}

// Selects the k_eff best of nc elements of view `v` and writes the row's
// outputs: out_idx[0..kout) ascending ids then -1, out_mass likewise (0 pad),
// *out_count = k_eff. Requires nc >= k_eff (every unit of the top-k present).
template <class View>
__device__ void select_row(View v, int nc, int k_eff, int kout, int32_t* out_idx,
                           float* out_mass, int32_t* out_count, SelectSmem& sm, unsigned* wkey,
                           unsigned* wval, int top_shift = 24, unsigned common = 0u) {
  const int tid = threadIdx.x;
  unsigned vstar = 0u, istar = 0xffffffffu;
  bool take_all = nc <= k_eff;
  bool all_ties = true;
  if (!take_all) {
    int above = 0, equal = 0;
    vstar = radix_kth_largest(
        nc, k_eff, [&](int t) { return v.val(t); }, [&](int) { return true; }, sm, &above,
        &equal, top_shift, common);
    const int need_eq = k_eff - above;
    if (need_eq < equal) {
      // exact-value tie at the boundary: the smallest ids win
      all_ties = false;
      int a2 = 0, e2 = 0;
      istar = ~radix_kth_largest(
          nc, need_eq, [&](int t) { return ~v.id(t); },
          [&](int t) { return v.val(t) == vstar; }, sm, &a2, &e2);
    }
  }
  if (tid == 0) sm.scal[3] = 0;
  __syncthreads();
  for (int t = tid; t < nc; t += kSelThreads) {
    const unsigned x = v.val(t);
    const unsigned id = v.id(t);
    const bool sel = take_all || x > vstar || (x == vstar && (all_ties || id <= istar));
    if (sel) {
      const int p = atomicAdd(&sm.scal[3], 1);
      if (p < kMaxBudget) {
        wkey[p] = id;
        wval[p] = x;
      }
    }
  }
  __syncthreads();
  const int got = min(sm.scal[3], k_eff);
  int S = 1;
  while (S < got) S <<= 1;
  for (int t = got + tid; t < S; t += kSelThreads) {
    wkey[t] = 0xffffffffu;
    wval[t] = 0u;
  }
  __syncthreads();
  for (int size = 2; size <= S; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (S >> 1); t += kSelThreads) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned a = wkey[lo], b = wkey[hi];
        if ((a > b) == up) {
          wkey[lo] = b;
          wkey[hi] = a;
          const unsigned va = wval[lo];
          wval[lo] = wval[hi];
          wval[hi] = va;
        }
      }
      __syncthreads();
    }
  }
  for (int t = tid; t < kout; t += kSelThreads) {
    out_idx[t] = t < got ? (int32_t)wkey[t] : -1;
    if (out_mass) out_mass[t] = t < got ? __uint_as_float(wval[t]) : 0.f;
  }
  if (tid == 0) *out_count = got;
  __syncthreads();
}

__device__ __forceinline__ int visible_units(int i, int key_block) {
  return key_block == 1 ? i + 1 : i / key_block + 1;
}

__global__ __launch_bounds__(kSelThreads) void select_pool_kernel(
    const uint2* __restrict__ cand, const int* __restrict__ cand_count,
    const int* __restrict__ row_bin, int n, int cap, int key_block, int budget,
    int32_t* __restrict__ idx, int32_t* __restrict__ count, float* __restrict__ mass) {
  __shared__ SelectSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = n - 1 - (int)blockIdx.x;
  const int nc = cand_count[i];
  if (nc > cap) return;   // overflowed: dense_row_kernel owns this row
  const int k_eff = min(budget, visible_units(i, key_block));
  const uint2* pool = cand + (size_t)i * cap;
  int32_t* out_idx = idx + (size_t)i * budget;
  float* out_mass = mass ? mass + (size_t)i * budget : nullptr;

  // keep the entries at or above the row's final bound bin, staged in LDS
  const unsigned floor_bits = filter_bin_floor_bits(row_bin[i]);
  if (tid == 0) {
    sm.scal[4] = 0;
    sm.scal[5] = 0;            // OR of kept masses
    sm.scal[6] = ~0;           // AND of kept masses
  }
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  unsigned vor = 0u, vand = ~0u;
  for (int b0 = 0; b0 < nc; b0 += kSelThreads) {
    const int t = b0 + tid;
    uint2 e = make_uint2(0u, 0u);
    if (t < nc) e = pool[t];
    const bool keep = t < nc && e.x >= floor_bits;
    const unsigned long long m = __ballot(keep);
    int off = 0;
    if (lane == 0 && m) off = atomicAdd(&sm.scal[4], __popcll(m));
    off = __shfl(off, 0, 64);
    if (keep) {
      const int pos = off + __popcll(m & below);
      if (pos < kSelLds) {
        sm.buf[0][pos] = e.x;
        sm.buf[1][pos] = e.y;
      }
      vor |= e.x;
      vand &= e.x;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    vor |= __shfl_xor(vor, o, 64);
    vand &= __shfl_xor(vand, o, 64);
  }
  if (lane == 0) {
    atomicOr(reinterpret_cast<unsigned*>(&sm.scal[5]), vor);
    atomicAnd(reinterpret_cast<unsigned*>(&sm.scal[6]), vand);
  }
  __syncthreads();
  const int kept = sm.scal[4];
  const unsigned diff = (unsigned)sm.scal[5] ^ (unsigned)sm.scal[6];
  const unsigned common = (unsigned)sm.scal[6];
  (void)wave;
  if (kept <= kSelLds && k_eff <= kSelLds) {
    const int hb = diff ? 31 - __clz(diff) : 0;   // highest differing bit
    select_row(LdsView{sm.buf[0], sm.buf[1]}, kept, k_eff, budget, out_idx, out_mass,
               count + i, sm, sm.buf[2], sm.buf[3], 8 * (hb / 8), common);
  } else {
    __syncthreads();
    select_row(PoolView{pool}, nc, k_eff, budget, out_idx, out_mass, count + i, sm, &sm.buf[0][0],
               &sm.buf[2][0]);
  }
}

// Dense per-row mass for overflow rows: P(u) = sum over the unit's keys of
// (1/Hq) sum_h exp(s_h(i,j) - LSE_h(i)), with the same exp2 formulation as
// pass 2. Q row in LDS (fp32), K streamed per thread.
template <typename T, int D, int G>
__global__ __launch_bounds__(kSelThreads) void dense_row_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ lse, int n,
    int hkv, float c, float inv_hq, int key_block, int budget, const int* __restrict__ ovf_count,
    const int* __restrict__ ovf_list, float* __restrict__ scratch, int units_max,
    int32_t* __restrict__ idx, int32_t* __restrict__ count, float* __restrict__ mass) {
  __shared__ SelectSmem sm;
  __shared__ float qs[kMaxQRow];
  __shared__ float bias[kMaxQRow / 64];
  const int hq = hkv * G;
  const int total = *ovf_count;
  float* P = scratch + (size_t)blockIdx.x * units_max;
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int i = ovf_list[t];
    for (int e = threadIdx.x; e < hq * D; e += kSelThreads)
      qs[e] = load_elem(Q + (size_t)i * hq * D + e);
    for (int h = threadIdx.x; h < hq; h += kSelThreads) bias[h] = lse[(size_t)h * n + i] * kLog2e;
    __syncthreads();
    const int units = visible_units(i, key_block);
    for (int u = threadIdx.x; u < units; u += kSelThreads) {
      const int j0 = u * key_block;
      const int j1 = min(j0 + key_block, i + 1);
      float m = 0.f;
      for (int j = j0; j < j1; ++j) {
        float ph = 0.f;
        for (int g = 0; g < hkv; ++g) {
          const T* kr = K + ((size_t)j * hkv + g) * D;
          float s[G];
#pragma unroll
          for (int h = 0; h < G; ++h) s[h] = 0.f;
          for (int e = 0; e < D; ++e) {
            const float kv = load_elem(kr + e);
#pragma unroll
            for (int h = 0; h < G; ++h) s[h] = fmaf(qs[(g * G + h) * D + e], kv, s[h]);
          }
#pragma unroll
          for (int h = 0; h < G; ++h) ph += fast_exp2(fmaf(s[h], c, -bias[g * G + h]));
        }
        m += ph * inv_hq;
      }
      P[u] = m;
    }
    __syncthreads();
    const int k_eff = min(budget, units);
    select_row(DenseView{P}, units, k_eff, budget, idx + (size_t)i * budget,
               mass ? mass + (size_t)i * budget : nullptr, count + i, sm, &sm.buf[0][0],
               &sm.buf[2][0]);
  }
}

template <typename T, int D, int G>
static hipError_t run_dense(const LayerShape& s, int key_block, int budget, const void* q,
                            const void* k, const float* lse, const CandidatePool& pool,
                            int units_max, int32_t* idx, int32_t* count, float* mass,
                            hipStream_t stream) {
  hipLaunchKernelGGL((dense_row_kernel<T, D, G>), dim3(pool.slots), dim3(kSelThreads), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), lse, s.n, s.hkv,
                     s.scale * kLog2e, 1.0f / (float)s.hq, key_block, budget, pool.ovf_count,
                     pool.ovf_list, pool.scratch, units_max, idx, count, mass);
  return hipGetLastError();
}

hipError_t launch_select(const LayerShape& s, int key_block, int budget, const void* q,
                         const void* k, const float* lse, const CandidatePool& pool, int32_t* idx,
                         int32_t* count, float* mass, hipStream_t stream) {
  hipLaunchKernelGGL(select_pool_kernel, dim3(s.n), dim3(kSelThreads), 0, stream, pool.cand,
                     pool.count, pool.bin, s.n, pool.cap, key_block, budget, idx, count, mass);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int units_max = key_block == 1 ? s.n : (s.n - 1) / key_block + 1;
  const int G = s.hq / s.hkv;
#define AMTK_DENSE(T_, D_, G_) \
  if (G == G_) return run_dense<T_, D_, G_>(s, key_block, budget, q, k, lse, pool, units_max, idx, count, mass, stream)
  if (s.dtype == kBF16) {
    if (s.d == 64) { AMTK_DENSE(bf16_t, 64, 1); AMTK_DENSE(bf16_t, 64, 2); AMTK_DENSE(bf16_t, 64, 4); AMTK_DENSE(bf16_t, 64, 8); }
    else { AMTK_DENSE(bf16_t, 128, 1); AMTK_DENSE(bf16_t, 128, 2); AMTK_DENSE(bf16_t, 128, 4); }
  } else {
    if (s.d == 64) { AMTK_DENSE(float, 64, 1); AMTK_DENSE(float, 64, 2); AMTK_DENSE(float, 64, 4); }
    else { AMTK_DENSE(float, 128, 1); AMTK_DENSE(float, 128, 2); }
  }
#undef AMTK_DENSE
  return hipErrorInvalidValue;
}

}  // namespace amtk
