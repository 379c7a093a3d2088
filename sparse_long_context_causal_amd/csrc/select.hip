// Exact per-row top-k selection (units ranked by mass descending, then by
// unit id ascending), output sorted by unit id.
//
// Method: gist.science page on arXiv 2606.07703, "Technischer Bericht"
// section 2.1: the support is the top-k units of the head-averaged mass
// under budget k. Rows with at most k visible units keep all of them; equal
// masses go to the smaller unit id (a fixed, deterministic order).
//
// Two kernels:
//   * select_wave_kernel: one wave per row picks the top-k from the row's
//     candidate pool (pass 2 output), which pass 2 appends in increasing unit
//     id; the selection keeps that order, so ids come out ascending without
//     a sort (details at the kernel).
//   * dense_row_kernel: rows whose pool overflowed are recomputed from Q/K
//     and pass 1's LSE into a dense per-row mass array (one row per
//     workgroup, persistent over the overflow list), then selected by a
//     workgroup radix select and a bitonic sort by id. It is exact for any
//     input, including massive ties.
#include "device_common.h"
#include "kernels.h"

namespace amtk {

constexpr int kSelThreads = 256;
constexpr int kSelLds = 4096;

struct SelectSmem {
  unsigned hist[256];
  int scal[8];
  // winner ids in buf[0..1] and masses in buf[2..3] (kMaxBudget each)
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

// One wave per row. Pass 2 appends each row's pool in increasing unit id,
// and every step below keeps that order, so the output needs no sort.
//   1. Stream the pool once and keep the entries at or above the floor of
//      the row's final bound bin (every top-k unit is among them, and so is
//      every unit of equal mass), staged in LDS in pool order with
//      order-preserving ballot compaction.
//   2. Find the k-th largest mass bit pattern v* exactly: with the kept
//      masses in registers, fix its bits from the highest one where the kept
//      masses differ downwards, keeping a bit when at least k kept masses are
//      >= the prefix with that bit set (a popcount of ballots per step).
//   3. Walk the kept entries in order and emit those above v*, plus the first
//      (k - #above) entries equal to v*: equal masses go to the smaller ids.
// Rows that keep more than the LDS holds run step 2 as an 8-bit radix select
// over the pool in global memory (LDS histogram) and step 3 over the pool.
template <int R>
__global__ __launch_bounds__(64) void select_wave_kernel(
    const uint2* __restrict__ cand, const int* __restrict__ cand_count,
    const int* __restrict__ row_bin, int n, int cap, int key_block, int budget,
    int32_t* __restrict__ idx, int32_t* __restrict__ count, float* __restrict__ mass) {
  constexpr int kCap = 64 * R;   // kept entries the LDS holds
  constexpr int U = 32;          // pool loads in flight per lane (the loop is latency bound)
  __shared__ unsigned sv[kCap];
  __shared__ unsigned si[kCap];
  const int lane = threadIdx.x;
  const int i = n - 1 - (int)blockIdx.x;
  const int nc = cand_count[i];
  if (nc > cap) return;   // overflowed: dense_row_kernel owns this row
  const int k_eff = min(budget, visible_units(i, key_block));
  const uint2* pool = cand + (size_t)i * cap;
  int32_t* out_idx = idx + (size_t)i * budget;
  float* out_mass = mass ? mass + (size_t)i * budget : nullptr;
  const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const unsigned floor_bits = filter_bin_floor_bits(row_bin[i]);

  // ---- 1. keep and stage
  int kept = 0;
  unsigned vor = 0u, vand = ~0u;
  for (int b0 = 0; b0 < nc; b0 += 64 * U) {
    uint2 e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = b0 + 64 * u + lane;
      e[u] = t < nc ? pool[t] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool keep = b0 + 64 * u + lane < nc && e[u].x >= floor_bits;
      const unsigned long long m = __ballot(keep);
      if (keep) {
        const int pos = kept + __popcll(m & below);
        if (pos < kCap) {
          sv[pos] = e[u].x;
          si[pos] = e[u].y;
        }
        vor |= e[u].x;
        vand &= e[u].x;
      }
      kept += __popcll(m);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    vor |= __shfl_xor(vor, o, 64);
    vand &= __shfl_xor(vand, o, 64);
  }
  const unsigned diff = vor ^ vand;
  const int hb = diff ? 31 - __clz(diff) : -1;   // highest bit where kept masses differ
  __syncthreads();

  int out = 0, eq_seen = 0;
  // emits entry (x, id) of a 64-entry group in order; valid marks real entries
  auto emit = [&](bool valid, unsigned x, unsigned id, unsigned vstar, int need_eq) {
    const unsigned long long em = __ballot(valid && x == vstar);
    const bool sel = valid && (x > vstar || (x == vstar && eq_seen + __popcll(em & below) < need_eq));
    const unsigned long long sm = __ballot(sel);
    if (sel) {
      const int p = out + __popcll(sm & below);
      out_idx[p] = (int32_t)id;
      if (out_mass) out_mass[p] = __uint_as_float(x);
    }
    out += __popcll(sm);
    eq_seen += __popcll(em);
  };

  if (kept <= kCap) {
    // ---- 2. exact k-th largest over the kept masses held in registers
    unsigned v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int t = 64 * r + lane;
      v[r] = t < kept ? sv[t] : 0u;
    }
    // number of kept masses >= x, for x > 0 (padding holds 0)
    auto count_ge = [&](unsigned x) {
      int c = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (64 * r >= kept) break;
        c += __popcll(__ballot(v[r] >= x));
      }
      return c;
    };
    unsigned vstar = 0u;
    int need_eq = kept;   // keep everything when kept == k_eff
    if (kept > k_eff) {
      vstar = vand;
      if (hb >= 0) {
        vstar = hb == 31 ? 0u : (vand & ~((2u << hb) - 1u));
        for (int b = hb; b >= 0; --b) {
          const unsigned t = vstar | (1u << b);
          if (count_ge(t) >= k_eff) vstar = t;
        }
      }
      need_eq = k_eff - count_ge(vstar + 1u);
    }
    // ---- 3. emit in order
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (64 * r >= kept) break;
      const int t = 64 * r + lane;
      emit(t < kept, v[r], t < kept ? si[t] : 0u, vstar, need_eq);
    }
  } else {
    // ---- 2'. radix select over the pool in global memory
    unsigned* hist = sv;   // 256 bins
    const int top_shift = 8 * (hb / 8);
    unsigned pmask = top_shift + 8 >= 32 ? 0u : ~((1u << (top_shift + 8)) - 1u);
    unsigned prefix = vand & pmask;
    int higher = 0;
    for (int shift = top_shift; shift >= 0; shift -= 8) {
      for (int b = lane; b < 256; b += 64) hist[b] = 0u;
      __syncthreads();
      for (int b0 = 0; b0 < nc; b0 += 64 * U) {
        unsigned x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int t = b0 + 64 * u + lane;
          x[u] = t < nc ? pool[t].x : 0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (b0 + 64 * u + lane < nc && (x[u] & pmask) == prefix)
            atomicAdd(&hist[(x[u] >> shift) & 255u], 1u);
      }
      __syncthreads();
      // lane L holds bins 4L..4L+3; a suffix sum over lanes finds the digit
      const unsigned h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
      const unsigned h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      const int lsum = (int)(h0 + h1 + h2 + h3);
      int incl = lsum;   // bins of lanes >= this one
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += o;
      }
      const int excl = incl - lsum;
      const int want = k_eff - higher;
      const bool hit = excl < want && incl >= want;
      int d = 4 * lane, acc = excl;
      if (hit) {
        const unsigned hv[4] = {h0, h1, h2, h3};
        for (int b = 3; b >= 0; --b) {
          if (acc + (int)hv[b] >= want) {
            d = 4 * lane + b;
            break;
          }
          acc += (int)hv[b];
        }
      }
      const int src = __ffsll((long long)__ballot(hit)) - 1;
      d = __shfl(d, src, 64);
      acc = __shfl(acc, src, 64);
      higher += acc;
      prefix |= (unsigned)d << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    const unsigned vstar = prefix;
    const int need_eq = k_eff - higher;
    // ---- 3'. emit in pool order
    for (int b0 = 0; b0 < nc && out < k_eff; b0 += 64 * U) {
      uint2 e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = b0 + 64 * u + lane;
        e[u] = t < nc ? pool[t] : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) emit(b0 + 64 * u + lane < nc, e[u].x, e[u].y, vstar, need_eq);
    }
  }
  for (int t = k_eff + lane; t < budget; t += 64) {
    out_idx[t] = -1;
    if (out_mass) out_mass[t] = 0.f;
  }
  if (lane == 0) count[i] = k_eff;
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
  // LDS rows per lane: room for about 2.5k kept entries (the top k plus the
  // rest of the boundary bin); rows keeping more take the global-memory path.
  auto kern = 5 * budget <= 2 * 1024   ? select_wave_kernel<16>
              : 5 * budget <= 2 * 2048 ? select_wave_kernel<32>
                                       : select_wave_kernel<64>;
  hipLaunchKernelGGL(kern, dim3(s.n), dim3(64), 0, stream, pool.cand, pool.count, pool.bin, s.n,
                     pool.cap, key_block, budget, idx, count, mass);
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
