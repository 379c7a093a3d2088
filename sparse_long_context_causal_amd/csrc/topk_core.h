// Workgroup top-k over a row of non-negative fp32 scores, ranked by (score
// descending, id ascending): a 4-pass 8-bit radix select on the score bit
// patterns (non-negative floats order like their bits) finds the k-th
// largest and how many of its equals to keep, then one ordered pass with
// ballot prefix sums emits the winners in id order. Used for the shared
// support of a selection block (oracle and indexer).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace amtk {

// LDS scratch of wg_topk for a workgroup of kThreads threads.
template <int kThreads>
struct TopkScratch {
  unsigned hist[256];
  int scal[2];
  int wsum[2][kThreads / 64];
};

// score(j) for j in [0, nk) must return the same value at every call. The
// winners land in win_id[0 .. kk) (ascending) and win_m (their scores);
// returns kk = min(k, nk). Every thread of the workgroup must call it.
template <int kThreads, class F>
__device__ __forceinline__ int wg_topk(F score, int nk, int k, TopkScratch<kThreads>& sc,
                                       int* win_id, float* win_m) {
  constexpr int kWaves = kThreads / 64;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const unsigned long long below = (1ull << l) - 1ull;
  const bool all = nk <= k;
  unsigned thr = 0u;
  int take = 0;
  if (!all) {
    unsigned prefix = 0u, pmask = 0u;
    int rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += kThreads) sc.hist[b] = 0u;
      __syncthreads();
      for (int j = tid; j < nk; j += kThreads) {
        const unsigned v = __float_as_uint(score(j));
        if ((v & pmask) == prefix) atomicAdd(&sc.hist[(v >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0, d = 255;
        for (; d > 0; --d) {
          if (acc + (int)sc.hist[d] >= rem) break;
          acc += (int)sc.hist[d];
        }
        sc.scal[0] = d;
        sc.scal[1] = rem - acc;
      }
      __syncthreads();
      prefix |= (unsigned)sc.scal[0] << shift;
      pmask |= 255u << shift;
      rem = sc.scal[1];
      __syncthreads();
    }
    thr = prefix;
    take = rem;
  }
  // ordered emission: scores above thr, and the first `take` equal to it
  int base = 0, eq_seen = 0;
  for (int j0 = 0; j0 < nk; j0 += kThreads) {
    const int j = j0 + tid;
    float m = 0.f;
    bool gt = false, eq = false;
    if (j < nk) {
      m = score(j);
      const unsigned v = __float_as_uint(m);
      gt = all || v > thr;
      eq = !all && v == thr;
    }
    const unsigned long long be = __ballot(eq);
    if (l == 0) sc.wsum[0][w] = __popcll(be);
    __syncthreads();
    int eq_before = eq_seen + __popcll(be & below);
    for (int ww = 0; ww < w; ++ww) eq_before += sc.wsum[0][ww];
    const bool keep = gt || (eq && eq_before < take);
    const unsigned long long bk = __ballot(keep);
    if (l == 0) sc.wsum[1][w] = __popcll(bk);
    __syncthreads();
    int pos = base + __popcll(bk & below);
    for (int ww = 0; ww < w; ++ww) pos += sc.wsum[1][ww];
    if (keep && pos < k) {   // (pos < k always holds: at most k scores are kept)
      win_id[pos] = j;
      win_m[pos] = m;
    }
    for (int ww = 0; ww < kWaves; ++ww) {
      eq_seen += sc.wsum[0][ww];
      base += sc.wsum[1][ww];
    }
    __syncthreads();
  }
  return base;   // = min(k, nk)
}

}  // namespace amtk
