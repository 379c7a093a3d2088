// Support diagnostics: how much of the dense attention mass a support keeps,
// and how many ids two supports share.
//
// Method: gist.science page on arXiv 2606.07703, "Technischer Bericht"
// section 2.3 separates the loss of a sparse layer into the oracle gap (the
// oracle's own support against dense attention), the indexer gap (a
// distilled indexer's support in place of the oracle's) and the realization
// gap (runtime constraints such as selection-block sharing). At the level of
// one layer their synthetic analogues are the head-averaged mass a support
// captures, sum_{j in S_i} P_i(j), and the overlap of two supports.
//
// captured: sum_{j in S} p_h(j) = sum_{j in S} exp(s_h(j) - LSE_h)
//         = exp(LSE^S_h - LSE_h), so the captured head-averaged mass follows
// from the dense per-head LSE (pass 1) and the support LSE that the sparse
// kernels return, with no further pass over the keys.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace amtk {

namespace {

__global__ __launch_bounds__(256) void captured_mass_kernel(const float* __restrict__ lse_dense,
                                                            const float* __restrict__ lse_support,
                                                            int n, int hq,
                                                            float* __restrict__ captured) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= n) return;
  float acc = 0.f;
  for (int h = 0; h < hq; ++h) {
    const float ls = lse_support[(size_t)h * n + i];
    if (ls == -INFINITY) continue;   // empty support: nothing captured
    acc += expf(ls - lse_dense[(size_t)h * n + i]);
  }
  captured[i] = acc / (float)hq;
}

// One wave per row: the lanes take the ids of support b 64 at a time and
// look each up in support a (ascending) by binary search; the hits are
// counted with a ballot.
__global__ __launch_bounds__(256) void support_overlap_kernel(
    const int32_t* __restrict__ idx_a, const int32_t* __restrict__ count_a, int max_a,
    const int32_t* __restrict__ idx_b, const int32_t* __restrict__ count_b, int max_b, int n,
    int32_t* __restrict__ overlap) {
  const int i = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const int ca = min(max(count_a[i], 0), max_a), cb = min(max(count_b[i], 0), max_b);
  const int32_t* a = idx_a + (size_t)i * max_a;
  const int32_t* b = idx_b + (size_t)i * max_b;
  int hits = 0;
  for (int p0 = 0; p0 < cb; p0 += 64) {
    bool hit = false;
    if (p0 + lane < cb) {
      const int x = b[p0 + lane];
      int lo = 0, hi = ca;   // first position with a[pos] >= x
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1;
        else hi = mid;
      }
      hit = x >= 0 && lo < ca && a[lo] == x;
    }
    hits += __popcll(__ballot(hit));
  }
  if (lane == 0) overlap[i] = hits;
}

}  // namespace

hipError_t launch_captured_mass(int n, int hq, const float* lse_dense, const float* lse_support,
                                float* captured, hipStream_t stream) {
  hipLaunchKernelGGL(captured_mass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     lse_dense, lse_support, n, hq, captured);
  return hipGetLastError();
}

hipError_t launch_support_overlap(int n, int max_a, const int32_t* idx_a, const int32_t* count_a,
                                  int max_b, const int32_t* idx_b, const int32_t* count_b,
                                  int32_t* overlap, hipStream_t stream) {
  hipLaunchKernelGGL(support_overlap_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream,
                     idx_a, count_a, max_a, idx_b, count_b, max_b, n, overlap);
  return hipGetLastError();
}

}  // namespace amtk
