// Shared support of a selection block of consecutive query rows.
//
// Method: gist.science page on arXiv 2606.07703, "Technischer Bericht"
// section 2.1: with selection-block-shared granularity (b_sel = 64) one
// support set is chosen for a block of consecutive queries. The block scores
// key j by the mean over its rows of the head-averaged mass P_i(j), a key
// after row i counting 0 for that row; the top-k keys by (score descending,
// id ascending) among the keys its last row sees are written, ascending,
// into the index row of every query of the block. Each query then attends
// over the shared keys j <= i (the sparse-attention contract skips keys
// after the row).
//
// Input: pass 2's column sums over its 32-row tiles, colsum[t][j] = the sum
// of P_i(j) over tile t's rows (written for keys j up to the tile's last
// row). One workgroup per selection block forms the score row on the fly
// from the block's tiles, finds the bit pattern of the k-th largest score
// with a 4-pass radix select (scores are >= 0, so bit order is value order),
// and emits the winners in id order in one ordered pass.
#include "device_common.h"
#include "kernels.h"

namespace amtk {

constexpr int kBsThreads = 256;
constexpr int kBsWaves = kBsThreads / 64;

__global__ __launch_bounds__(kBsThreads) void block_topk_kernel(
    const float* __restrict__ colsum, int n, int bsel, int k, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, float* __restrict__ mass) {
  __shared__ unsigned hist[256];
  __shared__ int scal[2];
  __shared__ int wsum[2][kBsWaves];
  extern __shared__ __align__(16) unsigned char dyn[];   // winners: ids [k], scores [k]
  int* win_id = reinterpret_cast<int*>(dyn);
  float* win_m = reinterpret_cast<float*>(dyn + (size_t)k * sizeof(int));

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const unsigned long long below = (1ull << l) - 1ull;
  const int i0 = (int)blockIdx.x * bsel, i1 = min(i0 + bsel, n) - 1;   // the block's rows
  const int nk = i1 + 1;                                                // keys its last row sees
  const float inv_rows = 1.0f / (float)(i1 - i0 + 1);
  const int ta = i0 >> 5, tb = i1 >> 5;                                 // its 32-row tiles
  // score of key j: the tiles that see j, summed in tile order
  auto score = [&](int j) -> float {
    float acc = 0.f;
    for (int tt = ta; tt <= tb; ++tt)
      if (j <= (tt << 5) + 31) acc += colsum[(size_t)tt * n + j];
    return acc * inv_rows;
  };

  // the k-th largest score's bit pattern thr, and how many scores equal to
  // it are taken (the rest of the k are above it); everything when nk <= k
  const bool all = nk <= k;
  unsigned thr = 0u;
  int take = 0;
  if (!all) {
    unsigned prefix = 0u, pmask = 0u;
    int rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += kBsThreads) hist[b] = 0u;
      __syncthreads();
      for (int j = tid; j < nk; j += kBsThreads) {
        const unsigned v = __float_as_uint(score(j));
        if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0, d = 255;
        for (; d > 0; --d) {
          if (acc + (int)hist[d] >= rem) break;
          acc += (int)hist[d];
        }
        scal[0] = d;
        scal[1] = rem - acc;
      }
      __syncthreads();
      prefix |= (unsigned)scal[0] << shift;
      pmask |= 255u << shift;
      rem = scal[1];
      __syncthreads();
    }
    thr = prefix;
    take = rem;
  }

  // ordered emission: keys above thr, and the first `take` equal to it
  int base = 0, eq_seen = 0;
  for (int j0 = 0; j0 < nk; j0 += kBsThreads) {
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
    if (l == 0) wsum[0][w] = __popcll(be);
    __syncthreads();
    int eq_before = eq_seen + __popcll(be & below);
    for (int ww = 0; ww < w; ++ww) eq_before += wsum[0][ww];
    const bool keep = gt || (eq && eq_before < take);
    const unsigned long long bk = __ballot(keep);
    if (l == 0) wsum[1][w] = __popcll(bk);
    __syncthreads();
    int pos = base + __popcll(bk & below);
    for (int ww = 0; ww < w; ++ww) pos += wsum[1][ww];
    if (keep && pos < k) {   // (pos < k always holds: at most k scores are kept)
      win_id[pos] = j;
      win_m[pos] = m;
    }
    for (int ww = 0; ww < kBsWaves; ++ww) {
      eq_seen += wsum[0][ww];
      base += wsum[1][ww];
    }
    __syncthreads();
  }
  const int kk = base;   // = min(k, nk)

  for (int i = i0; i <= i1; ++i) {
    for (int p = tid; p < k; p += kBsThreads) {
      idx[(size_t)i * k + p] = p < kk ? win_id[p] : -1;
      if (mass) mass[(size_t)i * k + p] = p < kk ? win_m[p] : 0.f;
    }
    if (tid == 0) count[i] = kk;
  }
}

hipError_t launch_block_topk(const LayerShape& s, int bsel, int budget, const float* colsum,
                             int32_t* idx, int32_t* count, float* mass, hipStream_t stream) {
  if (bsel % 32) return hipErrorInvalidValue;   // selection blocks are whole 32-row tiles
  const int nblocks = (s.n + bsel - 1) / bsel;
  const size_t lds = (size_t)budget * (sizeof(int) + sizeof(float));
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(block_topk_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_topk_kernel, dim3(nblocks), dim3(kBsThreads), lds, stream, colsum,
                     s.n, bsel, budget, idx, count, mass);
  return hipGetLastError();
}

}  // namespace amtk
