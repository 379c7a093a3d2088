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
// from the block's tiles and takes its top-k with wg_topk (radix select on
// the score bits, winners emitted in id order).
#include "device_common.h"
#include "kernels.h"
#include "topk_core.h"

namespace amtk {

constexpr int kBsThreads = 1024;   // 16 waves: the radix passes over up to N scores are the cost

__global__ __launch_bounds__(kBsThreads) void block_topk_kernel(
    const float* __restrict__ colsum, int n, int bsel, int k, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, float* __restrict__ mass) {
  __shared__ TopkScratch<kBsThreads> sc;
  extern __shared__ __align__(16) unsigned char dyn[];   // winners: ids [k], scores [k]
  int* win_id = reinterpret_cast<int*>(dyn);
  float* win_m = reinterpret_cast<float*>(dyn + (size_t)k * sizeof(int));

  const int tid = threadIdx.x;
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

  const int kk = wg_topk<kBsThreads>(score, nk, k, sc, win_id, win_m);

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
