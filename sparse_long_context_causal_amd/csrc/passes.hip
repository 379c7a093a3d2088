// Pass 1 (per-head row log-sum-exp) and pass 2 (head-averaged mass with a
// streaming top-k threshold filter) of the attention-mass top-k oracle.
//
// Method: "How Much Dense Attention is Necessary? Oracle-Guided Sparse
// Prefill for Full/GQA Layers in Hybrid Long-Context Models" (arXiv
// 2606.07703). gist.science page, "Technischer Bericht" section 2.1: for
// every query position the oracle forms each head's full causal softmax,
// averages the heads into one token-importance distribution and keeps its
// top-k units as the support. The abstract states the same oracle.
//
// Work decomposition (one workgroup = 32 consecutive query rows):
//   * wave g owns KV head g and the G query heads that read it; its G query
//     tiles stay in VGPRs for the whole launch (MFMA B operands);
//   * key tiles of 32 rows stream from HBM/L2 straight into VGPRs (MFMA A
//     operands), one tile ahead of the math;
//   * pass 1 keeps an online max / sum per (head, query) in registers;
//   * pass 2 turns logits into probabilities with pass 1's LSE, sums the G
//     heads of the wave in registers, sums the Hkv waves through LDS in a
//     fixed order, and filters the averaged mass against a per-row bound.
// Workgroups are issued longest-row first (causal load balance).
//
// Streaming filter (pass 2). Per query row, an LDS histogram over mass bins
// (exponent + 3 mantissa bits) counts the candidates kept so far. The bound
// bin b_tau only rises, and it always satisfies: at least k kept candidates
// lie in bins >= b_tau (or b_tau = 0). Every unit of the final top-k is
// therefore >= the bound when it is seen and is kept. Kept units are appended
// to the row's candidate pool in global memory; the select kernel then picks
// the exact top-k from the pool. A pool that overflows its capacity is
// detected (the count keeps running) and the row is redone densely.
#include "device_common.h"
#include "kernels.h"

namespace amtk {

// ------------------------------------------------------------------ pass 1
template <typename T, int D, int G>
__global__ __launch_bounds__(512) void pass1_lse_kernel(const T* __restrict__ Q,
                                                         const T* __restrict__ K,
                                                         float* __restrict__ lse, int n, int hkv,
                                                         float c, float tau,
                                                         int* __restrict__ zero_counter) {
  typedef Mma<T> M;
  constexpr int STEPS = D / M::kPerStep;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int g = wave;
  const int hq = hkv * G;
  const int ntiles = (n + 31) >> 5;
  const int qt = ntiles - 1 - (int)blockIdx.x;
  const int q0 = qt << 5;
  if (blockIdx.x == 0 && threadIdx.x == 0 && zero_counter) *zero_counter = 0;

  const int qrow = min(q0 + col, n - 1);
  typename M::frag qf[G][STEPS];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const T* qp = Q + ((size_t)qrow * hq + g * G + h) * D + hf * (D / 2);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) qf[h][s] = M::load(qp, s);
  }
  float mrun[G], lrun[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mrun[h] = kNegBig;
    lrun[h] = 0.f;
  }

  typename M::frag kf[STEPS];
  {
    const int kr = min(col, n - 1);
    const T* kp = K + ((size_t)kr * hkv + g) * D + hf * (D / 2);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) kf[s] = M::load(kp, s);
  }
  for (int kt = 0; kt <= qt; ++kt) {
    typename M::frag kn[STEPS];
    if (kt < qt) {
      const int kr = min(((kt + 1) << 5) + col, n - 1);
      const T* kp = K + ((size_t)kr * hkv + g) * D + hf * (D / 2);
#pragma unroll
      for (int s = 0; s < STEPS; ++s) kn[s] = M::load(kp, s);
    }
    const bool diag = (kt == qt);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < STEPS; ++s) M::mma(acc, kf[s], qf[h][s]);
      if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_row(r, hf) > col) acc[r] = -INFINITY;
      }
      float tmax = acc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, acc[r]);
      const float mnew = fmaxf(mrun[h], tmax);
      const float mc = mnew * c;
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += fast_exp2(fmaf(acc[r], c, -mc));
      lrun[h] = lrun[h] * fast_exp2((mrun[h] - mnew) * c) + sum;
      mrun[h] = mnew;
    }
    if (kt < qt) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) kf[s] = kn[s];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mo = xor32f(mrun[h]), lo = xor32f(lrun[h]);
    const float m = fmaxf(mrun[h], mo);
    const float l = lrun[h] * fast_exp2((mrun[h] - m) * c) + lo * fast_exp2((mo - m) * c);
    if (hf == 0 && q0 + col < n) lse[(size_t)(g * G + h) * n + q0 + col] = m * tau + logf(l);
  }
}

// ------------------------------------------------------------------ pass 2
struct RowState {
  int cnt[32];    // candidates appended (keeps counting past the capacity)
  int seen[32];   // cnt already folded into cge
  int cge[32];    // candidates in bins >= btau
  int btau[32];   // current bound bin
};

// Raise the row's bound while more than k candidates lie strictly above it.
__device__ __forceinline__ void raise_bound(RowState& rs, const unsigned* hist, int r, int budget) {
  const int fresh = rs.cnt[r] - rs.seen[r];
  rs.seen[r] = rs.cnt[r];
  int cg = rs.cge[r] + fresh;
  int bt = rs.btau[r];
  while (bt < kNumBins - 1 && cg - (int)hist[bt] >= budget) {
    cg -= (int)hist[bt];
    ++bt;
  }
  rs.cge[r] = cg;
  rs.btau[r] = bt;
}

template <typename T, int D, int G, int KB>
__global__ __launch_bounds__(512) void pass2_filter_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ lse, int n,
    int hkv, float c, float inv_hq, int budget, uint2* __restrict__ cand, int cap,
    int* __restrict__ cand_count, int* __restrict__ row_bin, int* __restrict__ ovf_count,
    int* __restrict__ ovf_list) {
  typedef Mma<T> M;
  constexpr int STEPS = D / M::kPerStep;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned* hist = reinterpret_cast<unsigned*>(smem);                      // [32][kNumBins]
  RowState& rs = *reinterpret_cast<RowState*>(hist + 32 * kNumBins);
  float* part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(&rs) + sizeof(RowState));

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int g = wave;
  const int hq = hkv * G;
  const int nthreads = hkv * 64;
  const int ntiles = (n + 31) >> 5;
  const int qt = ntiles - 1 - (int)blockIdx.x;
  const int q0 = qt << 5;
  const int q = q0 + col;
  const int qrow = min(q, n - 1);

  for (int t = threadIdx.x; t < 32 * kNumBins; t += nthreads) hist[t] = 0u;
  if (threadIdx.x < 32) {
    rs.cnt[threadIdx.x] = 0;
    rs.seen[threadIdx.x] = 0;
    rs.cge[threadIdx.x] = 0;
    rs.btau[threadIdx.x] = 0;
  }

  typename M::frag qf[G][STEPS];
  float bias[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const T* qp = Q + ((size_t)qrow * hq + g * G + h) * D + hf * (D / 2);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) qf[h][s] = M::load(qp, s);
    bias[h] = lse[(size_t)(g * G + h) * n + qrow] * kLog2e;
  }
  typename M::frag kf[STEPS];
  {
    const int kr = min(col, n - 1);
    const T* kp = K + ((size_t)kr * hkv + g) * D + hf * (D / 2);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) kf[s] = M::load(kp, s);
  }
  __syncthreads();

  float blk = 0.f;   // KB > 1: this query's mass over the current key block (this wave's heads)
  for (int kt = 0; kt <= qt; ++kt) {
    const int k0 = kt << 5;
    typename M::frag kn[STEPS];
    if (kt < qt) {
      const int kr = min(k0 + 32 + col, n - 1);
      const T* kp = K + ((size_t)kr * hkv + g) * D + hf * (D / 2);
#pragma unroll
      for (int s = 0; s < STEPS; ++s) kn[s] = M::load(kp, s);
    }
    const bool diag = (kt == qt);
    float pacc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pacc[r] = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < STEPS; ++s) M::mma(acc, kf[s], qf[h][s]);
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[r] += fast_exp2(fmaf(acc[r], c, -bias[h]));
    }
    if (diag) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, hf) > col) pacc[r] = 0.f;
    }

    if constexpr (KB == 1) {
      // ---- token units: sum the Hkv partial masses, filter, append
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(g * 16 + r) * 64 + lane] = pacc[r];
      __syncthreads();
      const int rpw = 16 / hkv;          // accumulator rows reduced by this wave
      const int bt = rs.btau[col];
      // element rr of this lane: its averaged mass, key id and filter verdict
      auto elem = [&](int rr, float& p, int& key) -> bool {
        const int r = wave * rpw + rr;
        p = 0.f;
        for (int gg = 0; gg < hkv; ++gg) p += part[(gg * 16 + r) * 64 + lane];
        p *= inv_hq;
        key = k0 + acc_row(r, hf);
        return (q < n) && (key <= q) && (mass_bin(p) >= bt);
      };
      int kept = 0;
      for (int rr = 0; rr < rpw; ++rr) {
        float p;
        int key;
        kept += elem(rr, p, key) ? 1 : 0;
      }
      const int other = xor32i(kept);
      int base = 0;
      if (hf == 0 && kept + other > 0) base = atomicAdd(&rs.cnt[col], kept + other);
      base = __shfl(base, col, 64);
      int pos = hf ? base + other : base;
      uint2* row = cand + (size_t)qrow * cap;
      unsigned* rh = hist + col * kNumBins;
      for (int rr = 0; rr < rpw; ++rr) {
        float p;
        int key;
        if (elem(rr, p, key)) {
          if (pos < cap) row[pos] = make_uint2(__float_as_uint(p), (unsigned)key);
          atomicAdd(&rh[mass_bin(p)], 1u);
          ++pos;
        }
      }
      __syncthreads();
      if (threadIdx.x < 32) raise_bound(rs, hist + threadIdx.x * kNumBins, threadIdx.x, budget);
    } else {
      // ---- key blocks of KB = 64 tokens = two key tiles
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ps += pacc[r];
      ps += xor32f(ps);
      blk += ps;
      const bool blk_end = (kt & 1) || diag;
      if (blk_end) {
        const int b = kt >> 1;
        float* pb = part + (b & 1) * hkv * 32;
        if (hf == 0) pb[g * 32 + col] = blk;
        blk = 0.f;
        __syncthreads();
        if (threadIdx.x < 32) {
          const int r = threadIdx.x;
          const int qq = q0 + r;
          float p = 0.f;
          for (int gg = 0; gg < hkv; ++gg) p += pb[gg * 32 + r];
          p *= inv_hq;
          if (qq < n && b * KB <= qq && mass_bin(p) >= rs.btau[r]) {
            const int pos = rs.cnt[r]++;
            if (pos < cap) cand[(size_t)qq * cap + pos] = make_uint2(__float_as_uint(p), (unsigned)b);
            hist[r * kNumBins + mass_bin(p)] += 1u;
            raise_bound(rs, hist + r * kNumBins, r, budget);
          }
        }
      }
    }
    if (kt < qt) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) kf[s] = kn[s];
    }
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    const int qq = q0 + threadIdx.x;
    if (qq < n) {
      const int cnt = rs.cnt[threadIdx.x];
      cand_count[qq] = cnt;
      row_bin[qq] = rs.btau[threadIdx.x];
      if (cnt > cap) ovf_list[atomicAdd(ovf_count, 1)] = qq;
    }
  }
}

// ------------------------------------------------------------ dispatching
template <typename T, int D, int G>
static hipError_t run_pass1(const LayerShape& s, const void* q, const void* k, float* lse,
                            int* zero_counter, hipStream_t stream) {
  const int ntiles = (s.n + 31) / 32;
  const float tau = s.scale;
  hipLaunchKernelGGL((pass1_lse_kernel<T, D, G>), dim3(ntiles), dim3(64 * s.hkv), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), lse, s.n, s.hkv,
                     tau * kLog2e, tau, zero_counter);
  return hipGetLastError();
}

static size_t pass2_lds_bytes(int hkv, int key_block) {
  size_t b = 32 * kNumBins * sizeof(unsigned) + sizeof(RowState);
  b += (key_block == 1) ? (size_t)hkv * 16 * 64 * sizeof(float) : (size_t)2 * hkv * 32 * sizeof(float);
  return b;
}

template <typename T, int D, int G, int KB>
static hipError_t run_pass2(const LayerShape& s, int budget, const void* q, const void* k,
                            const float* lse, const CandidatePool& pool, hipStream_t stream) {
  const int ntiles = (s.n + 31) / 32;
  const size_t lds = pass2_lds_bytes(s.hkv, KB);
  auto kern = pass2_filter_kernel<T, D, G, KB>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(ntiles), dim3(64 * s.hkv), lds, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), lse, s.n, s.hkv,
                     s.scale * kLog2e, 1.0f / (float)s.hq, budget, pool.cand, pool.cap, pool.count,
                     pool.bin, pool.ovf_count, pool.ovf_list);
  return hipGetLastError();
}

bool pass_shape_supported(const LayerShape& s) {
  if (s.hkv != 1 && s.hkv != 2 && s.hkv != 4 && s.hkv != 8) return false;
  if (s.hq % s.hkv) return false;
  const int G = s.hq / s.hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (s.d != 64 && s.d != 128) return false;
  // the wave's G query tiles live in VGPRs: G*d*elem_bytes <= 1024 per row
  if (G * s.d * (s.dtype == kBF16 ? 2 : 4) > 1024) return false;
  if (s.hq * s.d > kMaxQRow) return false;
  return s.dtype == kBF16 || s.dtype == kF32;
}

#define AMTK_PASS_DISPATCH(FN, ...)                                                  \
  do {                                                                               \
    const int G_ = s.hq / s.hkv;                                                     \
    if (s.dtype == kBF16) {                                                          \
      if (s.d == 64) {                                                               \
        if (G_ == 1) return FN<bf16_t, 64, 1>(__VA_ARGS__);                          \
        if (G_ == 2) return FN<bf16_t, 64, 2>(__VA_ARGS__);                          \
        if (G_ == 4) return FN<bf16_t, 64, 4>(__VA_ARGS__);                          \
        if (G_ == 8) return FN<bf16_t, 64, 8>(__VA_ARGS__);                          \
      } else {                                                                       \
        if (G_ == 1) return FN<bf16_t, 128, 1>(__VA_ARGS__);                         \
        if (G_ == 2) return FN<bf16_t, 128, 2>(__VA_ARGS__);                         \
        if (G_ == 4) return FN<bf16_t, 128, 4>(__VA_ARGS__);                         \
      }                                                                              \
    } else {                                                                         \
      if (s.d == 64) {                                                               \
        if (G_ == 1) return FN<float, 64, 1>(__VA_ARGS__);                           \
        if (G_ == 2) return FN<float, 64, 2>(__VA_ARGS__);                           \
        if (G_ == 4) return FN<float, 64, 4>(__VA_ARGS__);                           \
      } else {                                                                       \
        if (G_ == 1) return FN<float, 128, 1>(__VA_ARGS__);                          \
        if (G_ == 2) return FN<float, 128, 2>(__VA_ARGS__);                          \
      }                                                                              \
    }                                                                                \
    return hipErrorInvalidValue;                                                     \
  } while (0)

hipError_t launch_pass1_lse(const LayerShape& s, const void* q, const void* k, float* lse,
                            int* zero_counter, hipStream_t stream) {
  AMTK_PASS_DISPATCH(run_pass1, s, q, k, lse, zero_counter, stream);
}

template <typename T, int D, int G>
static hipError_t run_pass2_kb(const LayerShape& s, int key_block, int budget, const void* q,
                               const void* k, const float* lse, const CandidatePool& pool,
                               hipStream_t stream) {
  if (key_block == 1) return run_pass2<T, D, G, 1>(s, budget, q, k, lse, pool, stream);
  if (key_block == 64) return run_pass2<T, D, G, 64>(s, budget, q, k, lse, pool, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_pass2_filter(const LayerShape& s, int key_block, int budget, const void* q,
                               const void* k, const float* lse, const CandidatePool& pool,
                               hipStream_t stream) {
  AMTK_PASS_DISPATCH(run_pass2_kb, s, key_block, budget, q, k, lse, pool, stream);
}

}  // namespace amtk
