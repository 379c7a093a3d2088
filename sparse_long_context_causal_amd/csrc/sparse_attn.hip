// Gather sparse attention on a per-row support shared by all query heads.
//
// Method: gist.science page on arXiv 2606.07703, "Technischer Bericht"
// sections 2.1 and 2.2: after selection, the attention output of each query
// is recomputed with the original Q/K/V restricted to the chosen support
// (token ids, or 64-token key blocks from the indexer); the softmax is taken
// over the support only. The abstract states the same recompute step.
//
// One wavefront per query row, rows issued longest first. All Hq heads share
// the row's support, so one gathered token row K[j] (all Hkv heads, d
// contiguous: Hkv*d elements) serves every head: lane l holds a contiguous
// slice of E = Hkv*d/64 elements of that row, i.e. a d-slice of KV head
// g = l / (d/E). The lane keeps its G query heads' slices of Q and of the
// output in registers; logits are lane partial dot products summed over the
// d/E lanes of the group with xor shuffles. Tokens are processed in chunks:
// loads for a chunk are issued together, then one online-softmax rescale per
// chunk, then P*V in fp32 (no rounding of P).
#include "device_common.h"
#include "kernels.h"

namespace amtk {

template <typename T, int E>
struct RowSlice;

template <int E>
struct RowSlice<bf16_t, E> {
  __device__ __forceinline__ static void load(const bf16_t* p, float (&x)[E]) {
    if constexpr (E >= 8) {
#pragma unroll
      for (int v = 0; v < E / 8; ++v) {
        const uint4 u = reinterpret_cast<const uint4*>(p)[v];
        const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          x[8 * v + 2 * t] = __uint_as_float(w[t] << 16);
          x[8 * v + 2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
        }
      }
    } else if constexpr (E == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      x[0] = __uint_as_float(u.x << 16);
      x[1] = __uint_as_float(u.x & 0xffff0000u);
      x[2] = __uint_as_float(u.y << 16);
      x[3] = __uint_as_float(u.y & 0xffff0000u);
    } else if constexpr (E == 2) {
      const unsigned u = *reinterpret_cast<const unsigned*>(p);
      x[0] = __uint_as_float(u << 16);
      x[1] = __uint_as_float(u & 0xffff0000u);
    } else {
      x[0] = bf16_to_f32(*p);
    }
  }
};

template <int E>
struct RowSlice<float, E> {
  __device__ __forceinline__ static void load(const float* p, float (&x)[E]) {
    if constexpr (E >= 4) {
#pragma unroll
      for (int v = 0; v < E / 4; ++v) {
        const float4 u = reinterpret_cast<const float4*>(p)[v];
        x[4 * v] = u.x;
        x[4 * v + 1] = u.y;
        x[4 * v + 2] = u.z;
        x[4 * v + 3] = u.w;
      }
    } else if constexpr (E == 2) {
      const float2 u = *reinterpret_cast<const float2*>(p);
      x[0] = u.x;
      x[1] = u.y;
    } else {
      x[0] = *p;
    }
  }
};

constexpr int kAttnWaves = 4;

template <typename T, int E, int G, int CH>
__global__ __launch_bounds__(64 * kAttnWaves) void sparse_attn_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, float* __restrict__ O,
    float* __restrict__ lse_out, int n, int hkv, int D, int key_block, int max_units, float c,
    float tau) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = n - 1 - (int)(blockIdx.x * kAttnWaves + wave);
  if (i < 0) return;
  const int lpg = D / E;                 // lanes per KV head
  const int g = lane / lpg;
  const int e0 = (lane - g * lpg) * E;
  const int hq = hkv * G;
  const int rowlen = hkv * D;

  float qv[G][E], acc[G][E], m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    RowSlice<T, E>::load(Q + ((size_t)i * hq + g * G + h) * D + e0, qv[h]);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    m[h] = kNegBig;
    l[h] = 0.f;
  }
  const int cnt = min(max(count[i], 0), max_units);
  const int total = cnt * key_block;
  const int32_t* ids = idx + (size_t)i * max_units;
  const size_t off = (size_t)g * D + e0;

  for (int t0 = 0; t0 < total; t0 += CH) {
    int jj[CH];
    bool ok[CH];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const int tt = t0 + cc;
      bool v = tt < total;
      const int u = key_block == 1 ? tt : tt / key_block;
      const int base = v ? ids[u] : 0;
      const int j = key_block == 1 ? base : base * key_block + (tt - u * key_block);
      v = v && base >= 0 && j <= i;
      ok[cc] = v;
      jj[cc] = v ? j : i;
    }
    float kx[CH][E], vx[CH][E];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      RowSlice<T, E>::load(K + (size_t)jj[cc] * rowlen + off, kx[cc]);
      RowSlice<T, E>::load(V + (size_t)jj[cc] * rowlen + off, vx[cc]);
    }
    float s[CH][G];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) a = fmaf(qv[h][e], kx[cc][e], a);
        s[cc][h] = a;
      }
    }
    for (int w = 1; w < lpg; w <<= 1) {
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[cc][h] += __shfl_xor(s[cc][h], w, 64);
      }
    }
    // logits in log2 units; the running max m is kept in the same units
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cmax = kNegBig;
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) {
        s[cc][h] = __fmul_rn(s[cc][h], c);   // rounded product, never fused below
        cmax = ok[cc] ? fmaxf(cmax, s[cc][h]) : cmax;
      }
      const float mnew = fmaxf(m[h], cmax);
      const float alpha = m[h] == mnew ? 1.0f : fast_exp2(m[h] - mnew);
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) {
        // the running maximum weighs exactly 1 (exp2 of 0 is only ~1 ulp exact)
        const float p = !ok[cc] ? 0.f : (s[cc][h] == mnew ? 1.0f : fast_exp2(s[cc][h] - mnew));
        l[h] += p;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, vx[cc][e], acc[h][e]);
      }
      m[h] = mnew;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float inv = l[h] > 0.f ? 1.0f / l[h] : 0.f;
    float* op = O + ((size_t)i * hq + g * G + h) * D + e0;
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = acc[h][e] * inv;
    if (lse_out && lane == g * lpg)
      lse_out[(size_t)(g * G + h) * n + i] = l[h] > 0.f ? (m[h] + log2f(l[h])) * kLn2 : -INFINITY;
  }
}

template <typename T, int E, int G>
static hipError_t run_attn(const LayerShape& s, int key_block, int max_units, const void* q,
                           const void* k, const void* v, const int32_t* idx,
                           const int32_t* count, float* o, float* lse, hipStream_t stream) {
  constexpr int CH = (E >= 16) ? 4 : 8;
  const int blocks = (s.n + kAttnWaves - 1) / kAttnWaves;
  hipLaunchKernelGGL((sparse_attn_kernel<T, E, G, CH>), dim3(blocks), dim3(64 * kAttnWaves), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), idx, count, o, lse, s.n, s.hkv, s.d, key_block,
                     max_units, s.scale * kLog2e, s.scale);
  return hipGetLastError();
}

static int slice_width(const LayerShape& s) { return s.hkv * s.d / 64; }

bool sparse_shape_supported(const LayerShape& s) {
  if (s.hkv < 1 || s.hq % s.hkv) return false;
  const int G = s.hq / s.hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (s.d != 64 && s.d != 128) return false;
  if ((s.hkv * s.d) % 64) return false;
  const int E = slice_width(s);
  if (E != 1 && E != 2 && E != 4 && E != 8 && E != 16) return false;
  if (G * E > 64) return false;
  return s.dtype == kBF16 || s.dtype == kF32;
}

template <typename T, int E>
static hipError_t attn_by_g(const LayerShape& s, int key_block, int max_units, const void* q,
                            const void* k, const void* v, const int32_t* idx,
                            const int32_t* count, float* o, float* lse, hipStream_t stream) {
  const int G = s.hq / s.hkv;
  if constexpr (E <= 8) {
    if (G == 8) return run_attn<T, E, 8>(s, key_block, max_units, q, k, v, idx, count, o, lse, stream);
  }
  if (G == 1) return run_attn<T, E, 1>(s, key_block, max_units, q, k, v, idx, count, o, lse, stream);
  if (G == 2) return run_attn<T, E, 2>(s, key_block, max_units, q, k, v, idx, count, o, lse, stream);
  if (G == 4) return run_attn<T, E, 4>(s, key_block, max_units, q, k, v, idx, count, o, lse, stream);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t attn_by_e(const LayerShape& s, int key_block, int max_units, const void* q,
                            const void* k, const void* v, const int32_t* idx,
                            const int32_t* count, float* o, float* lse, hipStream_t stream) {
  switch (slice_width(s)) {
    case 1: return attn_by_g<T, 1>(s, key_block, max_units, q, k, v, idx, count, o, lse, stream);
    case 2: return attn_by_g<T, 2>(s, key_block, max_units, q, k, v, idx, count, o, lse, stream);
    case 4: return attn_by_g<T, 4>(s, key_block, max_units, q, k, v, idx, count, o, lse, stream);
    case 8: return attn_by_g<T, 8>(s, key_block, max_units, q, k, v, idx, count, o, lse, stream);
    case 16: return attn_by_g<T, 16>(s, key_block, max_units, q, k, v, idx, count, o, lse, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sparse_attn(const LayerShape& s, int key_block, int max_units, const void* q,
                              const void* k, const void* v, const int32_t* idx,
                              const int32_t* count, float* o, float* lse_sparse,
                              hipStream_t stream) {
  if (s.dtype == kBF16)
    return attn_by_e<bf16_t>(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, stream);
  return attn_by_e<float>(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, stream);
}

}  // namespace amtk
