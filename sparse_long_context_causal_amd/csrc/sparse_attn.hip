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

// ---------------------------------------------------------------------------
// Fast path for bf16, d = 128, 8 KV heads x 4 query heads each (the shape of
// the long-context GQA layers). One wave per query row; lane l serves KV head
// g = l/8 and the 16 elements d in [16*(l%8), 16*(l%8)+16) of the K/V rows.
//  * QK: v_dot2 on raw bf16 pairs (no conversion), 8 per head and token.
//  * The 8 lanes of a KV head finish its 4 logits with a transposed DPP
//    butterfly (half-mirror, xor1, xor2): afterwards lane l holds the full
//    logit of head h(l) = 2*((l>>2)&1) + (l&1) of its group (lanes l and l^2
//    share a head). The online softmax then costs one exp per lane and token.
//  * The 4 heads' weights are gathered back into every lane with DPP for the
//    fp32 P*V update (P is never rounded).
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppBcast0 = 0x00;      // quad_perm [0,0,0,0]
constexpr int kDppBcast1 = 0x55;      // quad_perm [1,1,1,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Values of x held by the lanes of heads 0..3 of this lane's group.
__device__ __forceinline__ void gather4(float x, bool b2, float (&out)[4]) {
  const float qa = dpp<kDppBcast0>(x), qb = dpp<kDppBcast1>(x);
  const float ma = dpp<kDppHalfMirror>(qa), mb = dpp<kDppHalfMirror>(qb);
  out[0] = b2 ? ma : qa;
  out[1] = b2 ? mb : qb;
  out[2] = b2 ? qa : ma;
  out[3] = b2 ? qb : mb;
}

template <int CH>
__global__ __launch_bounds__(64 * kAttnWaves) void sparse_attn_g4_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, float* __restrict__ O,
    float* __restrict__ lse_out, int n, int key_block, int max_units, float c) {
  constexpr int D = 128, HKV = 8, G = 4, E = 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = n - 1 - (int)(blockIdx.x * kAttnWaves + wave);
  if (i < 0) return;
  const int g = lane >> 3, sub = lane & 7;
  const bool b2 = (sub >> 2) & 1, b0 = sub & 1;
  const int myh = 2 * (int)b2 + (int)b0;
  const int e0 = sub * E;
  const size_t off = (size_t)g * D + e0;

  unsigned qd[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4* qp = reinterpret_cast<const uint4*>(Q + ((size_t)i * (HKV * G) + g * G + h) * D + e0);
    const uint4 a = qp[0], b = qp[1];
    qd[h][0] = a.x; qd[h][1] = a.y; qd[h][2] = a.z; qd[h][3] = a.w;
    qd[h][4] = b.x; qd[h][5] = b.y; qd[h][6] = b.z; qd[h][7] = b.w;
  }
  float acc[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
  float m = kNegBig, l = 0.f;   // softmax state of head myh

  const int cnt = min(max(count[i], 0), max_units);
  const int total = cnt * key_block;
  const int32_t* ids = idx + (size_t)i * max_units;

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
    uint4 kx[CH][2], vx[CH][2];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const uint4* kp = reinterpret_cast<const uint4*>(K + (size_t)jj[cc] * (HKV * D) + off);
      const uint4* vp = reinterpret_cast<const uint4*>(V + (size_t)jj[cc] * (HKV * D) + off);
      kx[cc][0] = kp[0];
      kx[cc][1] = kp[1];
      vx[cc][0] = vp[0];
      vx[cc][1] = vp[1];
    }
    // logits of head myh for the chunk's tokens, in log2 units
    float x[CH];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const unsigned kd[8] = {kx[cc][0].x, kx[cc][0].y, kx[cc][0].z, kx[cc][0].w,
                              kx[cc][1].x, kx[cc][1].y, kx[cc][1].z, kx[cc][1].w};
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int w = 0; w < 8; w += 2) {
          a0 = dot2(qd[h][w], kd[w], a0);
          a1 = dot2(qd[h][w + 1], kd[w + 1], a1);
        }
        s[h] = a0 + a1;
      }
      const float k0 = b2 ? s[2] : s[0], k1 = b2 ? s[3] : s[1];
      const float t0v = k0 + dpp<kDppHalfMirror>(b2 ? s[0] : s[2]);
      const float t1v = k1 + dpp<kDppHalfMirror>(b2 ? s[1] : s[3]);
      const float u = (b0 ? t1v : t0v) + dpp<kDppXor1>(b0 ? t0v : t1v);
      const float tot = u + dpp<kDppXor2>(u);
      x[cc] = ok[cc] ? __fmul_rn(tot, c) : -INFINITY;
    }
    float cmax = kNegBig;
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) cmax = fmaxf(cmax, x[cc]);
    const float mnew = fmaxf(m, cmax);
    const float alpha = m == mnew ? 1.0f : fast_exp2(m - mnew);
    float p[CH];
    float ps = 0.f;
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      // the running maximum weighs exactly 1 (exp2 of 0 is only ~1 ulp exact)
      p[cc] = x[cc] == mnew ? 1.0f : fast_exp2(x[cc] - mnew);
      ps += p[cc];
    }
    l = fmaf(l, alpha, ps);
    m = mnew;
    // The output rescale is skipped when no head's running maximum moved:
    // every factor is then exactly 1.
    if (__ballot(alpha != 1.0f)) {
      float a4[4];
      gather4(alpha, b2, a4);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] *= a4[h];
    }
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      float p4[4];
      gather4(p[cc], b2, p4);
      const unsigned vd[8] = {vx[cc][0].x, vx[cc][0].y, vx[cc][0].z, vx[cc][0].w,
                              vx[cc][1].x, vx[cc][1].y, vx[cc][1].z, vx[cc][1].w};
      float vf[E];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        vf[2 * w] = __uint_as_float(vd[w] << 16);
        vf[2 * w + 1] = __uint_as_float(vd[w] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p4[h], vf[e], acc[h][e]);
    }
  }
  float l4[4], m4[4];
  gather4(l, b2, l4);
  gather4(m, b2, m4);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float inv = l4[h] > 0.f ? 1.0f / l4[h] : 0.f;
    float4* op = reinterpret_cast<float4*>(O + ((size_t)i * (HKV * G) + g * G + h) * D + e0);
#pragma unroll
    for (int v4 = 0; v4 < E / 4; ++v4)
      op[v4] = make_float4(acc[h][4 * v4] * inv, acc[h][4 * v4 + 1] * inv,
                           acc[h][4 * v4 + 2] * inv, acc[h][4 * v4 + 3] * inv);
  }
  if (lse_out && (sub == 0 || sub == 1 || sub == 4 || sub == 5))
    lse_out[(size_t)(g * G + myh) * n + i] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// MFMA path for bf16, d = 128, 8 KV heads x 4 query heads, key blocks of 1
// or a multiple of 16 tokens. One wave per query row, the KV heads one after
// another over the row's support, in chunks of 16 tokens:
//  * logits: the 4 query heads of KV head g against 16 gathered key rows
//    with four 16x16x32 bf16 MFMAs (exact products, fp32 sums). Rows of the
//    A operand repeat the 4 heads, so every 16-lane row of the result holds
//    s[head r][token lane%16] in register r;
//  * online softmax per head on those lanes (16-lane DPP max), the running
//    maximum weighing exactly 1 as in the generic path;
//  * the fp32 weights of the chunk go through a 256-byte LDS slot to all
//    lanes; 16-lane row q loads the value rows of tokens q, q+4, q+8, q+12
//    (16 bytes a lane), lane l accumulates d [8(l%16), +8) of the 4 heads
//    over its row's tokens in fp32 (P is never rounded), and the 4 rows are
//    summed once per KV head;
//  * the (head, chunk) steps form one loop whose next step's key rows,
//    value pairs and query fragment are loaded while the current one runs.
// Each lane looks up the token ids of its own key and value rows.
constexpr int kMfmaWaves = 4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// max / sum over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_row<0x128>(x));
  x = fmaxf(x, dpp_row<0x124>(x));
  x = fmaxf(x, dpp_row<0x122>(x));
  return fmaxf(x, dpp_row<0x121>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_row<0x128>(x);
  x += dpp_row<0x124>(x);
  x += dpp_row<0x122>(x);
  return x + dpp_row<0x121>(x);
}

template <bool kUnitTokens>   // true: key_block == 1; false: key_block % 16 == 0
__global__ __launch_bounds__(64 * kMfmaWaves) void sparse_attn_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, float* __restrict__ O,
    float* __restrict__ lse_out, int n, int key_block, int max_units, float c) {
  constexpr int D = 128, HKV = 8, G = 4, HQ = HKV * G;
  __shared__ float4 pbuf[kMfmaWaves][16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int i = n - 1 - (int)(blockIdx.x * kMfmaWaves + wave);
  if (i < 0) return;
  const int tl = lane & 15, qb = lane >> 4;   // token / k block of the MFMA operands
  const int cnt = min(max(count[i], 0), max_units);
  const int total = cnt * key_block;
  const int nch = (total + 15) >> 4;
  if (nch == 0) {   // empty support: zero output, LSE -inf
    for (int e = lane; e < HQ * D; e += 64) O[(size_t)i * HQ * D + e] = 0.f;
    if (lse_out && lane < HQ) lse_out[(size_t)lane * n + i] = -INFINITY;
    return;
  }
  const int32_t* ids = idx + (size_t)i * max_units;

  // token tt of the support: key/value row j (row i stands in for padding)
  auto token = [&](int tt, int& j) -> bool {
    bool ok;
    if constexpr (kUnitTokens) {
      const int id = ids[min(tt, max_units - 1)];
      ok = tt < total && id >= 0 && id <= i;
      j = ok ? id : i;
    } else {
      const int u = min(tt / key_block, max_units - 1);
      const int id = ids[u];
      const int jj = id * key_block + (tt - u * key_block);
      ok = tt < total && id >= 0 && jj <= i;
      j = ok ? jj : i;
    }
    return ok;
  };
  struct Step {
    uint4 kf[4];   // key row of token tl, d [32s + 8qb, +8) for s = 0..3
    uint4 vq[4];   // value row of token 4u + qb, d [8tl, 8tl + 8) for u = 0..3
    bool okl;      // this lane's key token is valid
  };
  auto load_step = [&](int stp, Step& st) {
    const int g = stp / nch, t0 = (stp - g * nch) << 4;
    int jl;
    st.okl = token(t0 + tl, jl);
    const bf16_t* kr = K + ((size_t)jl * HKV + g) * D + 8 * qb;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) st.kf[s2] = *reinterpret_cast<const uint4*>(kr + 32 * s2);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int jv;
      token(t0 + 4 * u + qb, jv);   // padding tokens weigh 0; the row is valid
      st.vq[u] = *reinterpret_cast<const uint4*>(V + ((size_t)jv * HKV + g) * D + 8 * tl);
    }
  };
  auto load_q = [&](int g, uint4 (&qf)[4]) {
    const bf16_t* qr = Q + ((size_t)i * HQ + G * g + (tl & 3)) * D + 8 * qb;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) qf[s2] = *reinterpret_cast<const uint4*>(qr + 32 * s2);
  };

  uint4 qf[4];
  float acc[G][8], m[G], lp[G];
  const int steps = HKV * nch;
  // one (KV head, chunk) step on loaded data
  auto run_step = [&](int stp, const Step& cur) {
    const int g = stp / nch, ch = stp - g * nch;
    if (ch == 0) {
      load_q(g, qf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
        m[h] = kNegBig;
        lp[h] = 0.f;
      }
    }
    // logits of the 4 heads for the chunk's 16 tokens
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qf[s2]),
                                                   __builtin_bit_cast(bf16x8, cur.kf[s2]), sc, 0, 0, 0);
    float p[G], alpha[G];
    bool moved = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float x = cur.okl ? __fmul_rn(sc[h], c) : -INFINITY;
      const float mnew = fmaxf(m[h], row16_max(x));
      alpha[h] = m[h] == mnew ? 1.0f : fast_exp2(m[h] - mnew);
      moved |= m[h] != mnew;
      // the running maximum weighs exactly 1 (exp2 of 0 is only ~1 ulp exact)
      p[h] = !cur.okl ? 0.f : (x == mnew ? 1.0f : fast_exp2(x - mnew));
      m[h] = mnew;
    }
    if (moved) {   // uniform: the row maxima are the same in every lane
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
        lp[h] *= alpha[h];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) lp[h] += p[h];
    if (lane < 16) pbuf[wave][tl] = make_float4(p[0], p[1], p[2], p[3]);
    __builtin_amdgcn_wave_barrier();
    float4 pt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pt[u] = pbuf[wave][4 * u + qb];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned w4[4] = {cur.vq[u].x, cur.vq[u].y, cur.vq[u].z, cur.vq[u].w};
      const float pw[4] = {pt[u].x, pt[u].y, pt[u].z, pt[u].w};
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const float v0 = __uint_as_float(w4[k2] << 16), v1 = __uint_as_float(w4[k2] & 0xffff0000u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * k2] = fmaf(pw[h], v0, acc[h][2 * k2]);
          acc[h][2 * k2 + 1] = fmaf(pw[h], v1, acc[h][2 * k2 + 1]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (ch == nch - 1) {   // head group g done: sum the 4 row groups' tokens
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float l = row16_sum(lp[h]);   // the 16 lanes of a row hold one token each
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = acc[h][e];
          v += __shfl_xor(v, 16, 64);
          v += __shfl_xor(v, 32, 64);
          o[e] = v * inv;
        }
        if (qb == 0) {
          float4* op = reinterpret_cast<float4*>(O + ((size_t)i * HQ + G * g + h) * D + 8 * tl);
          op[0] = make_float4(o[0], o[1], o[2], o[3]);
          op[1] = make_float4(o[4], o[5], o[6], o[7]);
        }
        if (lse_out && lane == 0)
          lse_out[(size_t)(G * g + h) * n + i] = l > 0.f ? (m[h] + log2f(l)) * kLn2 : -INFINITY;
      }
    }
  };
  // two step buffers in turn: the next step's loads are in flight meanwhile
  Step sa, sb;
  load_step(0, sa);
  for (int stp = 0; stp < steps; stp += 2) {
    if (stp + 1 < steps) load_step(stp + 1, sb);
    run_step(stp, sa);
    if (stp + 1 >= steps) break;
    if (stp + 2 < steps) load_step(stp + 2, sa);
    run_step(stp + 1, sb);
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
  if (s.dtype == kBF16 && s.d == 128 && s.hkv == 8 && s.hq == 32 &&
      (key_block == 1 || key_block % 16 == 0)) {
    const int blocks = (s.n + kMfmaWaves - 1) / kMfmaWaves;
    auto kern = key_block == 1 ? sparse_attn_mfma_kernel<true> : sparse_attn_mfma_kernel<false>;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * kMfmaWaves), 0, stream,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), idx, count, o, lse_sparse, s.n, key_block,
                       max_units, s.scale * kLog2e);
    return hipGetLastError();
  }
  if (s.dtype == kBF16 && s.d == 128 && s.hkv == 8 && s.hq == 32) {
    constexpr int CH = 4;
    const int blocks = (s.n + kAttnWaves - 1) / kAttnWaves;
    hipLaunchKernelGGL((sparse_attn_g4_kernel<CH>), dim3(blocks), dim3(64 * kAttnWaves), 0, stream,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), idx, count, o, lse_sparse, s.n, key_block,
                       max_units, s.scale * kLog2e);
    return hipGetLastError();
  }
  if (s.dtype == kBF16)
    return attn_by_e<bf16_t>(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, stream);
  return attn_by_e<float>(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, stream);
}

}  // namespace amtk
