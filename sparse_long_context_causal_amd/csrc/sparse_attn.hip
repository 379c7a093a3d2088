// Gather sparse attention on a per-row support shared by all query heads.
//
// Method: gist.science page on arXiv 2606.07703, "Technischer Bericht"
// sections 2.1 and 2.2: after selection, the attention output of each query
// is recomputed with the original Q/K/V restricted to the chosen support
// (token ids, or 64-token key blocks from the indexer); the softmax is taken
// over the support only. The abstract states the same recompute step.
//
// Three attention kernels. bf16 with d = 128, 1, 2, 4 or 8 query heads per
// KV head and a power-of-two number of KV heads runs on MFMAs
// (sparse_attn_mfma_kernel, near the end of this file), in one pass or in key
// windows (support_windows_kernel finds where each window starts in every
// row's support; the windowed gather closes the file); the rows of a
// selection block may all read the block's first index row. The other
// shapes use one wavefront per query row, rows issued longest first: all Hq
// heads share the row's support, so one gathered token row K[j] (all Hkv
// heads, d contiguous: Hkv*d elements) serves every head. In the generic
// kernel lane l holds a contiguous slice of E = Hkv*d/64 elements of that
// row, i.e. a d-slice of KV head g = l / (d/E); it keeps its G query heads'
// slices of Q and of the output in registers, and logits are lane partial
// dot products summed over the d/E lanes of the group with xor shuffles.
// Tokens are processed in chunks: loads for a chunk are issued together,
// then one online-softmax rescale per chunk, then P*V in fp32 (no rounding
// of P).
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
    float tau, int qb_log2) {
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
  const int srow = (i >> qb_log2) << qb_log2;   // the row that holds row i's support
  const int cnt = min(max(count[srow], 0), max_units);
  const int total = cnt * key_block;
  const int32_t* ids = idx + (size_t)srow * max_units;
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
// VALU path for bf16, d = 128, 8 KV heads x 4 query heads each (the shape of
// the long-context GQA layers) where the MFMA path does not apply (token rows
// of all KV heads beyond 32-bit byte offsets). One wave per query row; lane l serves KV head
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
    float* __restrict__ lse_out, int n, int key_block, int max_units, float c, int qb_log2) {
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

  const int srow = (i >> qb_log2) << qb_log2;   // the row that holds row i's support
  const int cnt = min(max(count[srow], 0), max_units);
  const int total = cnt * key_block;
  const int32_t* ids = idx + (size_t)srow * max_units;

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
// MFMA path for bf16, d = 128, G = 1, 2, 4 or 8 query heads per KV head and
// a power-of-two number of KV heads, key blocks of 1 or a multiple of 16
// tokens. One single-wave workgroup per (query row, KV head), numbered
// row-major with the KV head fastest: workgroups are handed to the 8 XCDs
// round robin, so with 8 KV heads XCD g serves KV head g of every row and its
// L2 holds the keys and values of that one head (an eighth of the layer).
// The support is walked in chunks of 32 tokens (16 for short or key-block
// supports: one set); a chunk is two sets of 16
// (sigma = 0, 1), MFMA row m of set sigma being token 16*sigma + m.
//  * every global read of the loop is a DMA into LDS (no registers, no ALU
//    work): instruction c of a chunk brings the whole 256-byte key (and
//    value) rows of tokens 4c .. 4c+3, lane 16w + p taking 16-byte piece
//    p of row 4c + w; the piece of d-chunk x of row R sits at position
//    x ^ 2(R & 7) of the row, which keeps both LDS read patterns below
//    conflict free;
//  * logits S[token][head] with 16x16x32 bf16 MFMAs (exact products, fp32
//    sums): A = the key rows (lane l: token l%16, d 32s + 8(l/16) + [0, 8)
//    for s = 0..3, 16-byte LDS reads); B = the query fragment, column n
//    holding head n%4. Lane l ends with the logits of head l%4 for tokens
//    16*sigma + 4(l/16) + r in register r.
//  * online softmax per head: the maximum of the lane's 8 logits, then over
//    the 4 lane groups l/16 with two xor shuffles; rescaling only when a
//    maximum moved.
//  * P V with 16x16x32 bf16 MFMAs over the chunk's 32 tokens. Each weight
//    is split into two bf16 numbers, hi = p rounded and lo = (p - hi)
//    rounded, which keeps about 16 significant bits: A-operand rows 0-3
//    carry hi of the 4 heads, rows 4-7 lo (rows 8-15 repeat hi and are
//    never read). With the token order above, a lane's own weights already
//    sit where the A operand wants them (row l%16, k = 8(l/16) + 4 sigma + r).
//    B = the value rows through the transposing read ds_read_b64_tr_b16,
//    which hands every lane V[token][d] for 4 consecutive k. The two row
//    sums are added at the end.
//  * a chunk: wait for its loads, copy its keys and values out of LDS,
//    issue every load of the next chunk into the buffers just freed, then
//    compute from registers while those are in flight.
constexpr int kTileBytes = 8192;   // 32 rows of 256 bytes: keys or values of one chunk
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; the other counters left at their maximum)
constexpr int kWaitVm0 = 0x0F70;   // vmcnt(0)
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }   // vmcnt(n), n < 64

// A chunk's operands out of LDS: key fragment 4*sigma + s = 16-byte read at
// ka[s] + 4096*sigma; value fragment 2*blk + sigma = transposing read at
// va[blk] + 4096*sigma. Waits for them inside the same asm block.
__device__ __forceinline__ void read_chunk(const uint32_t (&ka)[4], const uint32_t (&va)[8],
                                           u32x4 (&kf)[8], u32x2 (&vt)[16]) {
  asm volatile(
      "ds_read_b128 %0, %24\n\t"
      "ds_read_b128 %1, %25\n\t"
      "ds_read_b128 %2, %26\n\t"
      "ds_read_b128 %3, %27\n\t"
      "ds_read_b128 %4, %24 offset:4096\n\t"
      "ds_read_b128 %5, %25 offset:4096\n\t"
      "ds_read_b128 %6, %26 offset:4096\n\t"
      "ds_read_b128 %7, %27 offset:4096\n\t"
      "ds_read_b64_tr_b16 %8, %28\n\t"
      "ds_read_b64_tr_b16 %9, %28 offset:4096\n\t"
      "ds_read_b64_tr_b16 %10, %29\n\t"
      "ds_read_b64_tr_b16 %11, %29 offset:4096\n\t"
      "ds_read_b64_tr_b16 %12, %30\n\t"
      "ds_read_b64_tr_b16 %13, %30 offset:4096\n\t"
      "ds_read_b64_tr_b16 %14, %31\n\t"
      "ds_read_b64_tr_b16 %15, %31 offset:4096\n\t"
      "ds_read_b64_tr_b16 %16, %32\n\t"
      "ds_read_b64_tr_b16 %17, %32 offset:4096\n\t"
      "ds_read_b64_tr_b16 %18, %33\n\t"
      "ds_read_b64_tr_b16 %19, %33 offset:4096\n\t"
      "ds_read_b64_tr_b16 %20, %34\n\t"
      "ds_read_b64_tr_b16 %21, %34 offset:4096\n\t"
      "ds_read_b64_tr_b16 %22, %35\n\t"
      "ds_read_b64_tr_b16 %23, %35 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]),
        "=&v"(kf[6]), "=&v"(kf[7]), "=&v"(vt[0]), "=&v"(vt[1]), "=&v"(vt[2]), "=&v"(vt[3]),
        "=&v"(vt[4]), "=&v"(vt[5]), "=&v"(vt[6]), "=&v"(vt[7]), "=&v"(vt[8]), "=&v"(vt[9]),
        "=&v"(vt[10]), "=&v"(vt[11]), "=&v"(vt[12]), "=&v"(vt[13]), "=&v"(vt[14]),
        "=&v"(vt[15])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
        "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7])
      : "memory");
}

// The same for a chunk of 16 tokens (one set): 4 key fragments, 8 value
// fragments.
__device__ __forceinline__ void read_chunk16(const uint32_t (&ka)[4], const uint32_t (&va)[8],
                                             u32x4 (&kf)[4], u32x2 (&vt)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b64_tr_b16 %4, %16\n\t"
      "ds_read_b64_tr_b16 %5, %17\n\t"
      "ds_read_b64_tr_b16 %6, %18\n\t"
      "ds_read_b64_tr_b16 %7, %19\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %21\n\t"
      "ds_read_b64_tr_b16 %10, %22\n\t"
      "ds_read_b64_tr_b16 %11, %23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(vt[0]), "=&v"(vt[1]),
        "=&v"(vt[2]), "=&v"(vt[3]), "=&v"(vt[4]), "=&v"(vt[5]), "=&v"(vt[6]), "=&v"(vt[7])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
        "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7])
      : "memory");
}

// lane c of each row of 16 lanes, broadcast to the row (c a constant after
// unrolling)
__device__ __forceinline__ int row_bcast16(int x, int c) {
  switch (c) {
    case 0: return __builtin_amdgcn_update_dpp(0, x, 0x150, 0xF, 0xF, false);
    case 1: return __builtin_amdgcn_update_dpp(0, x, 0x151, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_update_dpp(0, x, 0x152, 0xF, 0xF, false);
    case 3: return __builtin_amdgcn_update_dpp(0, x, 0x153, 0xF, 0xF, false);
    case 4: return __builtin_amdgcn_update_dpp(0, x, 0x154, 0xF, 0xF, false);
    case 5: return __builtin_amdgcn_update_dpp(0, x, 0x155, 0xF, 0xF, false);
    case 6: return __builtin_amdgcn_update_dpp(0, x, 0x156, 0xF, 0xF, false);
    default: return __builtin_amdgcn_update_dpp(0, x, 0x157, 0xF, 0xF, false);
  }
}

// broadcast of lane (l & ~3) | R to the 4 lanes of each quad
template <int R>
__device__ __forceinline__ float quad_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), R * 0x55, 0xF, 0xF, false));
}

// G query heads per KV head (1, 2, 4 or 8): the query fragment's column n
// holds head n % G, the weights' A-operand rows [0, G) carry hi and rows
// [G, 2G) lo, so result row 4q + r belongs to head (4q + r) % G. Per-head
// factors (rescale, normalisation, window merge) are the same in every lane
// of a head, and lane h < G holds head h: they are read with readlane.
template <int G>
__device__ __forceinline__ void head_factors(float x, float (&f)[4]) {
  float hv[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    hv[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), h));
  const bool odd = (threadIdx.x >> 4) & 1;   // lane group q odd
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (G == 8) f[r] = odd ? hv[4 + r] : hv[r];
    else f[r] = hv[r % G];
  }
}

// kTok: tokens per chunk, 32 (two sets of 16) or 16 (one set; half the LDS
// per wave, so more waves per CU)
template <bool kUnitTokens, int G, int kTok>   // kUnitTokens true: key_block == 1; false: key_block % 16 == 0
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kTok == 16 ? 4 : 3))) void sparse_attn_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, float* __restrict__ O,
    float* __restrict__ lse_out, int n, int hkv_log2, int key_block, int max_units, float c,
    const int32_t* __restrict__ wstart, int nwin, int win, int qb_log2) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "query heads per KV head");
  constexpr int D = 128;
  const int hkv = 1 << hkv_log2;   // a power of two: rows and heads by shifts
  const int HQ = hkv * G;
  const unsigned row_shift = (unsigned)hkv_log2 + 8u;   // bytes of one token, all KV heads: hkv * 256
  static_assert(kTok == 16 || kTok == 32, "chunks of one or two sets of 16 tokens");
  constexpr int kSets = kTok / 16, kDma = kTok / 4;   // DMA instructions per chunk (keys or values)
  constexpr int kBuf = kTok * 256;                     // bytes of a chunk's keys (or values)
  __shared__ __align__(256) unsigned char smem[2 * kBuf];   // keys, values of a chunk
  const int lane = threadIdx.x;
  const int i = n - 1 - (int)(blockIdx.x >> hkv_log2);   // longest rows first
  const int g = (int)(blockIdx.x & (unsigned)(hkv - 1));
  const int m = lane & 15, q = lane >> 4;
  // row i's support: its own index row, or with selection blocks of
  // 2^qb_log2 queries (one pass only) the block's first row
  const int srow = (i >> qb_log2) << qb_log2;
  int cnt = min(max(count[srow], 0), max_units);
  // Key windows (nwin > 0): this launch takes the support's units that lie
  // in window win, positions wstart[win] .. wstart[win + 1] of the row, and
  // merges its partial softmax with the earlier windows' (O normalised,
  // lse_out the running LSE). A row whose ids are not ascending
  // (wstart[0] < 0) is done whole in window 0.
  int s0 = 0;
  if (nwin > 0) {
    const int32_t* ws = wstart + (size_t)i * (nwin + 1);
    if (ws[0] >= 0) {
      s0 = ws[win];
      cnt = ws[win + 1] - s0;
    } else if (win > 0) {
      cnt = 0;
    }
    if (win > 0 && cnt <= 0) return;   // nothing in this window: keep the earlier result
  }
  const bool merge = nwin > 0 && win > 0;
  const int lim = max_units - 1 - s0;   // last readable position after the shift
  const int total = cnt * key_block;
  const int nch = (total + kTok - 1) / kTok;
  if (nch == 0) {   // empty support: zero output, LSE -inf
    for (int e = lane; e < G * D; e += 64) O[((size_t)i * HQ + G * g) * D + e] = 0.f;
    if (lse_out && lane < G) lse_out[(size_t)(G * g + lane) * n + i] = -INFINITY;
    return;
  }
  const int32_t* ids = idx + (size_t)srow * max_units + s0;
  unsigned char* kbuf = smem;
  unsigned char* vbuf = smem + kBuf;
  const unsigned char* Kb = reinterpret_cast<const unsigned char*>(K) + g * (D * 2);
  const unsigned char* Vb = reinterpret_cast<const unsigned char*>(V) + g * (D * 2);
  // DMA: lane 16q + m takes piece m of row 4c + q (c = 0..7), which holds
  // d-chunk m ^ 2((4c + q) & 7): byte offset in the row by the parity of c
  const unsigned xo0 = 16u * (unsigned)(m ^ (2 * q)), xo1 = 16u * (unsigned)(m ^ (8 + 2 * q));

  // Raw token ids of chunk ch. Single tokens: raw[0] in lane 16q + m holds
  // the id of token 4(m & 7) + q, the row that lane group q takes in DMA
  // instruction m & 7 (handed to the group's 16 lanes by a row broadcast
  // from lane m), and raw[8] the id of token lane % 32. Key blocks: the
  // block ids of the chunk's two sets in raw[0] and raw[4] (a set never
  // straddles two blocks).
  auto fetch_ids = [&](int ch, int (&raw)[9]) {
    const int t0 = ch * kTok;
    if constexpr (kUnitTokens) {
      raw[0] = ids[min(t0 + 4 * (m & (kDma - 1)) + q, lim)];
      raw[8] = ids[min(t0 + (lane & (kTok - 1)), lim)];
    } else {
      raw[0] = ids[min(t0 / key_block, lim)];
      if constexpr (kSets == 2) raw[4] = ids[min((t0 + 16) / key_block, lim)];
    }
  };
  // key/value row of token rr of the chunk starting at t0, given its raw id
  // (single tokens) or its set's block id; false for padding, negative ids
  // and keys after the query (row i then stands in: it weighs 0)
  auto token_row = [&](int t0, int rr, int id, int& r) -> bool {
    if constexpr (kUnitTokens) {
      r = id;
      return (t0 + rr < total) & (id >= 0) & (id <= i);
    } else {
      const int ts = t0 + (rr & 16);
      bool ok = (t0 + rr < total) & (id >= 0) & (id <= i / key_block);   // no overflow below
      r = ok ? id * key_block + (ts - (ts / key_block) * key_block) + (rr & 15) : i;
      return ok & (r <= i);
    }
  };
  // global byte offsets of the lane's 8 DMA pieces of chunk ch, and the
  // chunk's validity bits (bit t: token t is a support key; uniform)
  auto rows_of = [&](int ch, const int (&raw)[9], unsigned (&off)[8]) -> unsigned {
    const int t0 = ch * kTok;
    if constexpr (kUnitTokens) {
      // the row of token 4(m mod kDma) + q (row i for a token that weighs 0),
      // then row-broadcast from lane c of each 16-lane group for instruction c
      int r;
      const int rd = token_row(t0, 4 * (m & (kDma - 1)) + q, raw[0], r) ? r : i;
#pragma unroll
      for (int c8 = 0; c8 < kDma; ++c8)
        off[c8] = ((unsigned)row_bcast16(rd, c8) << row_shift) + ((c8 & 1) ? xo1 : xo0);
    } else {
#pragma unroll
      for (int c8 = 0; c8 < kDma; ++c8) {
        int r;
        const bool ok = token_row(t0, 4 * c8 + q, raw[4 * (c8 >> 2)], r);
        off[c8] = ((unsigned)(ok ? r : i) << row_shift) + ((c8 & 1) ? xo1 : xo0);
      }
    }
    int r;
    int own = raw[8];
    if constexpr (!kUnitTokens) {   // a select, not an indexed access (which would go to scratch)
      if constexpr (kSets == 2) own = (lane & 16) ? raw[4] : raw[0];
      else own = raw[0];
    }
    // (16-token chunks: lanes 16..31 repeat tokens 0..15, so the ballot's
    // upper half repeats its lower half)
    const bool okt = token_row(t0, lane & (kTok - 1), own, r);
    return (unsigned)__ballot(okt);   // lanes 0..31: tokens 0..31
  };
  const uint32_t kb_lds = lds_addr(kbuf), vb_lds = lds_addr(vbuf);
  auto issue = [&](const unsigned (&off)[8]) {
#pragma unroll
    for (int c8 = 0; c8 < kDma; ++c8) {
      __builtin_amdgcn_global_load_lds(Kb + off[c8], (lds_ptr_t)(uintptr_t)(kb_lds + 1024u * c8), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(Vb + off[c8], (lds_ptr_t)(uintptr_t)(vb_lds + 1024u * c8), 16, 0, 0);
    }
  };

  // query fragment: B operand column n = head n%G, d 32s + 8q + [0, 8)
  u32x4 qf[4];
  {
    const bf16_t* qr = Q + ((size_t)i * HQ + G * g + (lane & (G - 1))) * D + 8 * q;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qr + 32 * s);
  }
  // LDS read addresses. Keys: row 16 sigma + m, d-chunk q + 4s at position
  // (q + 4s) ^ 2(m & 7). Values: lane 16q + 4e + b reads row 4q + e of a
  // set, d 16 blk + 4b + [0, 4): d-chunk 2 blk + b/2 at position
  // (2 blk + b/2) ^ 2((4q + e) & 7).
  uint32_t ka[4], va[8];
  {
    const uint32_t kb0 = lds_addr(kbuf) + 256u * m + 16u * (unsigned)(q ^ (2 * (m & 1))) +
                         64u * (unsigned)((m & 7) >> 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) ka[s] = kb0 ^ (64u * s);
    const int r0 = 4 * q + ((lane >> 2) & 3), b = lane & 3;
    const uint32_t vb0 = lds_addr(vbuf) + 256u * r0 + 32u * (unsigned)(r0 & 7) + 16u * (b >> 1) + 8u * (b & 1);
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) va[blk] = vb0 ^ (32u * blk);
  }
  const float lo_sel = (m >= G && m < 2 * G) ? 1.0f : 0.0f;   // A-operand rows G..2G-1 carry lo

  // 32-token chunks: token ids run two chunks ahead, in two register sets
  // taken in turn (the loop is unrolled by two). The set a chunk reads was
  // filled before the previous chunk's wait, so the next chunk's load
  // addresses are formed before this chunk's wait, and between the wait and
  // the next chunk's loads there is only the copy out of LDS (1.3 % at 32K).
  // 16-token chunks keep one set, one chunk ahead, and form the addresses
  // after the copy: the second set and the early addresses would not fit
  // their 128 registers.
  constexpr bool kEarly = kTok == 32;
  int rawA[9], rawB[9];
  unsigned off[8];
  fetch_ids(0, rawA);
  unsigned valid_next = rows_of(0, rawA, off);
  if (nch > 1) fetch_ids(1, rawA);
  if (kEarly && nch > 2) fetch_ids(2, rawB);
  issue(off);
  if constexpr (kEarly) __builtin_amdgcn_s_waitcnt(vm_wait(2 * kDma));   // the ids of chunks 1 and 2

  f32x4 acc[8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) acc[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = kNegBig, lrun = 0.f;
  auto chunk = [&](int ch, int (&r)[9]) __attribute__((always_inline)) {
    const unsigned valid = valid_next;
    // r holds the ids of chunk ch + 1 (kEarly: fetched two chunks back, so
    // they have landed, and its load addresses are formed before the wait)
    if (kEarly && ch + 1 < nch) valid_next = rows_of(ch + 1, r, off);
    // every load in flight belongs to this chunk (and the ids of a later one)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // copying the chunk out and issuing the next one's loads go first among
    // the SIMD's waves: the gather is bound by the bytes its waves keep in
    // flight
    __builtin_amdgcn_s_setprio(2);
    u32x4 kf[4 * kSets];
    u32x2 vt[8 * kSets];
    if constexpr (kSets == 2) read_chunk(ka, va, kf, vt);
    else read_chunk16(ka, va, kf, vt);
    if (ch + 1 < nch) {   // the buffers are free again: start the next chunk
      if constexpr (kEarly) {
        issue(off);
        if (ch + 3 < nch) fetch_ids(ch + 3, r);
      } else {
        valid_next = rows_of(ch + 1, r, off);
        issue(off);
        if (ch + 2 < nch) fetch_ids(ch + 2, r);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    f32x4 sc[kSets];
#pragma unroll
    for (int sg = 0; sg < kSets; ++sg) {
      sc[sg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sc[sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[4 * sg + s]),
                                                         __builtin_bit_cast(bf16x8, qf[s]), sc[sg], 0, 0, 0);
    }
    constexpr int kE = 4 * kSets;   // logits per lane
    float x[kE];   // index 4 sigma + r: token 16 sigma + 4q + r, head lane%G
#pragma unroll
    for (int e = 0; e < kE; ++e) x[e] = sc[e >> 2][e & 3];
    if (valid != 0xffffffffu) {
      const unsigned vq = valid >> (4 * q);
#pragma unroll
      for (int e = 0; e < kE; ++e)
        if (!((vq >> ((e >> 2) * 16 + (e & 3))) & 1u)) x[e] = -INFINITY;
    }
    float smax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if constexpr (kSets == 2) smax = fmaxf(smax, fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    smax = max_xor<32>(max_xor<16>(smax));
    const float mnew = fmaxf(mrun, smax * c);
    if (__ballot(mnew != mrun)) {   // a head's maximum moved: rescale
      const float alpha = mnew == mrun ? 1.0f : fast_exp2(mrun - mnew);
      lrun *= alpha;
      float a[4];
      head_factors<G>(alpha, a);
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        acc[bb][0] *= a[0];
        acc[bb][1] *= a[1];
        acc[bb][2] *= a[2];
        acc[bb][3] *= a[3];
      }
      mrun = mnew;
    }
    float p[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) p[e] = fast_exp2(fmaf(x[e], c, -mnew));
    if constexpr (kSets == 2) lrun += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    else lrun += (p[0] + p[1]) + (p[2] + p[3]);
    // A operand: this lane's weights as bf16, hi or lo by its row
    unsigned pa[2 * kSets];
#pragma unroll
    for (int j = 0; j < 2 * kSets; ++j) {
      const unsigned hi =
          __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{p[2 * j], p[2 * j + 1]}, bf16x2));
      const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
      const f32x2 r2 = {fmaf(-lo_sel, h0, p[2 * j]), fmaf(-lo_sel, h1, p[2 * j + 1])};
      pa[j] = __builtin_bit_cast(unsigned, __builtin_convertvector(r2, bf16x2));
    }
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      if constexpr (kSets == 2) {
        const u32x4 pv = {pa[0], pa[1], pa[2], pa[3]};
        const u32x4 vv = {vt[2 * bb].x, vt[2 * bb].y, vt[2 * bb + 1].x, vt[2 * bb + 1].y};
        acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pv),
                                                          __builtin_bit_cast(bf16x8, vv), acc[bb], 0, 0, 0);
      } else {   // 16 tokens: k = 4q + r of the A operand is token 4q + r, as the value read gives it
        const u32x2 pv = {pa[0], pa[1]};
        acc[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, pv),
                                                           __builtin_bit_cast(bf16x4, vt[bb]), acc[bb], 0, 0, 0);
      }
    }
  };
  if constexpr (kEarly) {
    int ch = 0;
    for (; ch + 1 < nch; ch += 2) {
      chunk(ch, rawA);
      chunk(ch + 1, rawB);
    }
    if (ch < nch) chunk(ch, rawA);
  } else {
    for (int ch = 0; ch < nch; ++ch) chunk(ch, rawA);
  }
  const float l = sum_xor<32>(sum_xor<16>(lrun));   // every lane: head lane%G
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  // this window's LSE of head lane%G (log2 units)
  const float lw = l > 0.f ? mrun + log2f(l) : -INFINITY;
  float lnew = lw;
  const int rsel = (G == 4 ? q == 1 : G == 8 ? (q >> 1) == 1 : false) ? 2 : 0;
  const int hbase = G == 8 ? 4 * (q & 1) + rsel : rsel;
  const bool store = G == 8 ? true : G == 4 ? q < 2 : q == 0;
  float* const obase = O + ((size_t)i * HQ + G * g + hbase) * D + m;
  // merging: every earlier output value this lane rewrites, read in one batch
  // (in flight together with the running LSE read below)
  float prev[8][2];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) prev[bb][0] = prev[bb][1] = 0.f;
  if (merge && store) {
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      prev[bb][0] = obase[16 * bb];
      if constexpr (G > 1) prev[bb][1] = obase[D + 16 * bb];
    }
  }
  // Output of this window, combined with the earlier windows' when merging:
  // O = O_old * wa + O_win * wb per head (wa = 1 - wb = 0 without a merge),
  // with L = logaddexp(L_old, L_win), wa = exp(L_old - L), wb = exp(L_win - L).
  float wa = 0.f, wb = 1.f;
  if (merge) {
    const float lold = lse_out[(size_t)(G * g + (lane & (G - 1))) * n + i] * kLog2e;
    const float mx = fmaxf(lold, lw);
    wa = 1.f;
    wb = 0.f;
    lnew = lold;
    if (lw > -INFINITY) {
      const float ea = fast_exp2(lold - mx), eb = fast_exp2(lw - mx);
      const float sum = ea + eb;
      lnew = mx + log2f(sum);
      wa = ea / sum;
      wb = eb / sum;
    }
  }
  float fa[4], fb[4];   // per result row r of this lane: the head's wa and wb / l
  head_factors<G>(wa, fa);
  head_factors<G>(wb * inv, fb);
  // Result row 4q + r is head (4q + r) % G: hi for rows below G, lo for rows
  // G..2G-1 (higher rows are never used). A head's hi and lo rows meet in
  // one lane for G <= 2, in lane groups q and q^1 for G = 4 (xor 16) and q
  // and q^2 for G = 8 (xor 32). Then each storing lane group writes two
  // heads at d = 16 blk + m: G = 4: group 0 heads 0-1, group 1 heads 2-3;
  // G = 8: groups 0, 2, 1, 3 heads 0-1, 2-3, 4-5, 6-7.
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    f32x4 t = acc[bb];
    float o0, o1;
    if constexpr (G == 1) {
      o0 = t[0] + t[1];
      o1 = 0.f;
    } else if constexpr (G == 2) {
      o0 = t[0] + t[2];
      o1 = t[1] + t[3];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = G == 4 ? sum_xor<16>(t[r]) : sum_xor<32>(t[r]);
      o0 = rsel ? t[2] : t[0];
      o1 = rsel ? t[3] : t[1];
    }
    if (store) {
      const float fa0 = rsel ? fa[2] : fa[0], fa1 = rsel ? fa[3] : fa[1];
      const float fb0 = rsel ? fb[2] : fb[0], fb1 = rsel ? fb[3] : fb[1];
      float* orow = obase + 16 * bb;
      orow[0] = merge ? fmaf(prev[bb][0], fa0, o0 * fb0) : o0 * fb0;
      if constexpr (G > 1) orow[D] = merge ? fmaf(prev[bb][1], fa1, o1 * fb1) : o1 * fb1;
    }
  }
  if (lse_out && lane < G)
    lse_out[(size_t)(G * g + lane) * n + i] = lnew > -INFINITY ? lnew * kLn2 : -INFINITY;
}

// Start of each key window in every row's support (see the windowed gather
// below): out[i][w] = the first position of row i whose unit lies in window
// w or later, out[i][nwin] = the row's count; out[i][0] = -1 marks a row
// whose ids are not ascending. One wave per row.
__global__ __launch_bounds__(256) void support_windows_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int n, int max_units,
    int key_block, int win_tokens, int nwin, int32_t* __restrict__ out) {
  const int row = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;   // (uniform per wave)
  const int cnt = min(max(count[row], 0), max_units);
  const int32_t* ids = idx + (size_t)row * max_units;
  int32_t* o = out + (size_t)row * (nwin + 1);
  auto win_of = [&](int u) -> int {
    const long long t = (long long)max(u, 0) * key_block / win_tokens;
    return (int)min(t, (long long)(nwin - 1));
  };
  bool bad = false;
  for (int t = lane; t < cnt; t += 64) {
    const int u = ids[t];
    int wp = 0;
    if (t > 0) {
      const int up = ids[t - 1];
      bad |= u < up;
      wp = win_of(up);
    }
    for (int w = wp + 1; w <= win_of(u); ++w) o[w] = t;
  }
  const int wl = cnt > 0 ? win_of(ids[cnt - 1]) : 0;
  for (int w = wl + 1 + lane; w <= nwin; w += 64) o[w] = cnt;
  const bool any_bad = __ballot(bad) != 0ull;
  if (lane == 0) o[0] = any_bad ? -1 : 0;
}

template <typename T, int E, int G>
static hipError_t run_attn(const LayerShape& s, int key_block, int max_units, const void* q,
                           const void* k, const void* v, const int32_t* idx,
                           const int32_t* count, float* o, float* lse, int qb_log2,
                           hipStream_t stream) {
  constexpr int CH = (E >= 16) ? 4 : 8;
  const int blocks = (s.n + kAttnWaves - 1) / kAttnWaves;
  hipLaunchKernelGGL((sparse_attn_kernel<T, E, G, CH>), dim3(blocks), dim3(64 * kAttnWaves), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), idx, count, o, lse, s.n, s.hkv, s.d, key_block,
                     max_units, s.scale * kLog2e, s.scale, qb_log2);
  return hipGetLastError();
}

static int slice_width(const LayerShape& s) { return s.hkv * s.d / 64; }

// The MFMA gather: bf16, d = 128, G = Hq/Hkv in {1, 2, 4, 8}, a power-of-two
// number of KV heads as long as token rows of all KV heads stay within
// 32-bit byte offsets; single tokens or key blocks of a multiple of 16
// tokens.
static bool mfma_attn_shape(const LayerShape& s, int key_block) {
  if (s.dtype != kBF16 || s.d != 128 || s.hkv < 1 || s.hq % s.hkv) return false;
  if (s.hkv & (s.hkv - 1)) return false;
  const int G = s.hq / s.hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if ((unsigned long long)s.n * (unsigned long long)s.hkv * 256ull > 0xFFFFFFFFull) return false;
  return key_block == 1 || key_block % 16 == 0;
}

bool sparse_shape_supported(const LayerShape& s) {
  // key_block is 1 or 64 at every entry point: both run on the MFMA gather
  if (mfma_attn_shape(s, 1)) return true;
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
                            const int32_t* count, float* o, float* lse, int qb_log2,
                            hipStream_t stream) {
  const int G = s.hq / s.hkv;
#define AMTK_RUN_ATTN(GG) \
  run_attn<T, E, GG>(s, key_block, max_units, q, k, v, idx, count, o, lse, qb_log2, stream)
  if constexpr (E <= 8) {
    if (G == 8) return AMTK_RUN_ATTN(8);
  }
  if (G == 1) return AMTK_RUN_ATTN(1);
  if (G == 2) return AMTK_RUN_ATTN(2);
  if (G == 4) return AMTK_RUN_ATTN(4);
#undef AMTK_RUN_ATTN
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t attn_by_e(const LayerShape& s, int key_block, int max_units, const void* q,
                            const void* k, const void* v, const int32_t* idx,
                            const int32_t* count, float* o, float* lse, int qb_log2,
                            hipStream_t stream) {
#define AMTK_ATTN_E(EE) \
  attn_by_g<T, EE>(s, key_block, max_units, q, k, v, idx, count, o, lse, qb_log2, stream)
  switch (slice_width(s)) {
    case 1: return AMTK_ATTN_E(1);
    case 2: return AMTK_ATTN_E(2);
    case 4: return AMTK_ATTN_E(4);
    case 8: return AMTK_ATTN_E(8);
    case 16: return AMTK_ATTN_E(16);
  }
#undef AMTK_ATTN_E
  return hipErrorInvalidValue;
}

// Tokens per chunk of the MFMA gather: 16-token chunks halve the LDS per
// wave and let 16 waves share a CU; key-block supports (contiguous runs of
// rows) and short token supports run them, while token supports of more
// than kShortSupport units keep 32-token chunks (their rows' few hundred
// keys per key window would pay the per-chunk bookkeeping twice as often).
constexpr int kShortSupport = 128;

// One launch of the MFMA gather over rows >= n - rows (window w of nwin, or
// the whole support when nwin = 0).
static void launch_mfma_attn(const LayerShape& s, int key_block, int max_units, const void* q,
                             const void* k, const void* v, const int32_t* idx,
                             const int32_t* count, float* o, float* lse, long long rows,
                             const int32_t* starts, int nwin, int w, hipStream_t stream,
                             int qb_log2 = 0) {
  const int G = s.hq / s.hkv;
  const bool unit = key_block == 1;
  const bool t32 = unit && max_units > kShortSupport;
#define AMTK_GATHER_KERNEL(GG)                                                          \
  (t32 ? sparse_attn_mfma_kernel<true, GG, 32>                                          \
       : unit ? sparse_attn_mfma_kernel<true, GG, 16> : sparse_attn_mfma_kernel<false, GG, 16>)
  auto kern = G == 1 ? AMTK_GATHER_KERNEL(1) : G == 2 ? AMTK_GATHER_KERNEL(2)
            : G == 4 ? AMTK_GATHER_KERNEL(4) : AMTK_GATHER_KERNEL(8);
#undef AMTK_GATHER_KERNEL
  int hkv_log2 = 0;
  while ((1 << hkv_log2) < s.hkv) ++hkv_log2;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rows * s.hkv)), dim3(64), 0, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), idx, count, o, lse, s.n, hkv_log2, key_block,
                     max_units, s.scale * kLog2e, starts, nwin, w, qb_log2);
}

// One pass of the gather; row i reads the support of row (i >> qb_log2) << qb_log2.
static hipError_t sparse_attn_rows(const LayerShape& s, int key_block, int max_units,
                                   const void* q, const void* k, const void* v,
                                   const int32_t* idx, const int32_t* count, float* o,
                                   float* lse_sparse, int qb_log2, hipStream_t stream) {
  if (mfma_attn_shape(s, key_block)) {
    launch_mfma_attn(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, s.n, nullptr, 0,
                     0, stream, qb_log2);
    return hipGetLastError();
  }
  if (s.dtype == kBF16 && s.d == 128 && s.hkv == 8 && s.hq == 32) {
    constexpr int CH = 4;
    const int blocks = (s.n + kAttnWaves - 1) / kAttnWaves;
    hipLaunchKernelGGL((sparse_attn_g4_kernel<CH>), dim3(blocks), dim3(64 * kAttnWaves), 0, stream,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), idx, count, o, lse_sparse, s.n, key_block,
                       max_units, s.scale * kLog2e, qb_log2);
    return hipGetLastError();
  }
  if (s.dtype == kBF16)
    return attn_by_e<bf16_t>(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, qb_log2,
                             stream);
  return attn_by_e<float>(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, qb_log2,
                          stream);
}

hipError_t launch_sparse_attn(const LayerShape& s, int key_block, int max_units, const void* q,
                              const void* k, const void* v, const int32_t* idx,
                              const int32_t* count, float* o, float* lse_sparse,
                              hipStream_t stream) {
  return sparse_attn_rows(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, 0, stream);
}

hipError_t launch_sparse_attn_block_rows(const LayerShape& s, int key_block, int query_block,
                                         int max_units, const void* q, const void* k,
                                         const void* v, const int32_t* idx,
                                         const int32_t* count, float* o, float* lse_sparse,
                                         hipStream_t stream) {
  if (query_block < 1 || (query_block & (query_block - 1))) return hipErrorInvalidValue;
  int qb_log2 = 0;
  while ((1 << qb_log2) < query_block) ++qb_log2;
  return sparse_attn_rows(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, qb_log2,
                          stream);
}

// ------------------------------------------------------- windowed gather
// The per-row kernel above draws its keys and values from all of the row's
// history at once; at long N the rows in flight on one XCD touch far more
// K/V than its L2 holds. The windowed form walks the supports in key
// windows of kWindowTokens tokens (one KV head's keys and values of a
// window fill one XCD's 4 MB L2), one launch per window, each launch taking
// every row's units in that window and merging its partial softmax into
// the output (normalised O plus the running LSE). Rows below the window's
// first token have no keys there and are not launched.
constexpr int kWindowTokens = 8192;
constexpr int kMaxWindows = 64;

static bool windowed_shape(const LayerShape& s, int key_block) {
  return mfma_attn_shape(s, key_block);
}

static int window_tokens(const LayerShape& s) {
  const long long per = ((long long)s.n + kMaxWindows - 1) / kMaxWindows;
  const long long w = (per + 63) / 64 * 64;
  return (int)(w > kWindowTokens ? w : kWindowTokens);
}

static int window_count(const LayerShape& s) {
  const int w = window_tokens(s);
  return (int)(((long long)s.n + w - 1) / w);
}

size_t sparse_windowed_scratch_bytes(const LayerShape& s) {
  const size_t starts = (size_t)s.n * (size_t)(window_count(s) + 1) * sizeof(int32_t);
  const size_t lse = (size_t)s.hq * (size_t)s.n * sizeof(float);
  return ((starts + 255) & ~(size_t)255) + ((lse + 255) & ~(size_t)255);
}

hipError_t launch_sparse_attn_windowed(const LayerShape& s, int key_block, int max_units,
                                       const void* q, const void* k, const void* v,
                                       const int32_t* idx, const int32_t* count, float* o,
                                       float* lse_sparse, void* scratch, size_t scratch_bytes,
                                       hipStream_t stream) {
  const int nwin = window_count(s);
  if (!windowed_shape(s, key_block) || nwin < 2 || !scratch ||
      scratch_bytes < sparse_windowed_scratch_bytes(s))
    return launch_sparse_attn(s, key_block, max_units, q, k, v, idx, count, o, lse_sparse, stream);
  const int wt = window_tokens(s);
  unsigned char* b = static_cast<unsigned char*>(scratch);
  int32_t* starts = reinterpret_cast<int32_t*>(b);
  const size_t sb = ((size_t)s.n * (size_t)(nwin + 1) * sizeof(int32_t) + 255) & ~(size_t)255;
  float* lse_run = lse_sparse ? lse_sparse : reinterpret_cast<float*>(b + sb);
  hipLaunchKernelGGL(support_windows_kernel, dim3((unsigned)((s.n + 3) / 4)), dim3(256), 0, stream,
                     idx, count, s.n, max_units, key_block, wt, nwin, starts);
  hipError_t e = hipGetLastError();
  for (int w = 0; w < nwin && e == hipSuccess; ++w) {
    const long long rows = (long long)s.n - (long long)w * wt;   // rows >= the window's first token
    launch_mfma_attn(s, key_block, max_units, q, k, v, idx, count, o, lse_run, rows, starts, nwin,
                     w, stream);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace amtk
