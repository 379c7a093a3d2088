// KL-distillation loss of the head-collapsed indexer against the oracle's
// attention mass, with its gradients, in one streaming pass over the causal
// triangle (the N x N matrices are never stored).
//
// Method: gist.science page on arXiv 2606.07703, "Technischer Bericht"
// section 2.2: the indexer is trained by KL divergence from the dense
// head-averaged attention-mass distribution, the backbone frozen. With
// teacher P_i (the head-averaged mass over keys j <= i) and student
// Q_i = causal softmax of t_ij = tau_idx <q_idx[i], k_idx[j]>:
//   KL_i = sum_j P_ij (log P_ij - log Q_ij),   L = (1/N) sum_i KL_i,
//   dL/dt_ij = (Q_ij - P_ij) / N,
//   dL/dq_idx[i] = tau_idx sum_j dL/dt_ij k_idx[j],
//   dL/dk_idx[j] = tau_idx sum_{i >= j} dL/dt_ij q_idx[i].
// Both log-sum-exps come first from pass 1 (teacher per head, student with
// one head of d_idx).
//
// kl_tile_kernel (bf16, d = 128, 8 KV heads x 4 query heads, d_idx = 64):
// one workgroup of 8 waves per 32-query tile, wave g = KV head g, key tiles
// streamed as in pass 2. Per key tile:
//  * every wave scores its 4 heads (32x32x16 MFMAs), turns them into
//    probabilities with the dense LSE and sums them; the 8 partial tiles
//    meet in LDS and the workgroup assembles the teacher tile P[key][query];
//  * waves 0 and 1 compute the student tile t^T[key][query] (4 MFMAs),
//    Q and dS = Q - P in the score layout (lane = query), the KL terms of
//    half of the keys each, and accumulate dq^T[d][query] += k_idx^T dS^T for
//    their 32 of the 64 dimensions (A = k_idx columns by transposing LDS
//    reads, B = the lane's own dS); dS is split into bf16 hi + lo, so the
//    products keep about 16 significant bits;
//  * waves 2 and 3 compute the student tile the other way round
//    (lane = key), dS, and this tile pair's dk^T[d][key] = q_idx^T dS
//    for their 32 dimensions, written to the workspace;
// kl_dk_reduce_kernel then sums, per key tile, the pair partials over the
// query tiles in a fixed order (deterministic), and kl_loss_kernel the mean.
//
// The k_idx / q_idx tiles (32 rows of 128 bytes) sit in LDS with d-chunk x
// of row R at position x ^ f(R), f(R) = 2(R & 3) + ((R >> 2) & 1): the
// 16-byte operand reads (8 rows at one chunk) and the transposing reads
// (4 rows x 32 bytes) are both free of bank conflicts.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace amtk {

namespace {

constexpr int kKlD = 128, kKlG = 4, kKlHkv = 8, kKlHq = kKlHkv * kKlG, kKlDi = 64;
typedef KTile<bf16_t, kKlD> KlKT;
constexpr int kKlNc = KlKT::kChunks;

// LDS map (bytes)
constexpr unsigned kKlSlots = 0;                                  // 8 K slots
constexpr unsigned kKlPart = kKlSlots + kKlHkv * KlKT::kBytes;    // 8 partial tiles
constexpr unsigned kKlPTile = kKlPart + kKlHkv * 16 * 64 * 4;     // P [32][33] fp32
constexpr unsigned kKlKidx = kKlPTile + 4352;                     // k_idx tiles x2
constexpr unsigned kKlQidx = kKlKidx + 2 * 4096;                  // q_idx tile
constexpr unsigned kKlLseT = kKlQidx + 4096;                      // student LSE x log2e [32]
constexpr unsigned kKlRed = kKlLseT + 128;                        // KL of wave 1 [32]
constexpr unsigned kKlDq = kKlRed + 128;                          // dq^T accumulators of waves 0, 1
constexpr unsigned kKlBias = kKlDq + 2 * 16 * 64 * 4;             // dense LSE x log2e [32 heads][32]
constexpr unsigned kKlLds = kKlBias + kKlHq * 32 * 4;
constexpr int kKlPitch = 33;                                      // P row pitch (floats)

typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ unsigned idx_swizzle(unsigned r) { return ((r & 3u) << 1) | ((r >> 2) & 1u); }

__device__ __forceinline__ unsigned pack2_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// One operand fragment (row lane%32, d = 16 s + 8(lane/32) + [0, 8)) of
// each of two 32-row index tiles; one asm block that waits for them.
__device__ __forceinline__ void read_idx_frag2(uint32_t a, uint32_t b, u32x4& fa, u32x4& fb) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(fa), "=&v"(fb)
      : "v"(a), "v"(b)
      : "memory");
}

// The transposed operand of one 32-wide d tile: tr[2 ks + sec] holds rows
// 16 ks + 8 sec + 4(lane/32) + [0, 4) at d = 32 dt + lane%32.
__device__ __forceinline__ void read_idx_tr(uint32_t a, u32x2 (&tr)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:2048\n\t"
      "ds_read_b64_tr_b16 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(tr[0]), "=&v"(tr[1]), "=&v"(tr[2]), "=&v"(tr[3])
      : "v"(a)
      : "memory");
}

// The dq^T accumulator of a lane (4 float4 at a, a + 1024, a + 2048, a + 3072)
// out of and back into LDS. As asm, the compiler does not hold these behind
// the global->LDS loads in flight (it cannot tell the regions apart).
__device__ __forceinline__ void dq_load(uint32_t a, f32x16& acc) {
  f32x4 x0, x1, x2, x3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(a)
      : "memory");
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    acc[r] = x0[r];
    acc[4 + r] = x1[r];
    acc[8 + r] = x2[r];
    acc[12 + r] = x3[r];
  }
}
// The accumulator comes straight from an MFMA, and the compiler does not
// insert the wait states an LDS write of an MFMA result needs in front of an
// asm block: the three s_nop (24 wait states) cover them.
__device__ __forceinline__ void dq_store(uint32_t a, const f32x16& acc) {
  const f32x4 x0 = {acc[0], acc[1], acc[2], acc[3]}, x1 = {acc[4], acc[5], acc[6], acc[7]};
  const f32x4 x2 = {acc[8], acc[9], acc[10], acc[11]}, x3 = {acc[12], acc[13], acc[14], acc[15]};
  asm volatile(
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "ds_write_b128 %0, %1\n\t"
      "ds_write_b128 %0, %2 offset:1024\n\t"
      "ds_write_b128 %0, %3 offset:2048\n\t"
      "ds_write_b128 %0, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "v"(a), "v"(x0), "v"(x1), "v"(x2), "v"(x3)
      : "memory");
}

__global__ __launch_bounds__(512) void kl_tile_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ QI,
    const bf16_t* __restrict__ KI, const float* __restrict__ lse, const float* __restrict__ lse_t,
    int n, float c, float ct, float* __restrict__ kl_row, float* __restrict__ dq,
    float* __restrict__ dk_part, float grad_scale) {
  extern __shared__ __align__(1024) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int g = wave;
  const int ntiles = (n + 31) >> 5;
  const int qt = ntiles - 1 - (int)blockIdx.x;   // longest rows first
  const int q0 = qt << 5;
  const int qrow = min(q0 + col, n - 1);
  const uint32_t base = lds_addr(smem);
  float* part = reinterpret_cast<float*>(smem + kKlPart);
  float* ptile = reinterpret_cast<float*>(smem + kKlPTile);
  unsigned char* slot = smem + kKlSlots + wave * KlKT::kBytes;

  KLane<bf16_t, kKlD> kl;
  kl.init(lane, kKlHkv);
  kl.issue(K, n, kKlHkv, g, 0, slot);
  // k_idx tile kt, rows 8w .. 8w+7 by wave w < 4 (lane: row 8w + lane/8,
  // position lane%8, holding d-chunk (lane%8) ^ f(row))
  const unsigned drow = 8u * (unsigned)wave + ((unsigned)lane >> 3);
  const unsigned dpiece = 16u * (((unsigned)lane & 7u) ^ idx_swizzle(drow));
  auto issue_kidx = [&](int kt) {
    const int row = min((kt << 5) + (int)drow, n - 1);
    const unsigned char* src = reinterpret_cast<const unsigned char*>(KI) + (size_t)row * (kKlDi * 2) + dpiece;
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(uintptr_t)(base + kKlKidx + 4096u * (kt & 1) + 1024u * wave), 16, 0, 0);
  };
  if (wave < 4) issue_kidx(0);

  // the tile's q_idx rows and student LSE (log2 units) into LDS
  if (threadIdx.x < 256) {
    const unsigned r = threadIdx.x >> 3, m = threadIdx.x & 7;
    const int row = min(q0 + (int)r, n - 1);
    const uint4 v = *reinterpret_cast<const uint4*>(QI + (size_t)row * kKlDi + 8 * (m ^ idx_swizzle(r)));
    *reinterpret_cast<uint4*>(smem + kKlQidx + 128u * r + 16u * m) = v;
  } else if (threadIdx.x < 288) {
    const int r = (int)threadIdx.x - 256;
    reinterpret_cast<float*>(smem + kKlLseT)[r] = lse_t[min(q0 + r, n - 1)] * kLog2e;
  }

  uint4 qc[kKlG][kKlNc];
  load_q_tiles<bf16_t, kKlD, kKlG>(Q, qrow, kKlHq, g, lane, qc);
  // the tile's dense LSE (log2 units), read back per key tile
  float* biasl = reinterpret_cast<float*>(smem + kKlBias) + g * kKlG * 32 + col;
  if (hf == 0) {
#pragma unroll
    for (int h = 0; h < kKlG; ++h) biasl[32 * h] = lse[(size_t)(g * kKlG + h) * n + qrow] * kLog2e;
  }

  // operand addresses in the index tiles (tile base added per use)
  const unsigned fr = (unsigned)col;
  const uint32_t frag_off = 128u * fr + 16u * ((unsigned)hf ^ ((fr >> 2) & 1u)) + 32u * (fr & 3u);
  uint32_t tr_off;
  {
    const unsigned G16 = (unsigned)lane >> 4, e = ((unsigned)lane >> 2) & 3u, cc = (unsigned)lane & 3u;
    const unsigned u = 2u * (G16 & 1u) + (cc >> 1), sw = 2u * e + (G16 >> 1);
    tr_off = 128u * (4u * (G16 >> 1) + e) + 8u * (cc & 1u) + 16u * (u ^ sw);
  }
  const int dt = wave & 1;   // the d tile of waves 0-3

  // dq^T accumulators of waves 0 and 1 live in LDS between key tiles
  // (registers j*4 .. j*4+3 of lane l at float4 slot (wave, j, l))
  float4* dqs = reinterpret_cast<float4*>(smem + kKlDq) + (wave & 1) * 256 + lane;
  const uint32_t dq_lds = base + kKlDq + 16u * (unsigned)((wave & 1) * 256 + lane);
  if (wave < 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dqs[64 * j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float klacc = 0.f;
  barrier_lds();   // q_idx tile and student LSE visible

  for (int kt = 0; kt <= qt; ++kt) {
    const int k0 = kt << 5;
    const bool diag = kt == qt;
    // ---- teacher: this wave's 4 heads, summed
    uint4 kc[kKlNc];
    wait_vmem_all();   // this wave's K tile (and k_idx piece) have landed
    kl.read(slot, kc);
    if (kt < qt) kl.issue(K, n, kKlHkv, g, (kt + 1) << 5, slot);
    float pacc[16];
    f32x16 a;
#pragma unroll
    for (int h = 0; h < kKlG; ++h) {
      score_tile<bf16_t, kKlNc>(a, kc, qc[h]);
      const float bias = biasl[32 * h];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(a[r], c, -bias));
        pacc[r] = h == 0 ? e : pacc[r] + e;
      }
      // one head at a time: keeps the scheduler from hoisting the next
      // head's MFMAs (and their accumulators) above these exponentials
      __builtin_amdgcn_sched_barrier(0);
    }
    if (diag) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, hf) > col) pacc[r] = 0.f;
    }
    {
      const int wb = g * 1024 + lane;   // part_index(g, r, lane) = wb ^ (68 r)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[wb ^ (68 * r)] = pacc[r];
    }
    barrier_lds();   // partial tiles visible
    if (wave < 4 && kt < qt) issue_kidx(kt + 1);
    // ---- assemble P[key][query] = (1/Hq) sum over the 8 partial tiles
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = (int)threadIdx.x + 512 * u;
      const int key = e >> 5, qq = e & 31;
      const int r = ((key >> 3) << 2) | (key & 3), h2 = (key >> 2) & 1;
      const int src = (r * 64 + ((qq + 32 * h2) ^ (4 * r)));
      float p = part[src];
#pragma unroll
      for (int gg = 1; gg < kKlHkv; ++gg) p += part[src + gg * 1024];
      ptile[key * kKlPitch + qq] = p * (1.0f / (float)kKlHq);
    }
    barrier_lds();   // P visible
    if (wave >= 4) continue;

    // ---- student tile, dS = Q - P, and the gradient products
    const uint32_t kb = base + kKlKidx + 4096u * (unsigned)(kt & 1);
    const uint32_t qb = base + kKlQidx;
    const float* lse_tl = reinterpret_cast<const float*>(smem + kKlLseT);
    if (wave < 2) {
      // lane = query col: t^T[key][query] = k_idx q_idx^T
      f32x16 t = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 kf, qf;
        read_idx_frag2((kb + frag_off) ^ (32u * s), (qb + frag_off) ^ (32u * s), kf, qf);
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf),
                                                    __builtin_bit_cast(bf16x8, qf), t, 0, 0, 0);
      }
      const float lt = lse_tl[col];
      const bool qlive = q0 + col < n;
      u32x4 bh[2], bl[2];
#pragma unroll
      for (int r2 = 0; r2 < 16; r2 += 2) {
        float dsv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = r2 + u, key = acc_row(r, hf);
          const float p = ptile[key * kKlPitch + col];
          const float x = fmaf(t[r], ct, -lt);   // log2 Q
          const bool live = qlive && !(diag && key > col);
          dsv[u] = live ? fast_exp2(x) - p : 0.f;
          // KL terms, registers 0-7 in wave 0 and 8-15 in wave 1: P (log P - log Q)
          if ((r >> 3) == wave && live && p > 0.f) klacc = fmaf(p, (__log2f(p) - x) * kLn2, klacc);
        }
        const unsigned h = pack2_bf16(dsv[0], dsv[1]);
        bh[r2 >> 3][(r2 & 7) >> 1] = h;
        bl[r2 >> 3][(r2 & 7) >> 1] =
            pack2_bf16(dsv[0] - __uint_as_float(h << 16), dsv[1] - __uint_as_float(h & 0xffff0000u));
      }
      u32x2 tr[4];
      read_idx_tr((kb + tr_off) ^ (64u * (unsigned)dt), tr);   // k_idx^T, rows = keys
      f32x16 dqacc;
      dq_load(dq_lds, dqacc);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 av = {tr[2 * ks].x, tr[2 * ks].y, tr[2 * ks + 1].x, tr[2 * ks + 1].y};
        dqacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                        __builtin_bit_cast(bf16x8, bh[ks]), dqacc, 0, 0, 0);
        dqacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                        __builtin_bit_cast(bf16x8, bl[ks]), dqacc, 0, 0, 0);
      }
      dq_store(dq_lds, dqacc);
    } else {
      // lane = key col: t[query][key] = q_idx k_idx^T
      f32x16 t = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 kf, qf;
        read_idx_frag2((kb + frag_off) ^ (32u * s), (qb + frag_off) ^ (32u * s), kf, qf);
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qf),
                                                    __builtin_bit_cast(bf16x8, kf), t, 0, 0, 0);
      }
      u32x4 bh[2], bl[2];
#pragma unroll
      for (int r2 = 0; r2 < 16; r2 += 2) {
        float dsv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = r2 + u, qq = acc_row(r, hf);
          const float p = ptile[col * kKlPitch + qq];
          const float x = fmaf(t[r], ct, -lse_tl[qq]);
          const bool live = q0 + qq < n && !(diag && col > qq);
          dsv[u] = live ? fast_exp2(x) - p : 0.f;
        }
        const unsigned h = pack2_bf16(dsv[0], dsv[1]);
        bh[r2 >> 3][(r2 & 7) >> 1] = h;
        bl[r2 >> 3][(r2 & 7) >> 1] =
            pack2_bf16(dsv[0] - __uint_as_float(h << 16), dsv[1] - __uint_as_float(h & 0xffff0000u));
      }
      u32x2 tr[4];
      read_idx_tr((qb + tr_off) ^ (64u * (unsigned)dt), tr);   // q_idx^T, rows = queries
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 av = {tr[2 * ks].x, tr[2 * ks].y, tr[2 * ks + 1].x, tr[2 * ks + 1].y};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, bh[ks]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, bl[ks]), acc, 0, 0, 0);
      }
      // dk^T[d][key] of this (query tile, key tile) pair: lane = key col,
      // register r = d 32 dt + 8(r/4) + 4 hf + r%4
      float* dst = dk_part + ((size_t)qt * (qt + 1) / 2 + kt) * (32 * kKlDi) + col * kKlDi + 32 * dt + 4 * hf;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(dst + 8 * j) = make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
    }
  }
  // ---- per-row KL (waves 0 and 1) and dq (waves 0, 1)
  float klq = klacc + __shfl_xor(klacc, 32, 64);
  float* red = reinterpret_cast<float*>(smem + kKlRed);
  if (wave == 1 && hf == 0) red[col] = klq;
  barrier_lds();
  if (wave < 2 && q0 + col < n) {
    if (wave == 0 && hf == 0) kl_row[q0 + col] = klq + red[col];
    float* dst = dq + (size_t)(q0 + col) * kKlDi + 32 * dt + 4 * hf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = dqs[64 * j];
      *reinterpret_cast<float4*>(dst + 8 * j) =
          make_float4(v.x * grad_scale, v.y * grad_scale, v.z * grad_scale, v.w * grad_scale);
    }
  }
}

// dk[j] = grad_scale * sum over query tiles qt >= kt of the pair partials,
// in increasing qt (one workgroup per key tile kt).
__global__ __launch_bounds__(256) void kl_dk_reduce_kernel(const float* __restrict__ dk_part,
                                                           int n, float grad_scale,
                                                           float* __restrict__ dk) {
  const int kt = (int)blockIdx.x;
  const int ntiles = (n + 31) >> 5;
  const int e = (int)threadIdx.x * 8;   // 8 of the tile's 32 x 64 values
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
  // four query tiles' partials in flight per step, summed in query-tile order
  int qt = kt;
  for (; qt + 4 <= ntiles; qt += 4) {
    float4 x[4], y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t t = (size_t)(qt + u);
      const float4* src = reinterpret_cast<const float4*>(dk_part + (t * (t + 1) / 2 + kt) * (32 * kKlDi) + e);
      x[u] = src[0];
      y[u] = src[1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a.x += x[u].x; a.y += x[u].y; a.z += x[u].z; a.w += x[u].w;
      b.x += y[u].x; b.y += y[u].y; b.z += y[u].z; b.w += y[u].w;
    }
  }
  for (; qt < ntiles; ++qt) {
    const float4* src = reinterpret_cast<const float4*>(dk_part + ((size_t)qt * (qt + 1) / 2 + kt) * (32 * kKlDi) + e);
    const float4 x = src[0], y = src[1];
    a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
  }
  const int key = (kt << 5) + e / kKlDi;
  if (key >= n) return;
  float4* dst = reinterpret_cast<float4*>(dk + (size_t)key * kKlDi + e % kKlDi);
  dst[0] = make_float4(a.x * grad_scale, a.y * grad_scale, a.z * grad_scale, a.w * grad_scale);
  dst[1] = make_float4(b.x * grad_scale, b.y * grad_scale, b.z * grad_scale, b.w * grad_scale);
}

// loss = (1/n) sum_i kl_row[i], summed in a fixed order by one workgroup.
__global__ __launch_bounds__(256) void kl_loss_kernel(const float* __restrict__ kl_row, int n,
                                                      float* __restrict__ loss) {
  __shared__ double part[256];
  double s = 0.0;
  for (int i = (int)threadIdx.x; i < n; i += 256) s += (double)kl_row[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(part[0] / (double)n);
}

}  // namespace

bool kl_shape_supported(const LayerShape& s, int d_idx) {
  return s.dtype == kBF16 && s.d == kKlD && s.hkv == kKlHkv && s.hq == kKlHq && d_idx == kKlDi;
}

size_t kl_partial_bytes(int n) {
  const size_t nt = (size_t)(n + 31) / 32;
  return nt * (nt + 1) / 2 * 32 * kKlDi * sizeof(float);
}

hipError_t launch_kl_distill(const LayerShape& s, int d_idx, float idx_scale, const void* q,
                             const void* k, const void* q_idx, const void* k_idx,
                             const float* lse, const float* lse_t, float* kl_row, float* loss,
                             float* dq, float* dk, float* dk_part, hipStream_t stream) {
  if (!kl_shape_supported(s, d_idx)) return hipErrorInvalidValue;
  const int ntiles = (s.n + 31) / 32;
  const float grad_scale = idx_scale / (float)s.n;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kl_tile_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kKlLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kl_tile_kernel, dim3(ntiles), dim3(512), kKlLds, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_idx), lse,
                     lse_t, s.n, s.scale * kLog2e, idx_scale * kLog2e, kl_row, dq, dk_part,
                     grad_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kl_dk_reduce_kernel, dim3(ntiles), dim3(256), 0, stream, dk_part, s.n,
                     grad_scale, dk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (loss) {
    hipLaunchKernelGGL(kl_loss_kernel, dim3(1), dim3(256), 0, stream, kl_row, s.n, loss);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace amtk
