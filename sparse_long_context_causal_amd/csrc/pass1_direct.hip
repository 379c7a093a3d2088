// Pass 1 (per-head row log-sum-exp) reading the key tiles from a copy in
// MFMA operand order (written by key_operands_kernel in passes.hip), for
// bf16, d = 128 and 2 or 4 query heads per KV head.
//
// Method: "How Much Dense Attention is Necessary? Oracle-Guided Sparse
// Prefill for Full/GQA Layers in Hybrid Long-Context Models" (arXiv
// 2606.07703), gist.science page, "Technischer Bericht" section 2.1: every
// head's full causal softmax over the keys j <= i; this pass forms its
// normaliser, LSE_h(i) = log sum_j exp(tau <q_h(i), k(j)>).
//
// This file is built with the MFMA results in vector registers
// (-mllvm -amdgpu-mfma-vgpr-form=1, set by build.py for this file only): the
// kernel runs one wave per SIMD and keeps its query tiles in the
// accumulation registers, and MFMA results there would each need a copy
// before the exponential work could read them.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace amtk {

// ------------------------------------- pass 1 from the operand-order keys
// bf16, d = 128, 2 or 4 query heads per KV head, with the key tiles already in
// MFMA operand order (key_operands_kernel). One wave per (32-row
// tile, KV head) and no LDS: key tiles come from memory straight into
// registers, a ring of kP1Ring tiles ahead of the one in use, which the
// registers of a wave alone on its SIMD allow (the kernel above, two waves
// per SIMD, has none to spare and reads each tile out of LDS with a wait).
// The arithmetic and its order are those of pass1_lse_kernel, so the LSEs
// are the same bit for bit.
#ifndef AMTK_P1_RING
#define AMTK_P1_RING 3
#endif
constexpr int kP1Ring = AMTK_P1_RING;
static_assert(kP1Ring == 2 || kP1Ring == 3, "ring of 2 or 3 key tiles");
template <int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void
pass1_lse_direct_kernel(const bf16_t* __restrict__ Q, const uint4* __restrict__ kops,
                        float* __restrict__ lse, int n, int hkv, float c, float tau,
                        int* __restrict__ zero_counter) {
  typedef bf16_t T;
  constexpr int D = 128, NC = KTile<T, D>::kChunks;
  static_assert(NC == 8, "8 chunks of 16 bytes per lane and key tile");
  static_assert(G == 2 || G == 4, "an even number of query heads per KV head (interleaved heads)");
  const int lane = threadIdx.x;
  const int hf = lane >> 5, col = lane & 31;
  const int ntiles = (n + 31) >> 5;
  const int qt = ntiles - 1 - (int)(blockIdx.x / (unsigned)hkv);   // longest rows first
  const int g = (int)(blockIdx.x % (unsigned)hkv);   // (8 KV heads: XCD g serves head g)
  // (the kernel takes the KV head count at run time: a power of two up to 8)
  const int q0 = qt << 5;
  const int hq = hkv * G;
  if (blockIdx.x == 0 && lane == 0 && zero_counter) *zero_counter = 0;

  uint4 qc[G][NC];
  load_q_tiles<T, D, G>(Q, min(q0 + col, n - 1), hq, g, lane, qc);
  // the query tiles are only ever MFMA operands: kept in the accumulation
  // registers, they leave the vector registers to the scores and the
  // exponential work (which cannot read accumulation registers)
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      u32x4 v = __builtin_bit_cast(u32x4, qc[h][cc]);
      asm volatile("" : "+a"(v));
      qc[h][cc] = __builtin_bit_cast(uint4, v);
    }
  const uint4* kop = kops + (size_t)g * ntiles * (NC * 64) + lane;
  // key tile t (clamped to the diagonal tile) into registers; the compiler
  // waits for each chunk where it is first used
  auto ldk = [&](int t, uint4 (&dst)[NC]) __attribute__((always_inline)) {
    const uint4* src = kop + (size_t)min(t, qt) * (NC * 64);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) dst[cc] = src[64 * cc];
  };
  float mrun[G], lrun[G];
  auto stats = [&](f32x16& acc, int h, auto diag_c, auto track_c) __attribute__((always_inline)) {
    if constexpr (decltype(diag_c)::value) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, hf) > col) acc[r] = -INFINITY;
    }
    if constexpr (decltype(track_c)::value) {
      float tmax = fmaxf(acc[0], acc[1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) tmax = fmaxf(tmax, acc[r]);
      const float mnew = fmaxf(mrun[h], tmax);
      const float mc = mnew * c;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        s0 += fast_exp2(fmaf(acc[r], c, -mc));
        s1 += fast_exp2(fmaf(acc[r + 1], c, -mc));
      }
      lrun[h] = fmaf(lrun[h], fast_exp2((mrun[h] - mnew) * c), s0 + s1);
      mrun[h] = mnew;
    } else {
      const float mc = mrun[h] * c;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        s0 += fast_exp2(fmaf(acc[r], c, -mc));
        s1 += fast_exp2(fmaf(acc[r + 1], c, -mc));
      }
      lrun[h] += s0 + s1;
    }
  };
  auto tile = [&](int kt, auto diag_c, auto track_c) __attribute__((always_inline)) {
    uint4 kc[NC];
    ldk(kt, kc);
    f32x16 a0, a1;
    score_tile<T, NC>(a0, kc, qc[0]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h + 1 < G) score_tile<T, NC>((h & 1) ? a0 : a1, kc, qc[h + 1]);
      stats((h & 1) ? a1 : a0, h, diag_c, track_c);
    }
  };
  using yes = std::true_type;
  using no = std::false_type;
  // head h's exp/sum work beside head h+1's MFMAs, in the order held by
  // empty volatile asm statements (as in pass1_lse_kernel)
  constexpr int kEpg = 16 / NC;
  auto step = [&](f32x16& nxt, uint4 (&kk)[NC], const uint4 (&qq)[NC], const f32x16& cur,
                  int h) __attribute__((always_inline)) {
    const float mc = mrun[h] * c;
    float s0 = 0.f, s1 = 0.f;
    nxt = f32x16{};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      float x[kEpg];
#pragma unroll
      for (int e = 0; e < kEpg; ++e) x[e] = fmaf(cur[cc * kEpg + e], c, -mc);
      u32x4 kv = __builtin_bit_cast(u32x4, kk[cc]);
      asm volatile("" : "+v"(kv), "+v"(x[0]), "+v"(x[1]) : "v"(s0), "v"(s1));
      kk[cc] = __builtin_bit_cast(uint4, kv);
      ChunkMma<T>::mma(nxt, kk[cc], qq[cc]);
#pragma unroll
      for (int e = 0; e < kEpg; ++e) {
        const int r = cc * kEpg + e;
        const float y = fast_exp2(x[e]);
        if (r & 1) s1 += y;
        else s0 += y;
      }
    }
    lrun[h] += s0 + s1;
  };
  auto tail = [&](const f32x16& cur, int h) __attribute__((always_inline)) {
    const float mc = mrun[h] * c;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      s0 += fast_exp2(fmaf(cur[r], c, -mc));
      s1 += fast_exp2(fmaf(cur[r + 1], c, -mc));
    }
    lrun[h] += s0 + s1;
  };
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mrun[h] = kNegBig;
      lrun[h] = 0.f;
    }
  };
  reset();
  if (qt == 0) {
    tile(0, yes{}, yes{});
  } else {
    tile(0, no{}, yes{});
    if (qt >= 2) {
      // ring: at the start of tile kt, b0 holds tile kt and b1 tile kt+1
      // (kP1Ring = 3: b2 tile kt+2), loaded or in flight; the buffer of tile
      // kt takes tile kt + kP1Ring once the MFMAs of its last head have been
      // issued
      uint4 b0[NC], b1[NC], b2[NC];
      ldk(1, b0);
      ldk(2, b1);
      if constexpr (kP1Ring == 3) ldk(3, b2);
      f32x16 a0, a1;
      score_tile<T, NC>(a0, b0, qc[0]);
      auto run = [&](int kt, uint4 (&cur)[NC], uint4 (&nxt)[NC]) __attribute__((always_inline)) {
        const bool more = kt + 1 < qt;   // the next tile is interleaved too
#pragma unroll
        for (int h = 0; h < G; ++h) {
          f32x16& ca = (h & 1) ? a1 : a0;
          f32x16& na = (h & 1) ? a0 : a1;
          if (h + 1 < G) {
            step(na, cur, qc[h + 1], ca, h);
            if (h + 2 == G) ldk(kt + kP1Ring, cur);
          } else if (more) {
            step(na, nxt, qc[0], ca, h);
          } else {
            tail(ca, h);
          }
        }
      };
      int kt = 1;
      if constexpr (kP1Ring == 3) {
        for (; kt + 2 < qt; kt += 3) {
          run(kt, b0, b1);
          run(kt + 1, b1, b2);
          run(kt + 2, b2, b0);
        }
        if (kt < qt) run(kt, b0, b1);
        if (kt + 1 < qt) run(kt + 1, b1, b2);
      } else {
        for (; kt + 1 < qt; kt += 2) {
          run(kt, b0, b1);
          run(kt + 1, b1, b0);
        }
        if (kt < qt) run(kt, b0, b1);
      }
    }
    tile(qt, yes{}, no{});
  }
  bool over = false;
#pragma unroll
  for (int h = 0; h < G; ++h) over |= !(lrun[h] < INFINITY);
  if (__ballot(over)) {   // rare: redo the wave's rows with a running maximum
    reset();
    if (qt == 0) {
      tile(0, yes{}, yes{});
    } else {
      for (int kt = 0; kt < qt; ++kt) tile(kt, no{}, yes{});
      tile(qt, yes{}, yes{});
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


hipError_t launch_pass1_direct(const LayerShape& s, const void* q, const void* kops, float* lse,
                               int* zero_counter, hipStream_t stream) {
  const int ntiles = (s.n + 31) / 32;
  auto kern = s.hq == 2 * s.hkv ? pass1_lse_direct_kernel<2> : pass1_lse_direct_kernel<4>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(ntiles * s.hkv)), dim3(64), 0, stream,
                     static_cast<const bf16_t*>(q), static_cast<const uint4*>(kops), lse, s.n,
                     s.hkv, s.scale * kLog2e, s.scale, zero_counter);
  return hipGetLastError();
}

}  // namespace amtk
