// KL-distillation loss of the head-collapsed indexer against the oracle's
// attention mass, with its gradients, streamed over the causal triangle; no
// N x N matrix, and no array of that size, is stored.
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
// kl_tile_kernel (bf16, d = 128, 4 query heads per KV head, 1, 2, 4 or 8 KV
// heads, d_idx = 64), query-major: one workgroup of 8 waves per 32-query
// tile, wave g < hkv = KV head g, key tiles streamed as in pass 2. Per key
// tile:
//  * every wave g < hkv scores its 4 heads (32x32x16 MFMAs), turns them into
//    probabilities with the dense LSE and sums them; the hkv partial tiles
//    meet in LDS and the workgroup assembles the teacher tile P[key][query];
//  * waves 0 and 1 compute the student tile t^T[key][query] (4 MFMAs),
//    Q and dS = Q - P in the score layout (lane = query), the KL terms of
//    half of the keys each, and accumulate dq^T[d][query] += k_idx^T dS^T for
//    their 32 of the 64 dimensions (A = k_idx columns by transposing LDS
//    reads, B = the lane's own dS); dS is split into bf16 hi + lo, so the
//    products keep about 16 significant bits.
// kl_dk_kernel (key-major, below) computes the key gradient per KV group,
// kl_dk_sum_kernel adds the 8 groups per key in a fixed order, and
// kl_loss_kernel takes the mean; every sum has a fixed order (deterministic).
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

// kKlHkv, kKlHq: the most KV / query heads (the LDS map is sized for them)
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

template <int HKV>
__global__ __launch_bounds__(512) void kl_tile_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ QI,
    const bf16_t* __restrict__ KI, const float* __restrict__ lse, const float* __restrict__ lse_t,
    int n, float inv_hq, float c, float ct, float* __restrict__ kl_row,
    float* __restrict__ dq, float grad_scale) {
  constexpr int hkv = HKV;
  extern __shared__ __align__(1024) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int g = wave;
  const bool teacher = g < hkv;   // (uniform per wave) KV head g exists
  const int hq = kKlG * hkv;
  const int ntiles = (n + 31) >> 5;
  const int qt = ntiles - 1 - (int)blockIdx.x;   // longest rows first
  const int q0 = qt << 5;
  const int qrow = min(q0 + col, n - 1);
  const uint32_t base = lds_addr(smem);
  float* part = reinterpret_cast<float*>(smem + kKlPart);
  float* ptile = reinterpret_cast<float*>(smem + kKlPTile);
  unsigned char* slot = smem + kKlSlots + wave * KlKT::kBytes;

  KLane<bf16_t, kKlD> kl;
  kl.init(lane, hkv);
  if (teacher) kl.issue(K, n, hkv, g, 0, slot);
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
  if (teacher) load_q_tiles<bf16_t, kKlD, kKlG>(Q, qrow, hq, g, lane, qc);
  // the tile's dense LSE (log2 units), read back per key tile
  float* biasl = reinterpret_cast<float*>(smem + kKlBias) + g * kKlG * 32 + col;
  if (teacher && hf == 0) {
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
  const int dt = wave & 1;   // the d tile of waves 0 and 1

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
    // ---- teacher: this wave's 4 heads, summed (waves of existing KV heads)
    if (teacher) {
      uint4 kc[kKlNc];
      wait_vmem_all();   // this wave's K tile (and k_idx piece) have landed
      kl.read(slot, kc);
      if (kt < qt) kl.issue(K, n, hkv, g, (kt + 1) << 5, slot);
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
    } else {
      wait_vmem_all();   // this wave's k_idx piece has landed
    }
    barrier_lds();   // partial tiles visible
    if (wave < 4 && kt < qt) issue_kidx(kt + 1);
    // ---- assemble P[key][query] = (1/Hq) sum over the hkv partial tiles
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = (int)threadIdx.x + 512 * u;
      const int key = e >> 5, qq = e & 31;
      const int r = ((key >> 3) << 2) | (key & 3), h2 = (key >> 2) & 1;
      const int src = (r * 64 + ((qq + 32 * h2) ^ (4 * r)));
      float p = part[src];
#pragma unroll
      for (int gg = 1; gg < hkv; ++gg) p += part[src + gg * 1024];
      ptile[key * kKlPitch + qq] = p * inv_hq;
    }
    barrier_lds();   // P visible
    if (wave >= 2) continue;

    // ---- student tile, dS = Q - P, and the gradient products
    const uint32_t kb = base + kKlKidx + 4096u * (unsigned)(kt & 1);
    const uint32_t qb = base + kKlQidx;
    const float* lse_tl = reinterpret_cast<const float*>(smem + kKlLseT);
    {
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
    }
  }
  // ---- per-row KL (waves 0 and 1) and dq (waves 0, 1)
  float klq = sum_xor<32>(klacc);
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

// ------------------------------------------------------ key gradient
// dL/dk_idx[j] = (tau_idx/N) sum_{i>=j} (Q_ij - P_ij) q_idx[i] is linear in
// the teacher's head sum, P_ij = (1/Hq) sum_g sum_{h in g} p_h(i,j), so it
// splits over the KV groups g:
//   dk[j] = (tau_idx/N) sum_g C_g[j],
//   C_0[j] = sum_i (Q_ij - S_0(i,j)/Hq) q_idx[i],  C_g[j] = -sum_i S_g(i,j)/Hq q_idx[i] (g > 0),
// with S_g(i,j) = sum of p_h(i,j) over the 4 query heads of group g. Each
// group's share needs only that group's K and Q heads, so no workgroup
// exchanges partial masses with another, and the per-group sums (8 x n x
// d_idx floats) are added per key in increasing g by kl_dk_sum_kernel.
//
// kl_dk_kernel: one workgroup of 8 waves per (256 keys, KV group g), wave w
// owning key tile kb*8 + w. Workgroups are numbered so that XCD g serves
// group g. A wave holds its key tile of K (KV head g) in registers as the MFMA
// B operand and walks the query tiles from its own key tile to the last; the
// workgroup streams each query tile's 4 query heads (32 rows x 256 B each),
// the tile's q_idx rows, dense LSE and student LSE into LDS once for all 8
// waves (double buffered, one barrier per query tile). Per query tile a wave:
//  * scores S[query][key] = Q_h K^T (32x32x16 MFMAs, A = query rows from LDS,
//    lane = key, register r = query acc_row(r)), turns each head into
//    probabilities with the dense LSE and sums the 4 heads in registers;
//  * (group 0) scores the student t[query][key] = q_idx k_idx^T and adds Q;
//  * accumulates C^T[d][key] += q_idx^T[d][query] v[query][key] for both
//    32-wide d tiles, with v = (Q -) S/Hq split into bf16 hi + lo and the
//    transposed q_idx operand read to match the score layout's query order.
constexpr int kDkWaves = 8;                          // key tiles per workgroup
constexpr unsigned kDkQ = 0;                         // 4 query heads x 8 KiB
constexpr unsigned kDkQidx = 4 * 8192;               // q_idx tile (4 KiB)
constexpr unsigned kDkLse = kDkQidx + 4096;          // dense LSE x log2e [4][32]
constexpr unsigned kDkLseT = kDkLse + 512;           // student LSE x log2e [32]
constexpr unsigned kDkBuf = 40960;                   // one query tile's buffer
constexpr unsigned kDkLds = 2 * kDkBuf;

// The 16 floats at a, a + 32, a + 64, a + 96 (four runs of 4; byte address
// a in LDS), in the order of a lane's score registers (query acc_row(r)),
// read in one asm block that waits for them.
__device__ __forceinline__ void lds_floats16(uint32_t a, float (&f)[16]) {
  uint4 x[4];
  lds_read4(a, a + 32, a + 64, a + 96, x[0], x[1], x[2], x[3]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[4 * j] = __uint_as_float(x[j].x);
    f[4 * j + 1] = __uint_as_float(x[j].y);
    f[4 * j + 2] = __uint_as_float(x[j].z);
    f[4 * j + 3] = __uint_as_float(x[j].w);
  }
}

// One 1 KiB piece (instruction c: rows 4c .. 4c+3) of a 32-row x 256-byte
// tile of head `head` of X [n][heads][128] (rows r0 ..), laid out as the key
// tiles of KLane: chunk j of row R at 16-byte position R*16 + (j ^ (R & 15)).
// Rows past n repeat row n-1.
__device__ __forceinline__ void dk_dma_piece(const bf16_t* X, int heads, int head, int r0, int n,
                                             int c, unsigned char* slot, int lane) {
  const int row = 4 * c + (lane >> 4);
  const int rr = min(r0 + row, n - 1);
  const unsigned char* src = reinterpret_cast<const unsigned char*>(X + ((size_t)rr * heads + head) * kKlD) +
                             16 * ((lane & 15) ^ (row & 15));
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(slot + 1024 * c), 16, 0, 0);
}

template <int HKV>
__global__ __launch_bounds__(512) void kl_dk_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ QI,
    const bf16_t* __restrict__ KI, const float* __restrict__ lse, const float* __restrict__ lse_t,
    int n, float inv_hq, float c, float ct, float* __restrict__ cpart) {
  constexpr int hkv = HKV;
  extern __shared__ __align__(1024) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int g = (int)(blockIdx.x % hkv);             // with 8 groups, XCD g serves group g
  const int kb = (int)(blockIdx.x / hkv);            // longest rows first
  const int hq = kKlG * hkv;
  const int ntiles = (n + 31) >> 5;
  const int kt = kb * kDkWaves + wave;               // this wave's key tile
  const int k0 = kt << 5;
  const int qfirst = kb * kDkWaves;                  // first query tile the workgroup visits
  const uint32_t base = lds_addr(smem);

  // ---- the wave's key tile of K (B operand) through a temporary LDS slot
  uint4 kc[kKlNc];
  {
    KLane<bf16_t, kKlD> kl;
    kl.init(lane, hkv);
    unsigned char* tmp = smem + 8192u * (unsigned)wave;
    kl.issue(K, n, hkv, g, min(k0, ((n - 1) >> 5) << 5), tmp);
    wait_vmem_all();
    kl.read(tmp, kc);
  }
  // the key tile's k_idx rows (B operand of the student scores, group 0):
  // lane (key col, half hf) holds d = 16 s + 8 hf + [0, 8) for s = 0..3
  uint4 kif[4];
  {
    const int krow = min(k0 + col, n - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kif[s] = *reinterpret_cast<const uint4*>(KI + (size_t)krow * kKlDi + 16 * s + 8 * hf);
  }
  barrier_lds();   // temporary slots free

  // ---- streaming of query tiles (work split over the waves):
  //  waves 0-7: 4 pieces each of the 4 heads' Q tiles (wave w: head w/2,
  //             pieces 4(w%2) .. 4(w%2)+3);
  //  waves 0-3: 8 q_idx rows each; wave 4: dense LSE; wave 5: student LSE
  //             (both through registers, scaled by log2 e, written to LDS
  //             before the next barrier).
  const unsigned drow = 8u * (unsigned)wave + ((unsigned)lane >> 3);
  const unsigned dpiece = 16u * (((unsigned)lane & 7u) ^ idx_swizzle(drow));
  float lse_reg[2] = {0.f, 0.f};
  auto issue_tile = [&](int qt) {
    unsigned char* buf = smem + kDkBuf * (unsigned)(qt & 1);
    const int q0 = qt << 5;
    const int hh = wave >> 1;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      dk_dma_piece(Q, hq, g * kKlG + hh, q0, n, 4 * (wave & 1) + p, buf + kDkQ + 8192u * hh, lane);
    if (wave < 4) {
      const int row = min(q0 + (int)drow, n - 1);
      const unsigned char* src = reinterpret_cast<const unsigned char*>(QI) + (size_t)row * (kKlDi * 2) + dpiece;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(buf + kDkQidx + 1024u * wave), 16, 0, 0);
    }
    // every wave loads (only waves 4 and 5 publish): no branch merges the
    // loaded registers, which would make the compiler wait for all memory
    // (the DMA just issued included). Wave 4, lane l: heads (l >> 5) and
    // 2 + (l >> 5), query q0 + l % 32; wave 5: the student LSE.
    const int row = min(q0 + col, n - 1);
    lse_reg[0] = wave == 5 ? lse_t[row] : lse[(size_t)(g * kKlG + hf) * n + row];
    lse_reg[1] = lse[(size_t)(g * kKlG + 2 + hf) * n + row];
  };
  auto publish_regs = [&](int qt) {   // after this wave's loads of tile qt landed
    float* buf = reinterpret_cast<float*>(smem + kDkBuf * (unsigned)(qt & 1));
    if (wave == 4) {
      buf[kDkLse / 4 + 32 * hf + col] = lse_reg[0] * kLog2e;
      buf[kDkLse / 4 + 32 * (2 + hf) + col] = lse_reg[1] * kLog2e;
    } else if (wave == 5 && hf == 0) {
      buf[kDkLseT / 4 + col] = lse_reg[0] * kLog2e;
    }
  };

  // operand addresses in the index tiles (as in kl_tile_kernel)
  const unsigned fr = (unsigned)col;
  const uint32_t frag_off = 128u * fr + 16u * ((unsigned)hf ^ ((fr >> 2) & 1u)) + 32u * (fr & 3u);
  uint32_t tr_off;
  {
    const unsigned G16 = (unsigned)lane >> 4, e = ((unsigned)lane >> 2) & 3u, cc = (unsigned)lane & 3u;
    const unsigned u = 2u * (G16 & 1u) + (cc >> 1), sw = 2u * e + (G16 >> 1);
    tr_off = 128u * (4u * (G16 >> 1) + e) + 8u * (cc & 1u) + 16u * (u ^ sw);
  }
  KLane<bf16_t, kKlD> ql;   // read offsets of the Q tiles (same layout as key tiles)
  ql.init(lane, hq);

  f32x16 cacc[2] = {f32x16{}, f32x16{}};   // C^T[32 dt + acc_row][key col]
  const bool active_wave = kt < ntiles;
  const int key = k0 + col;

  issue_tile(qfirst);
  for (int qt = qfirst; qt < ntiles; ++qt) {
    // this wave's pieces and register loads of tile qt (the builtin, whose
    // wait the compiler accounts for)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    publish_regs(qt);
    barrier_lds();                   // tile qt complete; tile qt-1 no longer read
    if (qt + 1 < ntiles) issue_tile(qt + 1);
    if (!active_wave || qt < kt) continue;
    const unsigned char* buf = smem + kDkBuf * (unsigned)(qt & 1);
    const float* lsel = reinterpret_cast<const float*>(buf + kDkLse);
    const float* lsetl = reinterpret_cast<const float*>(buf + kDkLseT);
    const int q0 = qt << 5;
    // ---- teacher: the group's 4 heads, summed
    float psum[16];
#pragma unroll
    for (int h = 0; h < kKlG; ++h) {
      uint4 qc[kKlNc];
      ql.read(buf + kDkQ + 8192u * h, qc);
      f32x16 a;
      score_tile<bf16_t, kKlNc>(a, qc, kc);   // S[query][key]: lane = key, r = query
      // (as asm reads that wait for LDS only: the compiler would otherwise
      // wait for the next query tile's DMA before reading this buffer)
      float bias[16];
      lds_floats16(lds_addr(lsel + 32 * h + 4 * hf), bias);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(a[r], c, -bias[r]));
        psum[r] = h == 0 ? e : psum[r] + e;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- v = (Q -) S/Hq on the live pairs (key <= query < n)
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = -psum[r] * inv_hq;
    const uint32_t qb = base + kDkBuf * (unsigned)(qt & 1) + kDkQidx;
    if (g == 0) {
      f32x16 t = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 qf;
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(qf) : "v"((qb + frag_off) ^ (32u * s)) : "memory");
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qf),
                                                    __builtin_bit_cast(bf16x8, kif[s]), t, 0, 0, 0);
      }
      float bt[16];
      lds_floats16(lds_addr(lsetl + 4 * hf), bt);
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] += fast_exp2(fmaf(t[r], ct, -bt[r]));
    }
    u32x4 bh[2], bl[2];
#pragma unroll
    for (int r2 = 0; r2 < 16; r2 += 2) {
      float dsv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = r2 + u, qq = q0 + acc_row(r, hf);
        dsv[u] = (qq < n && key <= qq) ? v[r] : 0.f;
      }
      const unsigned h = pack2_bf16(dsv[0], dsv[1]);
      bh[r2 >> 3][(r2 & 7) >> 1] = h;
      bl[r2 >> 3][(r2 & 7) >> 1] =
          pack2_bf16(dsv[0] - __uint_as_float(h << 16), dsv[1] - __uint_as_float(h & 0xffff0000u));
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      u32x2 tr[4];
      read_idx_tr((qb + tr_off) ^ (64u * (unsigned)dt), tr);   // q_idx^T, rows = queries
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 av = {tr[2 * ks].x, tr[2 * ks].y, tr[2 * ks + 1].x, tr[2 * ks + 1].y};
        cacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                           __builtin_bit_cast(bf16x8, bh[ks]), cacc[dt], 0, 0, 0);
        cacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                           __builtin_bit_cast(bf16x8, bl[ks]), cacc[dt], 0, 0, 0);
      }
    }
  }
  // ---- this group's C[key][d] for the wave's key tile
  if (active_wave && key < n) {
    float* dst = cpart + ((size_t)g * n + key) * kKlDi + 4 * hf;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * j) =
            make_float4(cacc[dt][4 * j], cacc[dt][4 * j + 1], cacc[dt][4 * j + 2], cacc[dt][4 * j + 3]);
  }
}

// dk[j][d] = grad_scale * sum over the hkv KV groups of C_g[j][d], in
// increasing g.
template <int HKV>
__global__ __launch_bounds__(256) void kl_dk_sum_kernel(const float* __restrict__ cpart, int n,
                                                        float grad_scale, float* __restrict__ dk) {
  constexpr int hkv = HKV;
  const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;   // 4 values of dk
  const size_t total = (size_t)n * kKlDi;
  if (e >= total) return;
  float4 a = *reinterpret_cast<const float4*>(cpart + e);
#pragma unroll
  for (int g = 1; g < hkv; ++g) {
    const float4 x = *reinterpret_cast<const float4*>(cpart + (size_t)g * total + e);
    a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
  }
  *reinterpret_cast<float4*>(dk + e) =
      make_float4(a.x * grad_scale, a.y * grad_scale, a.z * grad_scale, a.w * grad_scale);
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
  const bool hkv_ok = s.hkv == 1 || s.hkv == 2 || s.hkv == 4 || s.hkv == kKlHkv;
  return s.dtype == kBF16 && s.d == kKlD && hkv_ok && s.hq == kKlG * s.hkv && d_idx == kKlDi;
}

size_t kl_partial_bytes(int n, int hkv) { return (size_t)hkv * (size_t)n * kKlDi * sizeof(float); }

template <int HKV>
static hipError_t run_kl_distill(const LayerShape& s, float idx_scale, const void* q,
                                 const void* k, const void* q_idx, const void* k_idx,
                                 const float* lse, const float* lse_t, float* kl_row, float* loss,
                                 float* dq, float* dk, float* dk_part, hipStream_t stream) {
  const int ntiles = (s.n + 31) / 32;
  const float grad_scale = idx_scale / (float)s.n;
  const float inv_hq = 1.0f / (float)s.hq;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kl_tile_kernel<HKV>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kKlLds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kl_dk_kernel<HKV>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDkLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kl_tile_kernel<HKV>, dim3(ntiles), dim3(512), kKlLds, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_idx), lse,
                     lse_t, s.n, inv_hq, s.scale * kLog2e, idx_scale * kLog2e, kl_row, dq,
                     grad_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int kblocks = (ntiles + kDkWaves - 1) / kDkWaves;
  hipLaunchKernelGGL(kl_dk_kernel<HKV>, dim3(kblocks * HKV), dim3(512), kDkLds, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_idx), lse,
                     lse_t, s.n, inv_hq, s.scale * kLog2e, idx_scale * kLog2e, dk_part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t quads = ((size_t)s.n * kKlDi + 3) / 4;
  hipLaunchKernelGGL(kl_dk_sum_kernel<HKV>, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                     stream, dk_part, s.n, grad_scale, dk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (loss) {
    hipLaunchKernelGGL(kl_loss_kernel, dim3(1), dim3(256), 0, stream, kl_row, s.n, loss);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_kl_distill(const LayerShape& s, int d_idx, float idx_scale, const void* q,
                             const void* k, const void* q_idx, const void* k_idx,
                             const float* lse, const float* lse_t, float* kl_row, float* loss,
                             float* dq, float* dk, float* dk_part, hipStream_t stream) {
  if (!kl_shape_supported(s, d_idx)) return hipErrorInvalidValue;
#define AMTK_KL(H) \
  run_kl_distill<H>(s, idx_scale, q, k, q_idx, k_idx, lse, lse_t, kl_row, loss, dq, dk, dk_part, stream)
  switch (s.hkv) {
    case 1: return AMTK_KL(1);
    case 2: return AMTK_KL(2);
    case 4: return AMTK_KL(4);
    case 8: return AMTK_KL(8);
  }
#undef AMTK_KL
  return hipErrorInvalidValue;
}

}  // namespace amtk
