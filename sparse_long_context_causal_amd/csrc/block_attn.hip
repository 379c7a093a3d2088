// Attention of a selection block's queries on their shared support.
//
// Method: gist.science page on arXiv 2606.07703, "Technischer Bericht"
// section 2.1: with selection-block-shared granularity one support set is
// chosen for a block of 64 consecutive queries, which amortises the cost of
// the support over the block; each query's output is then recomputed on the
// shared keys it may see (j <= i), the softmax taken over those keys only.
// Gathering the block's keys once turns the sparse step into a dense
// attention tile over a gathered key set.
//
// bf16, d = 128, 8 KV heads x 4 query heads, blocks of 64 queries. One
// workgroup of 8 waves per (block, KV head g), numbered block-major with g
// fastest: workgroups go to the 8 XCDs round robin, so XCD g serves KV head g
// and its L2 holds that head's keys and values only. Wave w computes query
// head 4g + (w & 3) for the 32 queries i0 + 32(w >> 2) + [0, 32):
//  * the support is walked in chunks of 32 keys. The chunk's 256-byte key
//    and value rows of head g are brought into LDS by DMA
//    (global_load_lds_dwordx4, no registers), wave w taking rows 4w..4w+3,
//    double buffered. d-chunk x (8 elements) of row R sits at position
//    x ^ f(R), f(R) = 2(R & 3) + ((R >> 2) & 1), which keeps both read
//    patterns below free of bank conflicts;
//  * S^T[key][query] = K Q^T with 32x32x16 bf16 MFMAs: A = the key rows
//    (16-byte LDS reads), B = the wave's query fragment, held in registers
//    for the whole launch. Lane l owns query l%32 and the 16 keys
//    8(r/4) + 4(l/32) + r%4 of the chunk (register r);
//  * keys after the query, invalid ids and padding weigh 0. Online softmax
//    per query: one xor-32 shuffle for the chunk maximum, the output is
//    rescaled only when a maximum moved;
//  * O^T[d][query] += V^T P^T with 32x32x16 bf16 MFMAs. B = the lane's own
//    weights as they come out of the score layout (the MFMA's k index runs
//    over the chunk's keys in that order), A = value columns through the
//    transposing read ds_read_b64_tr_b16, which hands lane l the elements of
//    4 consecutive key rows at d = l%32. Each weight is split into
//    hi = bf16(p) and lo = bf16(p - hi), two MFMAs, so the weights keep
//    about 16 significant bits (|p - hi - lo| <= 2^-16 p).
#include "device_common.h"
#include "kernels.h"
#include "topk_core.h"

namespace amtk {

namespace {

constexpr int kBaD = 128, kBaHkv = 8, kBaG = 4, kBaHq = kBaHkv * kBaG;
constexpr int kBaRows = 64;                              // queries per selection block
constexpr int kBaWaves = 8;
constexpr unsigned kBaTile = 8192;                       // 32 rows of 256 bytes
constexpr unsigned kBaRowBytes = kBaHkv * kBaD * 2;      // one token, all KV heads
constexpr unsigned kBaIdsOff = 4 * kBaTile;              // after K0, K1, V0, V1
constexpr unsigned kBaLds = kBaIdsOff + 2 * 128;          // bytes of LDS a tile uses
constexpr int kBaWaitVm0 = 0x0F70;                       // s_waitcnt vmcnt(0)

typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ unsigned row_swizzle(unsigned r) { return ((r & 3u) << 1) | ((r >> 2) & 1u); }

// The chunk's key fragments (k-step s at ka[s & 3] (+128 for s >= 4)) and
// the ids of the lane's 16 keys (4 consecutive slots at ia + 32 j), one
// asm block that also waits for them.
__device__ __forceinline__ void read_keys(const uint32_t (&ka)[4], uint32_t ia, u32x4 (&kf)[8],
                                          i32x4 (&iv)[4]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b128 %4, %12 offset:128\n\t"
      "ds_read_b128 %5, %13 offset:128\n\t"
      "ds_read_b128 %6, %14 offset:128\n\t"
      "ds_read_b128 %7, %15 offset:128\n\t"
      "ds_read_b128 %8, %16\n\t"
      "ds_read_b128 %9, %16 offset:32\n\t"
      "ds_read_b128 %10, %16 offset:64\n\t"
      "ds_read_b128 %11, %16 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]),
        "=&v"(kf[6]), "=&v"(kf[7]), "=&v"(iv[0]), "=&v"(iv[1]), "=&v"(iv[2]), "=&v"(iv[3])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ia)
      : "memory");
}

// The chunk's value fragments: vt[4 dt + 2 ks + sec] = transposing read at
// va[dt] + 4096 ks + 2048 sec (keys 16 ks + 8 sec + 4(l/32) + [0, 4) at
// d = 32 dt + l%32). One asm block that also waits for them.
__device__ __forceinline__ void read_values(const uint32_t (&va)[4], u32x2 (&vt)[16]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %3, %16 offset:6144\n\t"
      "ds_read_b64_tr_b16 %4, %17\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %7, %17 offset:6144\n\t"
      "ds_read_b64_tr_b16 %8, %18\n\t"
      "ds_read_b64_tr_b16 %9, %18 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %11, %18 offset:6144\n\t"
      "ds_read_b64_tr_b16 %12, %19\n\t"
      "ds_read_b64_tr_b16 %13, %19 offset:2048\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vt[0]), "=&v"(vt[1]), "=&v"(vt[2]), "=&v"(vt[3]), "=&v"(vt[4]), "=&v"(vt[5]),
        "=&v"(vt[6]), "=&v"(vt[7]), "=&v"(vt[8]), "=&v"(vt[9]), "=&v"(vt[10]), "=&v"(vt[11]),
        "=&v"(vt[12]), "=&v"(vt[13]), "=&v"(vt[14]), "=&v"(vt[15])
      : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3])
      : "memory");
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// One (selection block, KV head g) tile: wave w computes query head
// 4g + (w & 3) for the queries i0 + 32(w >> 2) + [0, 32) over the support
// units ids[0 .. cnt) (tokens, or KB-token key blocks), ids in global memory.
// Every wave of the workgroup must call it with the same arguments; the
// caller separates two calls on the same LDS with a barrier.
template <int KB>
__device__ __forceinline__ void shared_attn_tile(
    unsigned char* __restrict__ smem, const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
    const bf16_t* __restrict__ V, const int32_t* __restrict__ ids, int cnt, int i0, int g,
    float* __restrict__ O, float* __restrict__ lse_out, int n, float c) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5;                       // half of the wave
  const int hh = kBaG * g + (w & 3);              // query head of this wave
  const int qrow = i0 + 32 * (w >> 2) + (lane & 31);
  const int qld = min(qrow, n - 1);
  const int total = cnt * KB;                     // support tokens (before the causal clip)
  const int nch = (total + 31) >> 5;
  const int nunits = (n + KB - 1) / KB;

  const uint32_t base = lds_addr(smem);
  // DMA: lane 16q + m of wave w brings piece m of row R = 4w + q, which holds
  // d-chunk m ^ f(R)
  const unsigned dq = (unsigned)lane >> 4, dm = (unsigned)lane & 15u;
  const unsigned drow = 4u * (unsigned)w + dq;
  const unsigned dx = 16u * (dm ^ row_swizzle(drow));
  const unsigned char* Kb = reinterpret_cast<const unsigned char*>(K) + g * (kBaD * 2) + dx;
  const unsigned char* Vb = reinterpret_cast<const unsigned char*>(V) + g * (kBaD * 2) + dx;
  const uint32_t dma_k = base + 1024u * (unsigned)w, dma_v = dma_k + 2 * kBaTile;
  // token of the lane's DMA row in chunk ch (-1: padding or an invalid id)
  auto fetch_id = [&](int ch) -> int {
    const int slot = 32 * ch + (int)drow;
    if (slot >= total) return -1;
    if constexpr (KB == 1) {
      return ids[slot];
    } else {
      const int b = ids[slot / KB];
      return (b >= 0 && b < nunits) ? b * KB + slot % KB : -1;
    }
  };
  // stage chunk ch: its ids (INT_MAX for padding and invalid ids) into the
  // ids buffer, then its key and value rows (row 0 stands in for an
  // invalid id: it weighs 0)
  auto stage = [&](int ch, int raw) {
    const bool ok = raw >= 0 && raw < n;
    const unsigned b = (unsigned)ch & 1u;
    if (dm == 0)
      reinterpret_cast<int*>(smem + kBaIdsOff + 128u * b)[drow] = ok ? raw : 0x7fffffff;
    const size_t off = (size_t)(ok ? raw : 0) * kBaRowBytes;
    __builtin_amdgcn_global_load_lds(Kb + off, (lds_ptr_t)(uintptr_t)(dma_k + kBaTile * b), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(Vb + off, (lds_ptr_t)(uintptr_t)(dma_v + kBaTile * b), 16, 0, 0);
  };
  // query fragment: B operand of k-step s, query lane%32, d = 16 s + 8 hl + [0, 8)
  u32x4 qf[8];
  {
    const bf16_t* qp = Q + ((size_t)qld * kBaHq + hh) * kBaD + 8 * hl;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qp + 16 * s);
  }
  // LDS read addresses (buffer 0). Keys: row R = lane%32, k-step s at
  // position (2s + hl) ^ f(R) = 2(s ^ (R & 3)) + (hl ^ ((R >> 2) & 1)).
  // Values: lane 16 G + 4 e + cc reads row 4(G >> 1) + e (+ 16 ks + 8 sec),
  // d 32 dt + 16(G & 1) + 4 cc + [0, 4).
  uint32_t ka[4], va[4], ia;
  {
    const unsigned R = (unsigned)lane & 31u;
    const unsigned ak = base + 256u * R + 16u * ((unsigned)hl ^ ((R >> 2) & 1u)) + 32u * (R & 3u);
#pragma unroll
    for (int s = 0; s < 4; ++s) ka[s] = ak ^ (32u * (unsigned)s);
    const unsigned G16 = (unsigned)lane >> 4, e = ((unsigned)lane >> 2) & 3u, cc = (unsigned)lane & 3u;
    const unsigned u = 2u * (G16 & 1u) + (cc >> 1);
    const unsigned sw = 2u * e + (G16 >> 1);
    const unsigned av = base + 2 * kBaTile + 256u * (4u * (G16 >> 1) + e) + 8u * (cc & 1u) + 16u * (u ^ sw);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) va[dt] = av ^ (64u * (unsigned)dt);
    ia = base + kBaIdsOff + 16u * (unsigned)hl;
  }

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  float mrun = kNegBig, lrun = 0.f;

  int raw = 0;
  if (nch > 0) {
    stage(0, fetch_id(0));
    if (nch > 1) raw = fetch_id(1);
  }
  for (int ch = 0; ch < nch; ++ch) {
    const unsigned boff = kBaTile * ((unsigned)ch & 1u);
    __builtin_amdgcn_s_waitcnt(kBaWaitVm0);   // this wave's loads of the chunk have landed
    __syncthreads();                          // and every wave's; the other buffer is free
    u32x4 kf[8];
    i32x4 iv[4];
    {
      const uint32_t kk[4] = {ka[0] + boff, ka[1] + boff, ka[2] + boff, ka[3] + boff};
      read_keys(kk, ia + 128u * ((unsigned)ch & 1u), kf, iv);
    }
    if (ch + 1 < nch) {
      stage(ch + 1, raw);
      if (ch + 2 < nch) raw = fetch_id(ch + 2);
    }
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[s]),
                                                   __builtin_bit_cast(bf16x8, qf[s]), st, 0, 0, 0);
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = iv[r >> 2][r & 3] <= qrow ? st[r] : -INFINITY;
    float smax = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) smax = fmaxf(smax, x[r]);
    smax = max_xor<32>(smax);
    const float mnew = fmaxf(mrun, smax * c);
    if (__ballot(mnew != mrun)) {   // a query's maximum moved: rescale
      const float alpha = mnew == mrun ? 1.0f : fast_exp2(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      mrun = mnew;
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(x[r], c, -mnew));
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ps += p[r];
    lrun += ps;
    // B operands: k-step ks = the lane's weights 8 ks .. 8 ks + 7, hi and lo
    u32x4 phi[2], plo[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = p[8 * ks + 2 * j], b = p[8 * ks + 2 * j + 1];
        const unsigned hi = pack_bf16(a, b);
        phi[ks][j] = hi;
        plo[ks][j] = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
      }
    }
    u32x2 vt[16];
    {
      const uint32_t vv[4] = {va[0] + boff, va[1] + boff, va[2] + boff, va[3] + boff};
      read_values(vv, vt);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x2 a0 = vt[4 * dt + 2 * ks], a1 = vt[4 * dt + 2 * ks + 1];
        const u32x4 av = {a0.x, a0.y, a1.x, a1.y};
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, phi[ks]), acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, plo[ks]), acc[dt], 0, 0, 0);
      }
    }
  }
  const float l = sum_xor<32>(lrun);
  if (qrow >= n) return;   // (no barrier follows inside the tile)
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  // O^T register r of tile dt: d = 32 dt + 8(r/4) + 4 hl + r%4
  float* op = O + ((size_t)qrow * kBaHq + hh) * kBaD + 4 * hl;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(op + 32 * dt + 8 * j) =
          make_float4(acc[dt][4 * j] * inv, acc[dt][4 * j + 1] * inv, acc[dt][4 * j + 2] * inv,
                      acc[dt][4 * j + 3] * inv);
  if (lse_out && hl == 0)
    lse_out[(size_t)hh * n + qrow] = l > 0.f ? (mrun + log2f(l)) * kLn2 : -INFINITY;
}


template <int KB>
__global__ __launch_bounds__(64 * kBaWaves) void shared_attn_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, float* __restrict__ O,
    float* __restrict__ lse_out, int n, int max_units, float c) {
  __shared__ __align__(256) unsigned char smem[kBaLds];
  const int t = (int)(blockIdx.x / kBaHkv), g = (int)(blockIdx.x % kBaHkv);
  const int i0 = t * kBaRows;
  const int cnt = min(max(count[i0], 0), max_units);
  shared_attn_tile<KB>(smem, Q, K, V, idx + (size_t)i0 * max_units, cnt, i0, g, O, lse_out, n, c);
}

// ---------------------------------------------------------------------------
// The indexer's selection-block-shared support, and its fused realisation.
// One workgroup (8 waves) per block of 64 queries:
//  1. scores: unit u (KB tokens) gets the mean over the block's rows of the
//     indexer mass P_idx_i(j) = exp(t_ij - LSE_idx(i)) summed over its keys
//     j <= i. Wave w takes the units u = w (mod 8); per 32-key tile,
//     S[query][key] = q_idx k_idx^T over the block's 64 queries is two
//     32x32x16 MFMA tiles (A = the block's q_idx rows, held in registers;
//     B = the tile's k_idx rows, loaded straight into registers), so lane l
//     owns key l%32 and sums its 32 query registers, one xor-32 shuffle adds
//     the other half, and a shuffle tree over the 32 keys gives the tile sum,
//     all in a fixed order; the unit scores go to LDS;
//  2. the block's top-k units with wg_topk, written (ascending) into the
//     index row of every query of the block, with count and scores;
//  3. fused realisation (kAttend): the block's attention tile for each KV
//     head in turn (shared_attn_tile), reading the ids it just wrote.
constexpr int kIxD = 64;             // indexer head dim
constexpr int kIxMaxUnits = 2048;    // units a block's score row holds in LDS
constexpr int kIxMaxK = 1024;        // winners held in LDS

struct IndexerLds {
  float score[kIxMaxUnits];
  int win_id[kIxMaxK];
  float win_m[kIxMaxK];
  TopkScratch<512> sc;
};

template <int KB, bool kAttend>
__global__ __launch_bounds__(512) void indexer_shared_kernel(
    const bf16_t* __restrict__ QI, const bf16_t* __restrict__ KI, const float* __restrict__ lse_idx,
    int n, int k, float ct, int32_t* __restrict__ idx, int32_t* __restrict__ count,
    float* __restrict__ mass, const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
    const bf16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ lse_out, float c) {
  static_assert(KB % 32 == 0, "units are whole 32-key tiles");
  __shared__ __align__(256) unsigned char tile_lds[kAttend ? kBaLds : 16];
  __shared__ IndexerLds ix;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int t = (int)blockIdx.x;
  const int i0 = t * kBaRows, i1 = min(i0 + kBaRows, n) - 1;
  const int nu = i1 / KB + 1;                  // units the block's last row sees
  const float inv_rows = 1.0f / (float)(i1 - i0 + 1);

  // ---- 1. unit scores
  {
    // A operands: the block's q_idx rows, query tile qt2 = 0, 1, k-step s
    u32x4 qa[2][4];
    float lse2[2][16];   // LSE_idx x log2e of the query in each accumulator register
#pragma unroll
    for (int qt2 = 0; qt2 < 2; ++qt2) {
      const int qr = min(i0 + 32 * qt2 + col, n - 1);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        qa[qt2][s] = *reinterpret_cast<const u32x4*>(QI + (size_t)qr * kIxD + 16 * s + 8 * hf);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qq = i0 + 32 * qt2 + 8 * (r >> 2) + 4 * hf + (r & 3);
        lse2[qt2][r] = qq < n ? lse_idx[qq] * kLog2e : INFINITY;   // rows past n weigh 0
      }
    }
    for (int u = w; u < nu; u += 8) {
      float usum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KB / 32; ++kt) {
        const int k0 = u * KB + 32 * kt;
        if (k0 > i1) break;
        const int key = k0 + col;
        const int kr = min(key, n - 1);
        u32x4 kb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          kb[s] = *reinterpret_cast<const u32x4*>(KI + (size_t)kr * kIxD + 16 * s + 8 * hf);
        float csum = 0.f;
#pragma unroll
        for (int qt2 = 0; qt2 < 2; ++qt2) {
          f32x16 acc = f32x16{};
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[qt2][s]),
                                                          __builtin_bit_cast(bf16x8, kb[s]), acc, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qq = i0 + 32 * qt2 + 8 * (r >> 2) + 4 * hf + (r & 3);
            const float p = fast_exp2(fmaf(acc[r], ct, -lse2[qt2][r]));
            csum += (key <= qq) ? p : 0.f;
          }
        }
        csum = sum_xor<32>(csum);   // the other half's queries
        // then the 32 keys: pairs at distance 1, 2, 4, 8 (DPP; once a group
        // holds equal values, its mirror image pairs it with the next group)
        // and 16
        csum += dpp_f32<kDppQuadXor1>(csum);
        csum += dpp_f32<kDppQuadXor2>(csum);
        csum += dpp_f32<kDppRowHalfMirror>(csum);
        csum += dpp_f32<kDppRowMirror>(csum);
        csum = sum_xor<16>(csum);
        usum += csum;
      }
      if (lane == 0) ix.score[u] = usum * inv_rows;
    }
  }
  __syncthreads();

  // ---- 2. the block's top-k units
  auto score = [&](int u) -> float { return ix.score[u]; };
  const int kk = wg_topk<512>(score, nu, k, ix.sc, ix.win_id, ix.win_m);
  for (int i = i0; i <= i1; ++i) {
    for (int p = tid; p < k; p += 512) {
      idx[(size_t)i * k + p] = p < kk ? ix.win_id[p] : -1;
      if (mass) mass[(size_t)i * k + p] = p < kk ? ix.win_m[p] : 0.f;
    }
    if (tid == 0) count[i] = kk;
  }

  // ---- 3. the attention of the block's queries on the shared units
  if constexpr (kAttend) {
    __syncthreads();   // the block's index row is written (and visible to the workgroup)
    for (int g = 0; g < kBaHkv; ++g) {
      shared_attn_tile<KB>(tile_lds, Q, K, V, idx + (size_t)i0 * k, kk, i0, g, O, lse_out, n, c);
      __syncthreads();   // the tile's LDS is free for the next head
    }
  }
}

}  // namespace

bool shared_attn_shape_supported(const LayerShape& s, int query_block) {
  return s.dtype == kBF16 && s.d == kBaD && s.hkv == kBaHkv && s.hq == kBaHq &&
         query_block == kBaRows;
}

hipError_t launch_shared_attn(const LayerShape& s, int key_block, int query_block, int max_units,
                              const void* q, const void* k, const void* v, const int32_t* idx,
                              const int32_t* count, float* o, float* lse_sparse,
                              hipStream_t stream) {
  if (!shared_attn_shape_supported(s, query_block) || (key_block != 1 && key_block != 64))
    return hipErrorInvalidValue;
  const unsigned nblk = (unsigned)((s.n + kBaRows - 1) / kBaRows);
  auto kern = key_block == 1 ? shared_attn_mfma_kernel<1> : shared_attn_mfma_kernel<64>;
  hipLaunchKernelGGL(kern, dim3(nblk * kBaHkv), dim3(64 * kBaWaves), 0, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), idx, count, o, lse_sparse, s.n, max_units,
                     s.scale * kLog2e);
  return hipGetLastError();
}

bool indexer_shared_supported(int n, int d_idx, int dtype, int key_block, int query_block,
                              int budget) {
  return dtype == kBF16 && d_idx == kIxD && key_block == 64 && query_block == kBaRows &&
         (n + key_block - 1) / key_block <= kIxMaxUnits && budget <= kIxMaxK;
}

hipError_t launch_indexer_shared(int n, int key_block, int budget, float idx_scale,
                                 const void* q_idx, const void* k_idx, const float* lse_idx,
                                 int32_t* idx, int32_t* count, float* mass,
                                 const LayerShape* attn, const void* q, const void* k,
                                 const void* v, float* o, float* lse_sparse, hipStream_t stream) {
  if (!indexer_shared_supported(n, kIxD, kBF16, key_block, kBaRows, budget))
    return hipErrorInvalidValue;
  const unsigned nblk = (unsigned)((n + kBaRows - 1) / kBaRows);
  const float ct = idx_scale * kLog2e;
  if (attn) {
    if (!shared_attn_shape_supported(*attn, kBaRows) || attn->n != n) return hipErrorInvalidValue;
    hipLaunchKernelGGL((indexer_shared_kernel<64, true>), dim3(nblk), dim3(512), 0, stream,
                       static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_idx),
                       lse_idx, n, budget, ct, idx, count, mass, static_cast<const bf16_t*>(q),
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), o, lse_sparse,
                       attn->scale * kLog2e);
  } else {
    hipLaunchKernelGGL((indexer_shared_kernel<64, false>), dim3(nblk), dim3(512), 0, stream,
                       static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_idx),
                       lse_idx, n, budget, ct, idx, count, mass, nullptr, nullptr, nullptr,
                       nullptr, nullptr, 0.f);
  }
  return hipGetLastError();
}

}  // namespace amtk
