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
// Work decomposition (one workgroup = 32 consecutive query rows, one wave
// per KV head g):
//   * wave g keeps the 32 x d query tiles of its G heads in VGPRs for the
//     whole launch (MFMA B operands, 16-byte chunks per lane);
//   * 32-row key tiles of KV head g stream through the wave's own LDS slots
//     by direct global->LDS loads (no VGPRs held) issued two tiles ahead in
//     pass 1 (two slots) and one tile ahead in pass 2, and are read back as
//     MFMA A operands;
//   * pass 1 interleaves each head's exp/sum work with the next head's
//     MFMAs inside the wave; in pass 2 the two waves of a SIMD overlap one
//     wave's MFMAs with the other's exponentials;
//   * the diagonal tile (causal mask) is peeled out of the main loop;
//   * pass 1 keeps an online max / sum per (head, query) in registers;
//   * pass 2 turns logits into probabilities with pass 1's LSE, sums the G
//     heads in registers, and the Hkv partial sums meet in LDS (double
//     buffered, one barrier per key tile). Row owners then reduce their
//     rows' masses over the KV heads in a fixed order and filter them against
//     the row's bound, so row state needs no atomics. With 8 KV heads only
//     waves 0..3 own rows (8 each): waves 4..7, which share their SIMDs, go
//     on to the next key tile's MFMAs while the owners filter (a partial
//     buffer is rewritten two tiles later, after the next barrier); with
//     other head counts every wave owns 32/Hkv rows.
// Workgroups are issued longest-row first (causal load balance).
//
// Streaming filter (pass 2). Per query row, an LDS histogram over mass bins
// (exponent + 3 mantissa bits) counts the candidates kept so far. The bound
// bin b_tau only rises, and it always satisfies: at least k kept candidates
// lie in bins >= b_tau (or b_tau = 0). Every unit of the final top-k is
// therefore >= the bound when it is seen and is kept. Kept units are appended
// to the row's candidate pool in global memory; the select kernel then picks
// the exact top-k from the pool. Each row's pool is appended in increasing
// unit id, so the select kernel emits ascending ids without sorting. A pool
// that overflows its capacity is detected (the count keeps running) and the
// row is redone densely.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace amtk {

// Column-sum mode: tiles of per-wave key sums held in LDS before a fold.
constexpr int kCsRing = 32;


// Mass bins of the filter (kFBins, 8 per octave), u16 counts packed two
// per LDS word.
constexpr int kFBinWords = kFBins / 2;

__device__ __forceinline__ int filter_bin(float p) {
  const int b = (int)(__float_as_uint(p) >> kBinShift) - kFBinBase;
  return min(max(b, 0), kFBins - 1);
}

__device__ __forceinline__ int hist_count(const unsigned* words, int b) {
  return (int)((words[b >> 1] >> ((b & 1) * 16)) & 0xffffu);
}

// ------------------------------------------------------------------ pass 1
template <typename T, int D, int G>
__global__ __launch_bounds__(512) void pass1_lse_kernel(const T* __restrict__ Q,
                                                         const T* __restrict__ K,
                                                         float* __restrict__ lse, int n, int hkv,
                                                         float c, float tau,
                                                         int* __restrict__ zero_counter) {
  typedef KTile<T, D> KT;
  constexpr int NC = KT::kChunks;
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int g = wave;
  const int hq = hkv * G;
  const int ntiles = (n + 31) >> 5;
  const int qt = ntiles - 1 - (int)blockIdx.x;
  const int q0 = qt << 5;
  // two LDS slots per wave: key tile t+2 streams in while tile t is used
  unsigned char* slot0 = smem + (2 * wave) * KT::kBytes;
  unsigned char* slot1 = slot0 + KT::kBytes;
  if (blockIdx.x == 0 && threadIdx.x == 0 && zero_counter) *zero_counter = 0;

  uint4 qc[G][NC];
  load_q_tiles<T, D, G>(Q, min(q0 + col, n - 1), hq, g, lane, qc);
  wait_vmem_all();   // Q in registers before the DMA stream starts
  KLane<T, D> kl;
  kl.init(lane, hkv);
  kl.issue(K, n, hkv, g, 0, slot0);
  kl.issue(K, n, hkv, g, min(1, qt) << 5, slot1);
  float mrun[G], lrun[G];

  // exp/sum work of one head on its score tile (16 keys x 1 query per lane).
  // With a running maximum (kTrack) as in a streaming softmax; without it,
  // the lane's maximum over the first key tile stays the reference for the
  // rest of the row, which saves the per-element maximum. Terms far below
  // the reference underflow harmlessly next to its own weight of 1; a logit
  // more than ~127 (in log2 units) above it overflows the sum to infinity,
  // which the caller detects and redoes with a running maximum.
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
  // Each tile issues exactly NC DMA ops (the tile two ahead, clamped to the
  // diagonal), so waiting for <= NC in flight means tile kt has landed.
  auto tile = [&](int kt, auto diag_c, auto track_c) __attribute__((always_inline)) {
    uint4 kc[NC];
    unsigned char* slot = (kt & 1) ? slot1 : slot0;
    wait_vmem_below<NC>();
    kl.read(slot, kc);
    kl.issue(K, n, hkv, g, min(kt + 2, qt) << 5, slot);
    f32x16 a0, a1;
    score_tile<T, NC>(a0, kc, qc[0]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h + 1 < G) score_tile<T, NC>((h & 1) ? a0 : a1, kc, qc[h + 1]);
      stats((h & 1) ? a1 : a0, h, diag_c, track_c);
    }
    if constexpr (!decltype(diag_c)::value)
      interleave_mfma_valu<NC * ChunkMma<T>::kSteps, (G - 1) * NC * ChunkMma<T>::kSteps, 64 / (NC * ChunkMma<T>::kSteps)>();
  };
  using yes = std::true_type;
  using no = std::false_type;

  // Interleaved schedule for the fixed-reference tiles (bf16, even G): one
  // MFMA of the next head, then the exp/sum work of 16/NC elements of the
  // current head, and so on, so one wave keeps the matrix core and the VALU
  // busy together (left alone, the compiler issues the MFMAs in bursts that
  // stall the wave). The order is held by empty volatile asm statements
  // (which keep their program order): each one makes the next MFMA's key
  // operand and the next group's exponent arguments depend on the previous
  // group's sums. The statements tie the fma results, which are fresh
  // values, rather than elements of the score vector, which the compiler
  // would first copy out (one v_mov per element: tying the scores cost 5 %
  // of the pass). The sums are formed in the same order as in stats(), so
  // results match.
  constexpr bool kInterleave = std::is_same<T, bf16_t>::value && (G % 2 == 0);
  constexpr int kEpg = 16 / NC;   // elements of the current head per MFMA
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
      if constexpr (kEpg == 2)
        asm volatile("" : "+v"(kv), "+v"(x[0]), "+v"(x[1]) : "v"(s0), "v"(s1));
      else
        asm volatile("" : "+v"(kv), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]) : "v"(s0), "v"(s1));
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
  // exp/sum work of one head with no MFMA beside it (fixed reference)
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
  // key tile kt lands in registers (DMA accounting as in tile())
  auto load_tile = [&](int kt, uint4 (&kk)[NC]) __attribute__((always_inline)) {
    unsigned char* slot = (kt & 1) ? slot1 : slot0;
    wait_vmem_below<NC>();
    // the previous MFMAs read their key operands at issue; keep a margin
    // before the LDS read overwrites those registers
    asm volatile("s_nop 15" ::: "memory");
    kl.read(slot, kk);
    kl.issue(K, n, hkv, g, min(kt + 2, qt) << 5, slot);
  };
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mrun[h] = kNegBig;
      lrun[h] = 0.f;
    }
  };
  // One pass over the row's key tiles (tiles 0 and 1 are already in flight):
  // tile 0 sets the reference, tiles 1 .. qt-1 use it (interleaved schedule
  // where available), then the diagonal tile.
  reset();
  if (qt == 0) {
    tile(0, yes{}, yes{});
  } else {
    tile(0, no{}, yes{});
    if constexpr (kInterleave) {
      if (qt >= 2) {
        uint4 kc[NC];
        f32x16 a0, a1;
        load_tile(1, kc);
        score_tile<T, NC>(a0, kc, qc[0]);
        for (int kt = 1; kt < qt; ++kt) {
          const bool more = kt + 1 < qt;   // the next tile is interleaved too
          // head h beside head h+1 (G even: head h's scores are in a0 for
          // even h, a1 for odd h); the last head beside the next tile's head 0
#pragma unroll
          for (int h = 0; h < G; ++h) {
            f32x16& cur = (h & 1) ? a1 : a0;
            f32x16& nxt = (h & 1) ? a0 : a1;
            if (h + 1 < G) {
              step(nxt, kc, qc[h + 1], cur, h);
            } else if (more) {
              load_tile(kt + 1, kc);
              step(nxt, kc, qc[0], cur, h);
            } else {
              tail(cur, h);
            }
          }
        }
      }
    } else {
      for (int kt = 1; kt < qt; ++kt) tile(kt, no{}, no{});
    }
    tile(qt, yes{}, no{});
  }
  wait_vmem_all();   // the last (clamped) prefetch must land before the slots are reused
  bool over = false;
#pragma unroll
  for (int h = 0; h < G; ++h) over |= !(lrun[h] < INFINITY);
  if (__ballot(over)) {   // rare: redo the wave's rows with a running maximum
    kl.issue(K, n, hkv, g, 0, slot0);
    kl.issue(K, n, hkv, g, min(1, qt) << 5, slot1);
    reset();
    if (qt == 0) {
      tile(0, yes{}, yes{});
    } else {
      for (int kt = 0; kt < qt; ++kt) tile(kt, no{}, yes{});
      tile(qt, yes{}, yes{});
    }
    wait_vmem_all();
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mo = xor32f(mrun[h]), lo = xor32f(lrun[h]);
    const float m = fmaxf(mrun[h], mo);
    const float l = lrun[h] * fast_exp2((mrun[h] - m) * c) + lo * fast_exp2((mo - m) * c);
    if (hf == 0 && q0 + col < n) lse[(size_t)(g * G + h) * n + q0 + col] = m * tau + logf(l);
  }
}

// ------------------------------------------- pass 1, one head split by keys
// A single head (the head-collapsed indexer: Hq = Hkv = 1, d = 64) gives the
// kernel above one wave per 32-row tile: too few waves to fill a CU. Here
// kLseSplit waves share a tile, wave w taking key tiles w, w + kLseSplit, ...
// with its own running maximum (two LDS slots each, two tiles ahead); the
// waves' (max, sum) pairs meet in LDS at the end.
constexpr int kLseSplit = 4;

__global__ __launch_bounds__(64 * kLseSplit) void pass1_lse_split_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, float* __restrict__ lse, int n,
    float c, float tau, int* __restrict__ zero_counter) {
  typedef KTile<bf16_t, 64> KT;
  constexpr int NC = KT::kChunks;
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int ntiles = (n + 31) >> 5;
  const int qt = ntiles - 1 - (int)blockIdx.x;
  const int q0 = qt << 5;
  unsigned char* slot0 = smem + (2 * wave) * KT::kBytes;
  unsigned char* slot1 = slot0 + KT::kBytes;
  float* red = reinterpret_cast<float*>(smem + 2 * kLseSplit * KT::kBytes);   // [wave][m, l][32]
  if (blockIdx.x == 0 && threadIdx.x == 0 && zero_counter) *zero_counter = 0;

  uint4 qc[1][NC];
  load_q_tiles<bf16_t, 64, 1>(Q, min(q0 + col, n - 1), 1, 0, lane, qc);
  wait_vmem_all();   // Q in registers before the DMA stream starts
  KLane<bf16_t, 64> kl;
  kl.init(lane, 1);
  if (wave <= qt) kl.issue(K, n, 1, 0, wave << 5, slot0);
  if (wave + kLseSplit <= qt) kl.issue(K, n, 1, 0, (wave + kLseSplit) << 5, slot1);
  float m = kNegBig, l = 0.f;   // this lane's keys only (its half of each tile)
  int i = 0;
  for (int kt = wave; kt <= qt; kt += kLseSplit, ++i) {
    unsigned char* slot = (i & 1) ? slot1 : slot0;
    if (kt + kLseSplit <= qt) wait_vmem_below<NC>();   // the next tile's NC loads may fly on
    else wait_vmem_all();
    uint4 kc[NC];
    kl.read(slot, kc);
    if (kt + 2 * kLseSplit <= qt) kl.issue(K, n, 1, 0, (kt + 2 * kLseSplit) << 5, slot);
    f32x16 a;
    score_tile<bf16_t, NC>(a, kc, qc[0]);
    if (kt == qt) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, hf) > col) a[r] = -INFINITY;
    }
    float tmax = a[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, a[r]);
    const float mnew = fmaxf(m, tmax);
    const float mc = mnew * c;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      s0 += fast_exp2(fmaf(a[r], c, -mc));
      s1 += fast_exp2(fmaf(a[r + 1], c, -mc));
    }
    l = fmaf(l, fast_exp2((m - mnew) * c), s0 + s1);
    m = mnew;
  }
  wait_vmem_all();
  // the two halves of the wave, then the waves
  const float mo = xor32f(m), lo = xor32f(l);
  const float mh = fmaxf(m, mo);
  const float lh = l * fast_exp2((m - mh) * c) + lo * fast_exp2((mo - mh) * c);
  if (hf == 0) {
    red[(2 * wave) * 32 + col] = mh;
    red[(2 * wave + 1) * 32 + col] = lh;
  }
  __syncthreads();
  if (wave == 0 && hf == 0 && q0 + col < n) {
    float mm = red[col];
#pragma unroll
    for (int w = 1; w < kLseSplit; ++w) mm = fmaxf(mm, red[(2 * w) * 32 + col]);
    float ll = 0.f;
#pragma unroll
    for (int w = 0; w < kLseSplit; ++w)
      ll += red[(2 * w + 1) * 32 + col] * fast_exp2((red[(2 * w) * 32 + col] - mm) * c);
    lse[q0 + col] = mm * tau + logf(ll);
  }
}

// ------------------------------------------------------------------ pass 2
struct RowState {
  int cnt[32];    // candidates appended (keeps counting past the capacity)
  int seen[32];   // cnt already folded into cge
  int cge[32];    // candidates in bins >= btau
  int btau[32];   // current bound bin
};

// LDS add without return, as an explicit instruction: as a plain atomic the
// compiler would make it wait for every outstanding global load (vmcnt(0)),
// including the key tile streaming into LDS.
__device__ __forceinline__ void lds_add(unsigned* p, unsigned x) {
  asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(p)), "v"(x) : "memory");
}


// Raise the row's bound while more than k candidates lie strictly above it.
__device__ __forceinline__ void raise_bound(RowState& rs, const unsigned* words, int r,
                                            int budget) {
  const int fresh = rs.cnt[r] - rs.seen[r];
  rs.seen[r] = rs.cnt[r];
  int cg = rs.cge[r] + fresh;
  int bt = rs.btau[r];
  while (bt < kFBins - 1) {
    const int hb = hist_count(words, bt);
    if (cg - hb < budget) break;
    cg -= hb;
    ++bt;
  }
  rs.cge[r] = cg;
  rs.btau[r] = bt;
}

// The same on row state held in registers (cge = candidates in bins >= bt
// after cg, the count including this tile's appends; hb = the count of bin
// bt itself): every lane serving the row runs it, so all of them keep the
// same state. Called only when the bound must rise (cg - hb >= budget). The
// histogram words of the next 8 bins come in one batch of reads, as the
// bound rarely moves further; on return hb holds the count of the new bin.
__device__ __forceinline__ void raise_bound_regs(const unsigned* words, int budget, int cg,
                                                 int& cge, int& bt, int& hb_bt) {
  const int w0 = bt >> 1;
  unsigned wv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wv[j] = words[min(w0 + j, kFBinWords - 1)];
  // The walk moves from bin bt + t to bt + t + 1 while the candidates above
  // it still number at least k: cg - S_t >= budget, S_t the counts of bins
  // bt .. bt + t. S_t only grows, so the moves are a prefix and their number
  // is the number of t that pass; the words in hand cover bins bt .. bt + 6
  // (bt + 7 too when bt is even), so seven moves are counted without
  // branches and a longer walk (rare) continues in the loop below.
  const int odd = bt & 1;
  int cnt[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) cnt[h] = (int)((wv[h >> 1] >> ((h & 1) * 16)) & 0xffffu);
  int s = 0, sum = 0, moved = 0, hb = odd ? cnt[1] : cnt[0];
#pragma unroll
  for (int t = 0; t < 7; ++t) {
    const int c = odd ? cnt[t + 1] : cnt[t];   // bin bt + t
    sum += c;
    const bool step = bt + t < kFBins - 1 && cg - sum >= budget;   // (a prefix of t)
    s += step ? 1 : 0;
    moved += step ? c : 0;
    if (t < 6) hb = step ? (odd ? cnt[t + 2] : cnt[t + 1]) : hb;   // bin bt + s
  }
  cg -= moved;
  int b = bt + s;
  if (s == 7) {   // the walk goes on past the words in hand
    while (true) {
      hb = (int)((words[b >> 1] >> ((b & 1) * 16)) & 0xffffu);
      if (b >= kFBins - 1 || cg - hb < budget) break;
      cg -= hb;
      ++b;
    }
  }
  cge = cg;
  bt = b;
  hb_bt = hb;
}

// Partial-mass layout: element (register r, source lane) of KV head g's
// tile lives at word g*kPartHead + r*kPartPitch + lane. The pitch of 68
// words puts register r of lane l in bank (4r + l) mod 64, so the
// lane-major writes and the row-owner reads (one source lane, registers
// 0..7 across a row's lanes, four adjacent source lanes per wave) are
// bank-conflict free, and each write is one base plus a constant offset.
// A head's block of 17 x 64 words keeps the heads 64-word aligned for
// paired reads.
constexpr int kPartPitch = 68;
constexpr int kPartHead = 17 * 64;
__device__ __forceinline__ int part_index(int g, int r, int src_lane) {
  return g * kPartHead + r * kPartPitch + src_lane;
}

// The 8 KV heads' partial masses of a lane's two keys (LDS byte addresses a0,
// a1 of head 0), issued together with one wait: the owners of a tile run in
// step after the barrier, so nothing else hides a second round trip.
typedef __attribute__((ext_vector_type(2))) float f32x2;
__device__ __forceinline__ void read_partials_hk8(uint32_t a0, uint32_t a1, f32x2 (&v)[8]) {
  static_assert(kPartHead == 17 * 64, "head stride in 64-word units below");
  asm volatile(
      "ds_read2st64_b32 %0, %8 offset1:17\n\t"
      "ds_read2st64_b32 %1, %8 offset0:34 offset1:51\n\t"
      "ds_read2st64_b32 %2, %8 offset0:68 offset1:85\n\t"
      "ds_read2st64_b32 %3, %8 offset0:102 offset1:119\n\t"
      "ds_read2st64_b32 %4, %9 offset1:17\n\t"
      "ds_read2st64_b32 %5, %9 offset0:34 offset1:51\n\t"
      "ds_read2st64_b32 %6, %9 offset0:68 offset1:85\n\t"
      "ds_read2st64_b32 %7, %9 offset0:102 offset1:119\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(a0), "v"(a1)
      : "memory");
}

// The same for four keys (addresses a[0..3]), one wait.
__device__ __forceinline__ void read_partials_hk8x4(const uint32_t (&a)[4], f32x2 (&v)[16]) {
  asm volatile(
      "ds_read2st64_b32 %0, %16 offset1:17\n\t"
      "ds_read2st64_b32 %1, %16 offset0:34 offset1:51\n\t"
      "ds_read2st64_b32 %2, %16 offset0:68 offset1:85\n\t"
      "ds_read2st64_b32 %3, %16 offset0:102 offset1:119\n\t"
      "ds_read2st64_b32 %4, %17 offset1:17\n\t"
      "ds_read2st64_b32 %5, %17 offset0:34 offset1:51\n\t"
      "ds_read2st64_b32 %6, %17 offset0:68 offset1:85\n\t"
      "ds_read2st64_b32 %7, %17 offset0:102 offset1:119\n\t"
      "ds_read2st64_b32 %8, %18 offset1:17\n\t"
      "ds_read2st64_b32 %9, %18 offset0:34 offset1:51\n\t"
      "ds_read2st64_b32 %10, %18 offset0:68 offset1:85\n\t"
      "ds_read2st64_b32 %11, %18 offset0:102 offset1:119\n\t"
      "ds_read2st64_b32 %12, %19 offset1:17\n\t"
      "ds_read2st64_b32 %13, %19 offset0:34 offset1:51\n\t"
      "ds_read2st64_b32 %14, %19 offset0:68 offset1:85\n\t"
      "ds_read2st64_b32 %15, %19 offset0:102 offset1:119\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]),
        "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

// HK: the KV heads if fixed at 8, else 0. CS: instead of filtering each
// row, write the column sums of the mass over the tile's rows (selection
// blocks of consecutive queries share one support; KB = 1 only).
template <typename T, int D, int G, int KB, int HK, bool CS>
__global__ __launch_bounds__(512) void pass2_filter_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ lse, int n,
    int hkv_arg, float c, float inv_hq, int budget, uint2* __restrict__ cand, int cap,
    int* __restrict__ cand_count, int* __restrict__ row_bin, int* __restrict__ ovf_count,
    int* __restrict__ ovf_list, float* __restrict__ colsum, const uint4* __restrict__ kops) {
  static_assert(!CS || KB == 1, "column sums are per token");
  const int hkv = HK ? HK : hkv_arg;
  typedef KTile<T, D> KT;
  constexpr int NC = KT::kChunks;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned* hist = reinterpret_cast<unsigned*>(smem);                       // [32][kFBinWords]
  RowState& rs = *reinterpret_cast<RowState*>(hist + 32 * kFBinWords);
  float* part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(&rs) + sizeof(RowState));
  const int part_floats = (KB == 1) ? hkv * kPartHead : hkv * 32;        // one buffer
  // key slots start on a 1 KiB boundary (the key-tile swizzle needs slots
  // aligned to the row pitch)
  unsigned char* slots = smem + ((reinterpret_cast<unsigned char*>(part + 2 * part_floats) - smem + 1023) & ~(ptrdiff_t)1023);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int g = wave;
  const int hq = hkv * G;
  const int nthreads = hkv * 64;
  const int ntiles = (n + 31) >> 5;
  const int qt = ntiles - 1 - (int)blockIdx.x;
  const int q0 = qt << 5;
  const int qrow = min(q0 + col, n - 1);
  unsigned char* slot = slots + wave * KT::kBytes;

  KLane<T, D> kl;
  kl.init(lane, hkv);
  // kops (8 KV heads, bf16, d = 128, one support per query): every key tile
  // is already stored in MFMA operand order, and tile t+1 goes from memory
  // straight into the registers once tile t's last MFMAs have read them
  constexpr bool kDirect = HK == 8 && KB == 1 && !CS && std::is_same<T, bf16_t>::value && D == 128;
  const uint4* kop = kDirect ? kops + (size_t)g * ntiles * (NC * 64) + lane : nullptr;
  if constexpr (!kDirect) kl.issue(K, n, hkv, g, 0, slot);
  for (int t = threadIdx.x; t < 32 * kFBinWords; t += nthreads) hist[t] = 0u;
  if (threadIdx.x < 32) {
    rs.cnt[threadIdx.x] = 0;
    rs.seen[threadIdx.x] = 0;
    rs.cge[threadIdx.x] = 0;
    rs.btau[threadIdx.x] = 0;
  }
  uint4 qc[G][NC];
  load_q_tiles<T, D, G>(Q, qrow, hq, g, lane, qc);
  float bias[G];
#pragma unroll
  for (int h = 0; h < G; ++h) bias[h] = lse[(size_t)(g * G + h) * n + qrow] * kLog2e;

  // Row ownership: wave w owns query rows [w*qpw, (w+1)*qpw) of the tile;
  // lpq lanes serve one row, each with epl of its 32 keys.
  // With the KV heads fixed at 8 only waves 0..3 own rows (8 each, 8 lanes a
  // row, 4 keys a lane): waves 4..7, which share their SIMDs, run the next
  // tile's MFMAs while the owners filter.
  constexpr int kOwnerWaves = HK == 8 ? 4 : 0;
  const bool owner_wave = HK == 8 ? wave < kOwnerWaves : true;
  const int qpw = HK == 8 ? 8 : 32 / hkv, lpq = HK == 8 ? 8 : 2 * hkv, epl = HK == 8 ? 4 : 16 / hkv;
  const int own_n = owner_wave ? wave * qpw + lane / lpq : 0;   // tile-local row this lane serves
  const int own_j = lane % lpq;
  const int own_q = q0 + own_n;
  const bool own_ok = owner_wave && own_q < n;
  const unsigned long long grp_mask =
      (lpq == 64 ? ~0ull : ((1ull << lpq) - 1ull)) << ((lane / lpq) * lpq);
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  unsigned* own_hist = hist + own_n * kFBinWords;
  barrier_lds();

  uint4 kc[NC];
  f32x16 a0, a1;
  auto load_k = [&](int kt) {   // key tile kt is in the slot; start tile kt+1
    wait_vmem_all();
    kl.read(slot, kc);
    if (kt < qt) kl.issue(K, n, hkv, g, (kt + 1) << 5, slot);
  };
  // exp/sum work of head h on its scores `cur` into pacc (head 0 assigns)
  auto head_exps = [&](const f32x16& cur, int h, float (&pacc)[16]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(fmaf(cur[r], c, -bias[h]));
      pacc[r] = h == 0 ? e : pacc[r] + e;
    }
  };
  // bf16: the exp/sum work of head h runs beside the MFMAs of head h+1, one
  // MFMA per 16/NC elements, the order held by empty volatile asm statements
  // that tie each MFMA's key operand to the previous group's results (as in
  // pass 1). The per-element sums keep the head order, so results match.
  constexpr bool kInterleave = std::is_same<T, bf16_t>::value && G >= 2;
  constexpr int kEpg = 16 / NC;
  auto head_step = [&](f32x16& nxt, const uint4 (&qq)[NC], const f32x16& cur, int h,
                       float (&pacc)[16]) __attribute__((always_inline)) {
    nxt = f32x16{};
    float last = 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      float x[kEpg];
#pragma unroll
      for (int e = 0; e < kEpg; ++e) x[e] = fmaf(cur[cc * kEpg + e], c, -bias[h]);
      u32x4 kv = __builtin_bit_cast(u32x4, kc[cc]);
      if constexpr (kEpg == 2)
        asm volatile("" : "+v"(kv), "+v"(x[0]), "+v"(x[1]) : "v"(last));
      else
        asm volatile("" : "+v"(kv), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]) : "v"(last));
      kc[cc] = __builtin_bit_cast(uint4, kv);
      ChunkMma<T>::mma(nxt, kc[cc], qq[cc]);
#pragma unroll
      for (int e = 0; e < kEpg; ++e) {
        const int r = cc * kEpg + e;
        const float ev = fast_exp2(x[e]);
        pacc[r] = h == 0 ? ev : pacc[r] + ev;
      }
      last = pacc[cc * kEpg + kEpg - 1];
    }
  };
  // head-summed probabilities of the current key tile for this lane's query
  // (head 0's scores are already in a0)
  auto load_direct = [&](int kt) __attribute__((always_inline)) {
    const uint4* src = kop + (size_t)kt * (NC * 64);
#pragma unroll
    for (int c = 0; c < NC; ++c) kc[c] = src[64 * c];
  };
  // after_mfma runs once the tile's last MFMA has been issued (key tile free)
  auto tile_mass = [&](bool diag, float (&pacc)[16], auto after_mfma) {
    if constexpr (kInterleave) {
#pragma unroll
      for (int h = 0; h + 1 < G; ++h) head_step((h & 1) ? a0 : a1, qc[h + 1], (h & 1) ? a1 : a0, h, pacc);
      after_mfma();
      head_exps(((G - 1) & 1) ? a1 : a0, G - 1, pacc);
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (h > 0) score_tile<T, NC>(a0, kc, qc[h]);
        if (h == G - 1) after_mfma();   // (head 0's MFMAs ran before: G = 1 too)
        head_exps(a0, h, pacc);
      }
    }
    if (diag) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, hf) > col) pacc[r] = 0.f;
    }
  };
  float blk = 0.f;   // KB > 1: this query's mass over the current key block (this wave's heads)
  // KB = 1: the filter state of the row this lane serves, kept in registers
  // (the same in every lane of the row's group; written to rs at the end):
  // candidates appended, candidates in bins >= the bound bin, the bound bin
  // and the count of that bin itself
  int r_cnt = 0, r_cge = 0, r_bt = 0, r_hb = 0;
  if constexpr (kDirect) load_direct(0);
  if constexpr (kDirect) {
    // ---- 8 KV heads, bf16, d = 128, one support per query. Waves 0..3 own
    // 8 rows each; wave w + 4 (which shares wave w's SIMD) sums, after
    // producing tile t+1, the 8 KV heads' partial masses of tile t for
    // wave w's rows into a small LDS buffer, and wave w filters tile t from
    // those sums after the next barrier (a lag of one tile: partial
    // buffers are rewritten two tiles later, sum buffers two filters
    // later). The owners' filter, which the other waves wait for at every
    // barrier, then reads 4 sums per lane instead of 32 partial masses.
    float* const sums = part + 2 * part_floats;   // [2][4 owners][4 keys][64 lanes]
    const int ow = wave & 3;                        // the owner this wave serves or is
    const int s_n = ow * 8 + (lane >> 3), s_j = lane & 7;   // the owner's lane layout
    // LDS byte addresses as a per-tile uniform base plus a lane offset
    const uint32_t part_lds = lds_addr(part), sums_lds = lds_addr(sums);
    uint32_t hs_off[4];   // head 0's partial of keys 8e + s_j of row s_n, in a buffer
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int mo = e * 8 + s_j;
      const int r = ((mo >> 3) << 2) | (mo & 3), h2 = (mo >> 2) & 1;
      hs_off[e] = 4u * (uint32_t)part_index(0, r, s_n + 32 * h2);
    }
    const uint32_t sum_off = 4u * (uint32_t)(ow * 256 + lane);
    auto produce = [&](int kt) __attribute__((always_inline)) {
      score_tile<T, NC>(a0, kc, qc[0]);
      float pacc[16];
      tile_mass(kt == qt, pacc, [&]() __attribute__((always_inline)) {
        if (kt < qt) load_direct(kt + 1);
      });
      const int wb = (kt & 1) * part_floats + part_index(g, 0, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) part[wb + kPartPitch * r] = pacc[r];
    };
    // the mass of keys 8e + s_j of row s_n of tile ft: the 8 KV heads'
    // partial masses summed in order 0..7, times 1/hq
    auto head_sums = [&](int ft) __attribute__((always_inline)) {
      const uint32_t pb = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(part_lds + (uint32_t)((ft & 1) * part_floats * 4)));
      float* sb = sums + (ft & 1) * 1024 + ow * 256 + lane;
      // the four keys' partials in one round trip
      const uint32_t ad[4] = {pb + hs_off[0], pb + hs_off[1], pb + hs_off[2], pb + hs_off[3]};
      f32x2 v[16];
      read_partials_hk8x4(ad, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = v[4 * e].x;
        p += v[4 * e].y;
#pragma unroll
        for (int j = 1; j < 4; ++j) {
          p += v[4 * e + j].x;
          p += v[4 * e + j].y;
        }
        sb[64 * e] = p * inv_hq;
      }
    };
    // the owner's filter of tile ft (see the generic loop below)
    auto filter = [&](int ft) __attribute__((always_inline)) {
      // the owners' filter is a latency-bound chain that the other waves
      // wait for at the next barrier: it gets the SIMD's issue slots first
      __builtin_amdgcn_s_setprio(2);
      const int k0 = ft << 5;
      const bool diag = ft == qt;
      const float* sb = sums + (ft & 1) * 1024 + ow * 256 + lane;
      float pm[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pm[e] = sb[64 * e];
      const int pos0 = r_cnt;
      const unsigned thr = filter_bin_floor_bits(r_bt);
      const bool live = own_ok && pos0 <= cap;
      // the four keys' tests, ranks and bins first (independent of each
      // other), then the pool stores and histogram adds: each under one flat
      // condition, in key order
      const int lim = diag ? own_q - k0 - own_j : 31;   // key 8e + own_j is causal iff 8e <= lim
      bool fl[4];
      unsigned long long mk[4];
      int bn[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        fl[e] = own_ok && __float_as_uint(pm[e]) >= thr && 8 * e <= lim;
        mk[e] = __ballot(fl[e]) & grp_mask;
        bn[e] = filter_bin(pm[e]);
      }
      int pos = pos0, in_bt = 0, at[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        at[e] = pos + __popcll(mk[e] & below);
        pos += __popcll(mk[e]);
        in_bt += __popcll(__ballot(fl[e] && bn[e] == r_bt) & grp_mask);
      }
      uint2* const row_pool = cand + (size_t)own_q * cap;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (fl[e] && at[e] < cap)
          row_pool[at[e]] = make_uint2(__float_as_uint(pm[e]), (unsigned)(k0 + e * 8 + own_j));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (fl[e] && live) lds_add(&own_hist[bn[e] >> 1], 1u << ((bn[e] & 1) * 16));
      if (pos != pos0) {
        const int cg = r_cge + (pos - pos0);
        r_cnt = pos;
        if (pos <= cap) {
          r_hb += in_bt;
          if (r_bt < kFBins - 1 && cg - r_hb >= budget) raise_bound_regs(own_hist, budget, cg, r_cge, r_bt, r_hb);
          else r_cge = cg;
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    for (int kt = 0; kt <= qt; ++kt) {
      produce(kt);
      if (!owner_wave && kt > 0) head_sums(kt - 1);
      barrier_lds();   // partial masses of tile kt, sums of tile kt - 1 visible
      if (owner_wave && kt > 0) filter(kt - 1);
    }
    if (!owner_wave) head_sums(qt);
    barrier_lds();     // sums of the last tile
    if (owner_wave) filter(qt);
  } else
  for (int kt = 0; kt <= qt; ++kt) {
    const int k0 = kt << 5;
    const bool diag = kt == qt;
    if constexpr (!kDirect) load_k(kt);
    score_tile<T, NC>(a0, kc, qc[0]);
    float pacc[16];
    tile_mass(diag, pacc, [&]() __attribute__((always_inline)) {
      if constexpr (kDirect) {
        if (kt < qt) load_direct(kt + 1);
      }
    });

    if constexpr (CS) {
      // ---- column sums: each wave sums its heads' masses over the tile's
      // rows in registers (a reduce-scatter over the 32 query lanes of each
      // half: one xor-16 exchange, then DPP row mirror, half mirror, xor 2,
      // xor 1), leaving the sum of key 16 b4 + 8 b3 + 4 hf + 2 b2 + b1 (lane
      // bits b) in lanes l and l^1; the 8 waves' sums go to an LDS ring of
      // kCsRing tiles that the workgroup folds (fixed order) and stores every
      // kCsRing tiles, so there is no barrier per tile.
      if (q0 + col >= n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] = 0.f;   // rows past n
      }
      const bool u16 = lane & 16, u8 = lane & 8, u4 = lane & 4, u2 = lane & 2;
      float v8[8], v4[4], v2[2];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v8[i] = (u16 ? pacc[i + 8] : pacc[i]) + __shfl_xor(u16 ? pacc[i] : pacc[i + 8], 16, 64);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v4[i] = (u8 ? v8[i + 4] : v8[i]) + dpp_f32<kDppRowMirror>(u8 ? v8[i] : v8[i + 4]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        v2[i] = (u4 ? v4[i + 2] : v4[i]) + dpp_f32<kDppRowHalfMirror>(u4 ? v4[i] : v4[i + 2]);
      float v1 = (u2 ? v2[1] : v2[0]) + dpp_f32<kDppQuadXor2>(u2 ? v2[0] : v2[1]);
      v1 += dpp_f32<kDppQuadXor1>(v1);
      const int slot = kt % kCsRing;
      if ((lane & 1) == 0) {
        const int key = 16 * (int)u16 + 8 * (int)u8 + 4 * hf + 2 * (int)u4 + (int)u2;
        part[(slot * hkv + g) * 32 + key] = v1;
      }
      if (slot == kCsRing - 1 || diag) {
        barrier_lds();   // the ring's tiles are complete
        const int kt0 = kt - slot;
        for (int e = (int)threadIdx.x; e < (slot + 1) * 32; e += nthreads) {
          const int sl = e >> 5, key = e & 31;
          const float* src = part + sl * hkv * 32 + key;
          float sum = src[0];
          for (int gg = 1; gg < hkv; ++gg) sum += src[gg * 32];
          const int j = ((kt0 + sl) << 5) + key;
          if (j < n) colsum[(size_t)qt * n + j] = sum * inv_hq;
        }
        barrier_lds();   // the ring is free again
      }
      continue;
    }
    if constexpr (KB == 1) {
      float* pb = part + (kt & 1) * part_floats;
      const int wb = (kt & 1) * part_floats + part_index(g, 0, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) part[wb + kPartPitch * r] = pacc[r];
      barrier_lds();   // partial masses visible
      if (!owner_wave) continue;   // (uniform per wave)
      // the owners' filter is a latency-bound chain that the other waves wait
      // for at the next barrier: it gets the SIMD's issue slots first
      if constexpr (HK == 8) __builtin_amdgcn_s_setprio(2);
      // ---- row owner: reduce over KV heads, filter, append, raise the bound
      // A mass passes the bound bin exactly when its bit pattern is at least
      // the bin's floor pattern, so the bin itself is only formed for the
      // histogram of appended entries.
      const int pos0 = r_cnt;
      const unsigned thr = filter_bin_floor_bits(r_bt);
      int pos = pos0;
      const bool live = own_ok && pos <= cap;
      // Lane j of a row's lane group takes the row's keys k0 + m with
      // m = e*lpq + j, so each ballot round appends in increasing key order
      // and, tile after tile, every row's pool is sorted by key. Key offset m
      // sits in accumulator register r = 4*(m/8) + m%4 of lane half (m/4)%2.
      // mass of the lane's key offset e*lpq + own_j, summed over the KV
      // heads in a fixed order
      auto mass = [&](int e) -> float {
        const int mo = e * lpq + own_j;
        const int r = ((mo >> 3) << 2) | (mo & 3), h2 = (mo >> 2) & 1;
        const float* src = pb + part_index(0, r, own_n + 32 * h2);
        float p = src[0];
        if constexpr (HK == 8) {
#pragma unroll
          for (int gg = 1; gg < 8; ++gg) p += src[gg * kPartHead];
        } else {
          for (int gg = 1; gg < hkv; ++gg) p += src[gg * kPartHead];
        }
        return p * inv_hq;
      };
      // with the KV heads fixed at 8 both masses are read in one batch first
      float pm[4];
      if constexpr (HK == 8) {
        uint32_t ad[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int mo = e * lpq + own_j;
          const int r = ((mo >> 3) << 2) | (mo & 3), h2 = (mo >> 2) & 1;
          ad[e] = lds_addr(pb + part_index(0, r, own_n + 32 * h2));
        }
        f32x2 v[16];
        read_partials_hk8x4(ad, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) {   // heads in order 0..7, as mass() sums them
          float p = v[4 * e].x;
          p += v[4 * e].y;
#pragma unroll
          for (int j = 1; j < 4; ++j) {
            p += v[4 * e + j].x;
            p += v[4 * e + j].y;
          }
          pm[e] = p * inv_hq;
        }
      }
      int in_bt = 0;   // this tile's appends that fall in the bound's own bin
      for (int e = 0; e < epl; ++e) {
        const int mo = e * lpq + own_j;
        float p;
        if constexpr (HK == 8) p = pm[e];
        else p = mass(e);
        const unsigned bits = __float_as_uint(p);
        const int key = k0 + mo;
        const bool flag = own_ok && bits >= thr && (!diag || key <= own_q);
        const unsigned long long m = __ballot(flag) & grp_mask;
        const int bin = filter_bin(p);
        if (flag) {
          const int at = pos + __popcll(m & below);
          if (at < cap) cand[(size_t)own_q * cap + at] = make_uint2(bits, (unsigned)key);
          if (live) lds_add(&own_hist[bin >> 1], 1u << ((bin & 1) * 16));
        }
        in_bt += __popcll(__ballot(flag && bin == r_bt) & grp_mask);
        pos += __popcll(m);
      }
      // The bound can only rise after appends (the histogram is unchanged
      // otherwise), and only when more than k candidates lie above its own
      // bin; both counts are kept in registers, so the histogram is read
      // only when the bound moves. (uniform over the row's group; never for
      // rows past n)
      if (pos != pos0) {
        const int cg = r_cge + (pos - pos0);
        r_cnt = pos;
        if (pos <= cap) {
          r_hb += in_bt;
          if (r_bt < kFBins - 1 && cg - r_hb >= budget) raise_bound_regs(own_hist, budget, cg, r_cge, r_bt, r_hb);
          else r_cge = cg;
        }
      }
      if constexpr (HK == 8) __builtin_amdgcn_s_setprio(0);
    } else {
      // ---- key blocks of KB = 64 tokens = two key tiles
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ps += pacc[r];
      ps += xor32f(ps);
      blk += ps;
      if ((kt & 1) || diag) {
        const int b = kt >> 1;
        float* pb = part + (b & 1) * part_floats;
        if (hf == 0) pb[g * 32 + col] = blk;
        blk = 0.f;
        barrier_lds();
        if (own_j == 0 && own_ok) {
          float p = 0.f;
          for (int gg = 0; gg < hkv; ++gg) p += pb[gg * 32 + own_n];
          p *= inv_hq;
          const int bin = filter_bin(p);
          if (bin >= rs.btau[own_n]) {
            const int at = rs.cnt[own_n];
            if (at < cap) cand[(size_t)own_q * cap + at] = make_uint2(__float_as_uint(p), (unsigned)b);
            rs.cnt[own_n] = at + 1;
            if (at + 1 <= cap) {
              own_hist[bin >> 1] += 1u << ((bin & 1) * 16);
              raise_bound(rs, own_hist, own_n, budget);
            }
          }
        }
      }
    }
  }
  wait_vmem_all();
  if constexpr (CS) return;
  if constexpr (KB == 1) {
    if (owner_wave && own_j == 0) {
      rs.cnt[own_n] = r_cnt;
      rs.btau[own_n] = r_bt;
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

// Key tiles in MFMA operand order (hkv KV heads, bf16, d = 128): entry
// ((g * T + t) * 8 + c) * 64 + l is the 16-byte chunk c of lane l's operand
// of tile t of KV head g, i.e. K[32 t + l % 32][g][64 (l / 32) + 8 c ..]
// (rows past n repeat row n - 1), so a wave loads one tile as 8 fully
// contiguous 1 KiB reads.
__global__ __launch_bounds__(256) void key_operands_kernel(const bf16_t* __restrict__ K,
                                                           uint4* __restrict__ kops, int n,
                                                           int ntiles, int hkv) {
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (size_t)hkv * ntiles * 512) return;
  const int l = (int)(id & 63), c = (int)((id >> 6) & 7);
  const size_t gt = id >> 9;
  const int t = (int)(gt % (size_t)ntiles), g = (int)(gt / (size_t)ntiles);
  const int row = min(t * 32 + (l & 31), n - 1);
  kops[id] = *reinterpret_cast<const uint4*>(K + ((size_t)row * hkv + g) * 128 + 64 * (l >> 5) + 8 * c);
}

// ------------------------------------------------------------ dispatching
template <typename T, int D, int G>
static hipError_t run_pass1(const LayerShape& s, const void* q, const void* k, float* lse,
                            int* zero_counter, hipStream_t stream) {
  const int ntiles = (s.n + 31) / 32;
  const float tau = s.scale;
  const size_t lds = (size_t)2 * s.hkv * KTile<T, D>::kBytes;
  auto kern = pass1_lse_kernel<T, D, G>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(ntiles), dim3(64 * s.hkv), lds, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), lse, s.n, s.hkv,
                     tau * kLog2e, tau, zero_counter);
  return hipGetLastError();
}

// direct: key tiles straight into registers (no key slots), with the head
// sums' buffer of the 8-KV-head path
template <typename T, int D>
static size_t pass2_lds_bytes(int hkv, int key_block, bool direct = false) {
  size_t b = 32 * kFBinWords * sizeof(unsigned) + sizeof(RowState);
  b += 2 * ((key_block == 1) ? (size_t)hkv * kPartHead : (size_t)hkv * 32) * sizeof(float);
  if (direct) return b + 2 * 4 * 4 * 64 * sizeof(float);
  b = (b + 1023) & ~(size_t)1023;   // key slots on a 1 KiB boundary
  return b + (size_t)hkv * KTile<T, D>::kBytes;
}

size_t pass2_key_operand_bytes(const LayerShape& s, int key_block) {
  if (s.dtype != kBF16 || s.d != 128 || s.hkv != 8 || key_block != 1) return 0;
  return (size_t)((s.n + 31) / 32) * 32 * 8 * 128 * sizeof(bf16_t);
}

template <typename T, int D, int G, int KB>
static hipError_t run_pass2(const LayerShape& s, int budget, const void* q, const void* k,
                            const float* lse, const CandidatePool& pool, hipStream_t stream) {
  const int ntiles = (s.n + 31) / 32;
  const size_t lds = pass2_lds_bytes<T, D>(s.hkv, KB, pass2_key_operand_bytes(s, KB) != 0);
  auto kern = s.hkv == 8 ? pass2_filter_kernel<T, D, G, KB, 8, false>
                         : pass2_filter_kernel<T, D, G, KB, 0, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  uint4* kops = nullptr;
  if (pass2_key_operand_bytes(s, KB)) {   // the keys in operand order, for this call's K
    kops = static_cast<uint4*>(pool.kops);
    if (!kops) return hipErrorInvalidValue;
    const size_t total = (size_t)8 * ntiles * 512;
    if (!pool.kops_ready)
      hipLaunchKernelGGL(key_operands_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                         stream, static_cast<const bf16_t*>(k), kops, s.n, ntiles, 8);
  }
  hipLaunchKernelGGL(kern, dim3(ntiles), dim3(64 * s.hkv), lds, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), lse, s.n, s.hkv,
                     s.scale * kLog2e, 1.0f / (float)s.hq, budget, pool.cand, pool.cap, pool.count,
                     pool.bin, pool.ovf_count, pool.ovf_list, nullptr, kops);
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t run_pass2_colsum(const LayerShape& s, const void* q, const void* k,
                                   const float* lse, float* colsum, hipStream_t stream) {
  const int ntiles = (s.n + 31) / 32;
  const size_t lds = pass2_lds_bytes<T, D>(s.hkv, 1);
  auto kern = s.hkv == 8 ? pass2_filter_kernel<T, D, G, 1, 8, true>
                         : pass2_filter_kernel<T, D, G, 1, 0, true>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(ntiles), dim3(64 * s.hkv), lds, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), lse, s.n, s.hkv,
                     s.scale * kLog2e, 1.0f / (float)s.hq, 0, nullptr, 0, nullptr, nullptr, nullptr,
                     nullptr, colsum, nullptr);
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
  if (s.dtype != kBF16 && s.dtype != kF32) return false;
  // both passes' LDS (pass 1: two key slots per wave; pass 2: one slot per
  // wave, the histograms and the partial masses) within one CU's 160 KiB
  const size_t slot = (size_t)s.d * (s.dtype == kBF16 ? 2 : 4) * 32;   // KTile<T, D>::kBytes
  const size_t lds1 = 2 * (size_t)s.hkv * slot;
  const size_t lds2 = s.dtype == kBF16
                          ? (s.d == 64 ? pass2_lds_bytes<bf16_t, 64>(s.hkv, 1)
                                       : pass2_lds_bytes<bf16_t, 128>(s.hkv, 1))
                          : (s.d == 64 ? pass2_lds_bytes<float, 64>(s.hkv, 1)
                                       : pass2_lds_bytes<float, 128>(s.hkv, 1));
  return lds1 <= kLdsBytesPerCu && lds2 <= kLdsBytesPerCu;
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

#ifndef AMTK_P1_DIRECT
#define AMTK_P1_DIRECT 1
#endif

bool pass1_writes_kops(const LayerShape& s) {
  // the direct kernel's shapes: bf16, d = 128, 1, 2, 4 or 8 KV heads, 2 or 4
  // query heads per KV head
  if (!AMTK_P1_DIRECT || s.dtype != kBF16 || s.d != 128) return false;
  if (s.hkv != 1 && s.hkv != 2 && s.hkv != 4 && s.hkv != 8) return false;
  return s.hq == 2 * s.hkv || s.hq == 4 * s.hkv;
}

size_t pass1_key_operand_bytes(const LayerShape& s) {
  if (!pass1_writes_kops(s)) return 0;
  return (size_t)((s.n + 31) / 32) * 32 * s.hkv * 128 * sizeof(bf16_t);
}

hipError_t launch_pass1_lse_kops(const LayerShape& s, const void* q, const void* k, float* lse,
                                 int* zero_counter, void* kops, hipStream_t stream) {
  if (!kops || !pass1_writes_kops(s)) return launch_pass1_lse(s, q, k, lse, zero_counter, stream);
  const int ntiles = (s.n + 31) / 32;
  const size_t total = (size_t)s.hkv * ntiles * 512;
  hipLaunchKernelGGL(key_operands_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, static_cast<const bf16_t*>(k), static_cast<uint4*>(kops), s.n, ntiles,
                     s.hkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_pass1_direct(s, q, kops, lse, zero_counter, stream);
}

hipError_t launch_pass1_lse(const LayerShape& s, const void* q, const void* k, float* lse,
                            int* zero_counter, hipStream_t stream) {
  if (s.hq == 1 && s.hkv == 1 && s.d == 64 && s.dtype == kBF16) {   // one head: split by keys
    const int ntiles = (s.n + 31) / 32;
    const size_t lds = (size_t)2 * kLseSplit * KTile<bf16_t, 64>::kBytes + 2 * kLseSplit * 32 * sizeof(float);
    hipLaunchKernelGGL(pass1_lse_split_kernel, dim3(ntiles), dim3(64 * kLseSplit), lds, stream,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), lse, s.n,
                       s.scale * kLog2e, s.scale, zero_counter);
    return hipGetLastError();
  }
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

hipError_t launch_pass2_colsum(const LayerShape& s, const void* q, const void* k, const float* lse,
                               float* colsum, hipStream_t stream) {
  AMTK_PASS_DISPATCH(run_pass2_colsum, s, q, k, lse, colsum, stream);
}

hipError_t launch_pass2_filter(const LayerShape& s, int key_block, int budget, const void* q,
                               const void* k, const float* lse, const CandidatePool& pool,
                               hipStream_t stream) {
  AMTK_PASS_DISPATCH(run_pass2_kb, s, key_block, budget, q, k, lse, pool, stream);
}

}  // namespace amtk
