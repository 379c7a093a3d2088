// Device-side building blocks shared by the attention-mass kernels (gfx950).
//
// Score tiles are computed transposed, S^T[key][query], with one
// 32x32 MFMA tile per (head, 32 keys, 32 queries): the A operand holds key
// rows, the B operand query rows, so after the MFMA each lane owns ONE query
// (lane % 32) and 16 keys. Row-wise reductions over keys are then mostly
// lane-local, with one exchange between lanes l and l^32.
//
// Accumulator layout of a 32x32 MFMA on CDNA (16 floats per lane):
//   register r of lane l holds C[m][n] with n = l % 32 and
//   m = 8*(r/4) + 4*(l/32) + (r%4).
// The reduction dimension (head_dim) is split so that lane half hf = l/32
// feeds the contiguous half [hf*D/2, (hf+1)*D/2) of every row; A and B use
// the same split, so each MFMA sums the same d-slice of both operands.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace amtk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef uint16_t bf16_t;   // bf16 storage

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for running maxima

// ---------------------------------------------------------------- mass bins
// Positive fp32 values order like their bit patterns. A bin keeps the
// exponent and the top 3 mantissa bits (8 bins per octave) from 2^-64 up to
// 2^1; everything smaller shares bin 0.
constexpr int kBinShift = 20;
constexpr int kBinBase = (127 - 64) << 3;
constexpr int kNumBins = 65 * 8;

__device__ __forceinline__ int mass_bin(float p) {
  int b = (int)(__float_as_uint(p) >> kBinShift) - kBinBase;
  return min(max(b, 0), kNumBins - 1);
}

// Filter bins of the pass-2 streaming bound: 8 per octave from 2^-48 to
// 2^1 (everything smaller shares bin 0). Bin b > 0 starts at mass bit
// pattern (b + kFBinBase) << kBinShift.
constexpr int kFBinBase = (127 - 48) << 3;
constexpr int kFBins = 49 * 8;

__device__ __forceinline__ unsigned filter_bin_floor_bits(int b) {
  return b > 0 ? (unsigned)(b + kFBinBase) << kBinShift : 0u;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// ------------------------------------------------------------- MFMA operands
// One k-step of the 32x32 MFMA for element type T: bf16 uses the 32x32x16
// instruction (8 bf16 per lane), fp32 the 32x32x2 one (1 float per lane).
template <typename T>
struct Mma;

template <>
struct Mma<bf16_t> {
  static constexpr int kPerStep = 16;   // d consumed per instruction
  typedef bf16x8 frag;
  // lane-half row pointer -> fragment for step s (8 contiguous bf16)
  __device__ __forceinline__ static frag load(const bf16_t* p, int s) {
    uint4 u = *reinterpret_cast<const uint4*>(p + 8 * s);
    return __builtin_bit_cast(frag, u);
  }
  __device__ __forceinline__ static void mma(f32x16& acc, frag a, frag b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static constexpr int kPerStep = 2;
  typedef float frag;
  __device__ __forceinline__ static frag load(const float* p, int s) { return p[s]; }
  __device__ __forceinline__ static void mma(f32x16& acc, frag a, frag b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
  }
};

// ------------------------------------------------------ K tiles through LDS
// A wave stages a 32-row key tile for one KV head in its own LDS slot with
// direct global->LDS loads (global_load_lds_dwordx4: lane l's 16 bytes land
// at M0 + 16*l), so the prefetch holds no VGPRs. Each lane's MFMA A operand
// is row l%32, d half l/32, as kChunks 16-byte chunks.
template <typename T, int D>
struct KTile {
  static constexpr int kChunks = (D / 2) * (int)sizeof(T) / 16;   // 16 B chunks per lane
  static constexpr int kBytes = kChunks * 1024;                   // LDS bytes per slot
};

// Layout of a key tile in its slot. A key row is kCpr 16-byte chunks; each
// DMA instruction c loads kRpi whole rows (c*kRpi ..), so its 64 lanes read
// contiguous rows and every cache line they touch is used in full. Chunk j
// of tile row r sits at 16-byte position r*kCpr + (j ^ sw(r)); the XOR
// spreads the 16 rows read together by an MFMA operand load over all 16
// bank groups. DMA lane l of instruction c lands at position 64*c + l, i.e.
// row c*kRpi + l/kCpr, chunk (l%kCpr) ^ sw(row); that lane offset repeats
// with period kPer in c and is computed once (KLane).
template <typename T, int D>
struct KLayout {
  static constexpr int kCpr = D * (int)sizeof(T) / 16;
  static constexpr int kRpi = 64 / kCpr;
  static constexpr int kNc = kCpr / 2;                 // = KTile::kChunks
  static constexpr int kPer = kCpr == 8 ? 2 : (kCpr == 16 ? 4 : 8);
  __device__ __forceinline__ static int sw(int r) { return kCpr == 8 ? (r >> 1) & 7 : r & 15; }
};

// MFMA over one 16-byte chunk per lane of A and B: one 32x32x16 bf16 step,
// or four 32x32x2 fp32 steps.
template <typename T>
struct ChunkMma;

template <>
struct ChunkMma<bf16_t> {
  static constexpr int kSteps = 1;   // MFMA instructions per chunk
  __device__ __forceinline__ static void mma(f32x16& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <>
struct ChunkMma<float> {
  static constexpr int kSteps = 4;
  __device__ __forceinline__ static void mma(f32x16& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Waits until at most N vector-memory operations of this wave are in flight
// (vector memory operations retire in issue order for this count).
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// Reads 4 16-byte chunks (one address each) and waits for them inside the
// same asm block. The outputs are early-clobber ("=&v"): a load that lands
// while later loads of the block are still being issued must not overwrite
// an address register they use.
__device__ __forceinline__ void lds_read4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                          uint4& x0, uint4& x1, uint4& x2, uint4& x3) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// The same for 8 chunks: one round trip instead of two.
__device__ __forceinline__ void lds_read8(const uint32_t (&a)[8], uint4 (&x)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
        "=&v"(x[6]), "=&v"(x[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// Per-lane constants of the key-tile layout for one launch, two VGPRs.
// The swizzle only flips address bits that the row and slot bases leave
// clear, so every offset is one of these XOR a compile-time constant:
//   DMA lane offset of instruction c = d0 ^ (kXs * (c % kPer)),
//   read address of chunk k (of the lane's half) = (slot + rx) ^ (16 * k),
// where slots are aligned to a multiple of the row pitch (kCpr * 16 bytes).
template <typename T, int D>
struct KLane {
  typedef KLayout<T, D> L;
  static constexpr unsigned kXs = 16u * (L::kCpr == 8 ? 4u : (unsigned)L::kRpi);
  unsigned d0;   // DMA: byte offset from instruction 0's first row
  unsigned rx;   // read: byte offset of chunk 0 of the lane's half, in a slot
  __device__ __forceinline__ void init(int lane, int hkv) {
    const unsigned rs = (unsigned)(hkv * D * (int)sizeof(T));   // global row stride (bytes)
    d0 = (unsigned)(lane / L::kCpr) * rs + 16u * (unsigned)((lane % L::kCpr) ^ L::sw(lane / L::kCpr));
    const int r = lane & 31;
    rx = (unsigned)(r * L::kCpr * 16) | (16u * (unsigned)(((lane >> 5) * L::kNc) ^ L::sw(r)));
  }

  // DMA of key tile k0 .. k0+31 of KV head g into `slot`. A tile that runs
  // past the last key repeats key n-1 in its place (those keys are causally
  // masked or belong to rows past n).
  __device__ __forceinline__ void issue(const T* K, int n, int hkv, int g, int k0,
                                        unsigned char* slot) const {
    const size_t rs = (size_t)hkv * D * sizeof(T);
    const unsigned char* base = reinterpret_cast<const unsigned char*>(K + ((size_t)k0 * hkv + g) * D);
    if (k0 + 31 < n) {
#pragma unroll
      for (int c = 0; c < L::kNc; ++c)
        __builtin_amdgcn_global_load_lds(base + (size_t)(c * L::kRpi) * rs + (d0 ^ (kXs * (unsigned)(c % L::kPer))),
                                         (lds_ptr_t)(slot + 1024 * c), 16, 0, 0);
    } else {
      const int lane = (int)(threadIdx.x & 63);
#pragma unroll
      for (int c = 0; c < L::kNc; ++c) {
        const int r = c * L::kRpi + lane / L::kCpr;
        const int rr = min(r, n - 1 - k0);
        const unsigned off =
            (unsigned)rr * (unsigned)rs + 16u * (unsigned)((lane % L::kCpr) ^ L::sw(r));
        __builtin_amdgcn_global_load_lds(base + off, (lds_ptr_t)(slot + 1024 * c), 16, 0, 0);
      }
    }
  }

  // The lane's MFMA A operand chunks (row lane%32, d half lane/32) of the
  // tile in `slot`.
  __device__ __forceinline__ void read(const unsigned char* slot, uint4 (&kc)[L::kNc]) const {
    const uint32_t a = lds_addr(slot) + rx;
    if constexpr (L::kNc == 8) {   // one round trip for the whole operand
      uint32_t ad[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) ad[k] = a ^ (16u * k);
      lds_read8(ad, kc);
    } else {
#pragma unroll
      for (int k = 0; k < L::kNc; k += 4)
        lds_read4(a ^ (16u * k), a ^ (16u * (k + 1)), a ^ (16u * (k + 2)), a ^ (16u * (k + 3)),
                  kc[k], kc[k + 1], kc[k + 2], kc[k + 3]);
    }
  }
};

// Scheduling hint for a software-pipelined tile: the first `lead` MFMAs
// alone, then one MFMA per `valu` VALU instructions for `pairs` rounds, then
// the remaining VALU work. Masks: 0x008 = MFMA, 0x002 = VALU.
template <int lead, int pairs, int valu>
__device__ __forceinline__ void interleave_mfma_valu() {
#ifndef AMTK_NO_SCHED_HINTS
  __builtin_amdgcn_sched_group_barrier(0x008, lead, 0);
#pragma unroll
  for (int i = 0; i < pairs; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, valu, 0);
  }
#endif
}

// Workgroup barriers that do not drain vector memory: __syncthreads() makes
// the compiler wait for every outstanding load (vmcnt(0)), which would stall
// the per-wave global->LDS key prefetch at each barrier. barrier_lds() waits
// for this wave's LDS accesses only (LDS data handed to other waves);
// barrier_phase() only aligns the waves (no data exchanged through it).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void barrier_phase() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The wave's G query tiles as MFMA B operands (query row qrow, d half lane/32),
// held in registers for a whole pass.
template <typename T, int D, int G>
__device__ __forceinline__ void load_q_tiles(const T* __restrict__ Q, int qrow, int hq, int g,
                                             int lane, uint4 (&qc)[G][KTile<T, D>::kChunks]) {
  typedef KTile<T, D> KT;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4* src = reinterpret_cast<const uint4*>(Q + ((size_t)qrow * hq + g * G + h) * D +
                                                      (lane >> 5) * (D / 2));
#pragma unroll
    for (int c = 0; c < KT::kChunks; ++c) qc[h][c] = src[c];
  }
}

template <typename T, int NC>
__device__ __forceinline__ void score_tile(f32x16& acc, const uint4 (&kc)[NC],
                                           const uint4 (&qc)[NC]) {
  acc = f32x16{};
#pragma unroll
  for (int c = 0; c < NC; ++c) ChunkMma<T>::mma(acc, kc[c], qc[c]);
}

// Row of key / query m inside a 32-row tile held by accumulator register r.
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// -------------------------------------------------------------- wave helpers
// DPP lane permutations within rows of 16 lanes
constexpr int kDppRowMirror = 0x140;       // lane i <-> 15 - i
constexpr int kDppRowHalfMirror = 0x141;   // lane i <-> 7 - i within each 8
constexpr int kDppQuadXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;         // quad_perm [1,0,3,2]
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

// The values of x in lanes l and l ^ W (W = 16 or 32) as {lo, hi}, lo from
// the lower lane of the pair: a permlane swap of two copies of x, in the
// VALU (no LDS round trip). Every use below is symmetric in the pair or
// picks the partner by comparing with its own value.
template <int W>
__device__ __forceinline__ void lane_pair(unsigned u, unsigned& lo, unsigned& hi) {
  static_assert(W == 16 || W == 32, "permlane swaps exchange rows of 16 or halves of 32");
  if constexpr (W == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = p[0];
    hi = p[1];
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = p[0];
    hi = p[1];
  }
}
template <int W>
__device__ __forceinline__ float max_xor(float x) {
  unsigned lo, hi;
  lane_pair<W>(__float_as_uint(x), lo, hi);
  return fmaxf(__uint_as_float(lo), __uint_as_float(hi));
}
template <int W>
__device__ __forceinline__ float sum_xor(float x) {
  unsigned lo, hi;
  lane_pair<W>(__float_as_uint(x), lo, hi);
  return __uint_as_float(lo) + __uint_as_float(hi);
}
// the value of x in lane l ^ W: the member of the pair that is not this
// lane's own (when both are equal, either)
template <int W>
__device__ __forceinline__ unsigned partner_u32(unsigned u) {
  unsigned lo, hi;
  lane_pair<W>(u, lo, hi);
  return lo == u ? hi : lo;
}
__device__ __forceinline__ float xor32f(float v) { return __uint_as_float(partner_u32<32>(__float_as_uint(v))); }
__device__ __forceinline__ int xor32i(int v) { return (int)partner_u32<32>((unsigned)v); }

// Generic element loads for the VALU kernels.
__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const bf16_t* p) { return bf16_to_f32(*p); }

}  // namespace amtk
