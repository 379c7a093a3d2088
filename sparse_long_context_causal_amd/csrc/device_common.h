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

namespace amtk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
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

// Row of key / query m inside a 32-row tile held by accumulator register r.
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// -------------------------------------------------------------- wave helpers
__device__ __forceinline__ float xor32f(float v) { return __shfl_xor(v, 32, 64); }
__device__ __forceinline__ int xor32i(int v) { return __shfl_xor(v, 32, 64); }

// Generic element loads for the VALU kernels.
__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const bf16_t* p) { return bf16_to_f32(*p); }

}  // namespace amtk
