// Read-bandwidth calibration of the on-chip L2 caches (gfx950), built as
// libamtk_calib.so beside the library. It measures a ceiling for kernels whose
// reads are served from L2 rather than HBM (the windowed gather): every XCD
// re-reads a region of its own that fits its L2, so after the first pass all
// reads hit that XCD's L2.
//
// Workgroups are handed to the 8 XCDs round robin, so workgroup b runs on
// XCD b % 8 and reads region b % 8 of the buffer; the workgroups of one XCD
// split its region among themselves.
//   mode 0: contiguous 16-byte loads, 256 threads walking the region in
//           strides (the plain streaming ceiling);
//   mode 1: 256-byte rows at pseudo-random row positions of the region, one
//           row per 16 lanes (the access shape of a row gather);
//   mode 2: the rows of mode 1 brought into LDS by direct global->LDS loads,
//           as the gather stages them (kernel below).
// Nothing is written unless the XOR of everything read hits a fixed 128-bit
// value, which keeps the loads alive without adding write traffic.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kXcds = 8;
constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr unsigned kRowsPerPass = 64;   // rows one 16-lane group reads per pass (mode 1)

__global__ __launch_bounds__(kThreads) void l2_stream_kernel(const uint4* __restrict__ buf,
                                                             long region, int iters,
                                                             uint4* __restrict__ sink) {
  const int xcd = blockIdx.x % kXcds;
  const long local = blockIdx.x / kXcds;
  const long per_xcd = gridDim.x / kXcds;
  const uint4* base = buf + (long)xcd * region;
  const long stride = per_xcd * kThreads;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int it = 0; it < iters; ++it) {
    long e = local * kThreads + threadIdx.x;
    for (; e + (kUnroll - 1) * stride < region; e += kUnroll * stride) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = base[e + u * stride];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w;
      }
    }
    for (; e < region; e += stride) {
      uint4 v = base[e];
      acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
    }
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu && acc.w == 0xc2b2ae35u)
    sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void l2_rows_kernel(const uint4* __restrict__ buf,
                                                           long region, int iters,
                                                           uint4* __restrict__ sink) {
  const int xcd = blockIdx.x % kXcds;
  const unsigned local = blockIdx.x / kXcds;
  const uint4* base = buf + (long)xcd * region;
  const unsigned rows = (unsigned)(region / 16);          // 256-byte rows
  const unsigned group = local * (kThreads / 16) + threadIdx.x / 16;
  const int piece = threadIdx.x % 16;
  // each group reads kRowsPerPass rows per pass at scrambled positions
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int it = 0; it < iters; ++it) {
    for (unsigned r0 = 0; r0 < kRowsPerPass; r0 += kUnroll) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const unsigned t = (group * kRowsPerPass + r0 + u) + (unsigned)it * 7919u;
        const unsigned row = (t * 2654435761u) % rows;
        v[u] = base[(long)row * 16 + piece];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w;
      }
    }
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu && acc.w == 0xc2b2ae35u)
    sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

// mode 2: the same 256-byte rows as mode 1, but brought into LDS with
// global_load_lds_dwordx4 (16 bytes per lane, 4 rows per instruction), the
// way the gather stages its keys and values: one 64-lane workgroup with a
// 16 KiB LDS buffer (32 rows of keys and of values), 16 loads per round, all
// of a round in flight before it is waited for; a lane then reads one word
// of the buffer back so the loads cannot be elided.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__global__ __launch_bounds__(64) void l2_rows_lds_kernel(const uint4* __restrict__ buf,
                                                        long region, int iters,
                                                        uint4* __restrict__ sink) {
  __shared__ __align__(256) unsigned char smem[16384];
  const int xcd = blockIdx.x % kXcds;
  const unsigned local = blockIdx.x / kXcds;
  const unsigned char* base = reinterpret_cast<const unsigned char*>(buf + (long)xcd * region);
  const unsigned rows = (unsigned)(region / 16);
  const int lane = threadIdx.x;
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const unsigned t = (local * 64u + (unsigned)(4 * c + (lane >> 4))) + (unsigned)it * 7919u;
      const unsigned row = (t * 2654435761u) % rows;
      const unsigned char* src = base + (size_t)row * 256 + 16 * (lane & 15);
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(uintptr_t)(lds + 1024u * c), 16, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    acc ^= *reinterpret_cast<const volatile unsigned*>(smem + 4 * lane + 256 * (it & 63));
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x * 64 + lane] = make_uint4(acc, 0, 0, 0);
}

}  // namespace

extern "C" __attribute__((visibility("default")))
/* Launches one calibration pass on `stream`.
 * buf: device buffer of 8 * region_bytes (one region per XCD); region_bytes a
 * multiple of 4096. grid: workgroups (a multiple of 8). mode 0 or 1 as above.
 * sink: device buffer of grid * 256 * 16 bytes (written only in the
 * practically impossible case above). Returns 0, -1 on bad arguments, or the
 * hipError_t of the launch. Bytes read per pass: mode 0: iters * 8 *
 * region_bytes; mode 1: iters * grid * 16 * 64 * 256 (64 rows of 256 bytes per
 * 16-lane group and pass); mode 2 (64-lane workgroups): iters * grid * 16384. */
int amtk_calib_l2_read(const void* buf, size_t region_bytes, int iters, int grid, int mode,
                       void* sink, void* stream) {
  if (!buf || !sink || region_bytes == 0 || region_bytes % 4096 || iters < 1 || grid < kXcds ||
      grid % kXcds || mode < 0 || mode > 2)
    return -1;
  const long region = (long)(region_bytes / sizeof(uint4));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == 2)
    l2_rows_lds_kernel<<<grid, 64, 0, st>>>(static_cast<const uint4*>(buf), region, iters,
                                            static_cast<uint4*>(sink));
  else if (mode == 0)
    l2_stream_kernel<<<grid, kThreads, 0, st>>>(static_cast<const uint4*>(buf), region, iters,
                                                 static_cast<uint4*>(sink));
  else
    l2_rows_kernel<<<grid, kThreads, 0, st>>>(static_cast<const uint4*>(buf), region, iters,
                                               static_cast<uint4*>(sink));
  return (int)hipGetLastError();
}
