// kernel_rmsnorm.hip -- bf16 RMSNorm over the last axis of a (rows, dim)
// tensor: the transformer's block norms of the xDiT PR "LTX-2.5
// optimizations: add parallel VAE decoding and AITER RMSNorm" (Changes,
// item 2), y = x * w / sqrt(mean(x^2) + eps), bf16 in and out, fp32 inside.
//
// The op reads every element once and writes it once, so HBM bandwidth is
// the bound and the design is about keeping loads in flight:
//   - one wave owns a row; lane l holds the 16-byte pieces l, l + 64, ...,
//     so every wave-wide load or store is one contiguous 1 KiB;
//   - the weight is loaded into registers once per wave and reused for all
//     the rows the wave visits (grid-stride over rows);
//   - the loads of the wave's next row are issued before the current row is
//     reduced and written (two row buffers in turn, so no register copies),
//     so a wave always has a row of loads in flight;
//   - the sum of squares is an fp32 per-lane sum followed by a butterfly
//     over the wave, which leaves the identical value in every lane;
//   - stores are non-temporal (nothing reads y back here); loads are
//     ordinary: measured on 24576 x 4096, non-temporal stores with ordinary
//     loads ran at 58 us, both non-temporal at 68 us, neither at 74 us.
// In place (y == x) is safe: a row is fully in registers before any of it
// is written, and no two waves share a row.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace na3d {
namespace {

// Waves per workgroup: 8, except for the longest rows, whose 400+ registers
// per lane leave room for one wave per SIMD only (a workgroup must fit one
// CU's four SIMDs).
template <int KCH>
constexpr int rms_waves() { return KCH >= 16 ? 4 : 8; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 8 bf16

struct RmsArgs {
  const u32x4* x;
  const u32x4* w;  // nullptr: unit weight
  u32x4* y;
  int rows;
  int pieces;  // 16-byte pieces per row (dim / 8)
  float dim;
  float eps;
};

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats to a packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 v = __builtin_convertvector((f2){lo, hi}, b2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float sq_sum(uint32_t u, float acc) {
  const float a = bf_lo(u), b = bf_hi(u);
  return b * b + (a * a + acc);
}

__device__ __forceinline__ uint32_t scale2(uint32_t xu, uint32_t wu, float r) {
  return pack_bf16(bf_lo(xu) * r * bf_lo(wu), bf_hi(xu) * r * bf_hi(wu));
}

// One row of pieces per lane: load, and normalise-and-store.  FULL: the
// row is exactly 64 * KCH pieces, so no lane is ever idle; otherwise lanes
// past the row's end load a clamped (valid) piece, zero it and skip its
// store, which keeps the loads free of branches.
template <int KCH>
__device__ __forceinline__ void load_row(u32x4 (&v)[KCH], const u32x4* row, const int (&pc)[KCH]) {
#pragma unroll
  for (int j = 0; j < KCH; ++j) v[j] = row[pc[j]];
  // keep the loads where they are issued: ahead of the other row's work
  __builtin_amdgcn_sched_barrier(0);
}

template <int KCH, bool FULL>
__device__ __forceinline__ void norm_row(u32x4 (&v)[KCH], const u32x4 (&w)[KCH], u32x4* row,
                                         const int (&pc)[KCH], const bool (&ok)[KCH],
                                         const RmsArgs& a) {
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    if (!FULL && !ok[j]) v[j] = (u32x4){0u, 0u, 0u, 0u};
    ss = sq_sum(v[j].x, ss);
    ss = sq_sum(v[j].y, ss);
    ss = sq_sum(v[j].z, ss);
    ss = sq_sum(v[j].w, ss);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float rinv = rsqrtf(ss / a.dim + a.eps);
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    u32x4 o;
    o.x = scale2(v[j].x, w[j].x, rinv);
    o.y = scale2(v[j].y, w[j].y, rinv);
    o.z = scale2(v[j].z, w[j].z, rinv);
    o.w = scale2(v[j].w, w[j].w, rinv);
    if (FULL || ok[j]) __builtin_nontemporal_store(o, row + pc[j]);
  }
}

// Rows first, first + step, ... of the wave, two row buffers in turn: the
// next row's loads are issued before the current row is normalised.  The
// prefetch row is clamped to the last row, so the loads are unconditional
// (a wave's final prefetch re-reads that one row, which the caches hold).
template <int KCH, bool FULL>
__global__ void __launch_bounds__(64 * rms_waves<KCH>()) rms_norm_kernel(const RmsArgs a) {
  constexpr int kRmsWaves = rms_waves<KCH>();
  const int lane = threadIdx.x & 63;
  const int first = __builtin_amdgcn_readfirstlane(blockIdx.x * kRmsWaves + (threadIdx.x >> 6));
  const int step = gridDim.x * kRmsWaves;
  if (first >= a.rows) return;
  const int64_t last = a.rows - 1;

  bool ok[KCH];
  int pc[KCH];
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int p = lane + 64 * j;
    ok[j] = FULL || p < a.pieces;
    pc[j] = ok[j] ? p : a.pieces - 1;
  }
  const uint32_t one = 0x3f803f80u;  // two bf16 1.0
  u32x4 w[KCH];
#pragma unroll
  for (int j = 0; j < KCH; ++j) w[j] = (u32x4){one, one, one, one};
  if (a.w != nullptr) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) w[j] = a.w[pc[j]];
  }

  u32x4 bufa[KCH], bufb[KCH];
  int64_t r = first;
  load_row<KCH>(bufa, a.x + r * a.pieces, pc);
  for (;;) {
    int64_t rn = r + step < last ? r + step : last;
    load_row<KCH>(bufb, a.x + rn * a.pieces, pc);
    norm_row<KCH, FULL>(bufa, w, a.y + r * a.pieces, pc, ok, a);
    r += step;
    if (r > last) break;
    rn = r + step < last ? r + step : last;
    load_row<KCH>(bufa, a.x + rn * a.pieces, pc);
    norm_row<KCH, FULL>(bufb, w, a.y + r * a.pieces, pc, ok, a);
    r += step;
    if (r > last) break;
  }
}

// wgs == 0: about one and a half rows per wave, many more waves than the
// GPU holds at once; the hardware hands the late workgroups to whichever CUs
// free up first, which evens out the end of the launch better than a grid
// sized to what is resident (measured on 24576 x 4096: 56.9 us with 8-wave
// workgroups at 1.5 rows per wave, 58.0 us with 4-wave ones at 2 rows, 58.6
// us with a resident-sized grid).
template <int KCH, bool FULL>
int launch_kch(const RmsArgs& a, int wgs, hipStream_t s) {
  constexpr int kRmsWaves = rms_waves<KCH>();
  if (wgs == 0) {
    const int64_t g = (2 * (int64_t)a.rows + 3 * kRmsWaves - 1) / (3 * kRmsWaves);
    wgs = (int)(g < (1 << 20) ? g : (1 << 20));  // beyond that, waves stride over rows
  }
  hipLaunchKernelGGL((rms_norm_kernel<KCH, FULL>), dim3(wgs), dim3(64 * kRmsWaves), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int KCH>
int launch_k(const RmsArgs& a, int wgs, hipStream_t s) {
  return a.pieces == 64 * KCH ? launch_kch<KCH, true>(a, wgs, s)
                              : launch_kch<KCH, false>(a, wgs, s);
}

}  // namespace

int rms_norm_pieces_per_lane(int dim) {
  const int pieces = dim / 8;
  int k = 1;
  while (64 * k < pieces) k *= 2;
  return k;
}

int launch_rms_norm(const void* x, const void* w, void* y, int rows, int dim, float eps, int wgs,
                    hipStream_t s) {
  RmsArgs a;
  a.x = static_cast<const u32x4*>(x);
  a.w = static_cast<const u32x4*>(w);
  a.y = static_cast<u32x4*>(y);
  a.rows = rows;
  a.pieces = dim / 8;
  a.dim = (float)dim;
  a.eps = eps;
  switch (rms_norm_pieces_per_lane(dim)) {
    case 1: return launch_k<1>(a, wgs, s);
    case 2: return launch_k<2>(a, wgs, s);
    case 4: return launch_k<4>(a, wgs, s);
    case 8: return launch_k<8>(a, wgs, s);
    case 16: return launch_k<16>(a, wgs, s);
    default: return -1;
  }
}

}  // namespace na3d
