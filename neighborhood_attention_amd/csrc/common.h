// common.h -- types and helpers shared by the NA3D kernel families and the
// host-side planner (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

#include <cstdint>

namespace na3d {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Swizzled, unpadded staging layout (rolling family).  A staged row is HD*2
// bytes = HD/8 chunks of 16 bytes; logical chunk c of row r is stored at
// physical chunk c ^ swz(r).  swz depends only on r mod 16, and the operand
// reads of a 32-key block start at multiples of 16 rows, so the XOR term is a
// per-lane constant.
//
// Measured on gfx950 (bank-conflict counters over probe patterns): a 16-byte
// LDS read is served 32 lanes at a time against 128 banks of 4 bytes, the
// 8-byte transpose read 32 lanes at a time against 64 banks.  The K operand
// read puts 16 rows x 2 chunks in one pass, the V operand (transpose) read 8
// rows x 32 bytes.  With the key order of key_perm below, swz makes both
// passes hit distinct banks: for every row offset when HD = 16, 64 or 256,
// for even row offsets when HD = 128 (the usual case: halo widths are even),
// and the V read stays 2-way when HD = 32.
__host__ __device__ constexpr int swz(int hd, int r) {
  return hd == 16    ? (r >> 3) & 1
         : hd == 32  ? (r >> 2) & 3
         : hd == 64  ? ((r >> 2) & 3) << 1
         : hd == 128 ? ((((r >> 1) + 4 * (r & 1)) & 7) << 1)
                     : (r & 15) << 1;
}

// Which key of a 16-key tile feeds MFMA row/column m.  Any permutation is
// valid as long as the K rows, the V rows and the window mask agree on it;
// for HD = 64 a 4 x 4 transpose makes the V read touch rows 4 apart, which is
// what lets swz serve both operand reads without conflicts.
__host__ __device__ constexpr int key_perm(int hd, int m) {
  return hd == 64 ? 4 * (m & 3) + (m >> 2) : m;
}

// Inward-shifted window start on one axis: clamp(i - K/2, 0, L - K).
__host__ __device__ __forceinline__ int win_start(int i, int K, int L) {
  int s = i - (K >> 1);
  s = s < 0 ? 0 : s;
  return s > L - K ? L - K : s;
}

// Spread consecutive logical tiles over one XCD: the dispatcher hands
// workgroup i to XCD i % 8, so XCD x receives logical tiles [x*n/8, (x+1)*n/8)
// in order and neighbouring tiles (which share K/V halo rows) meet in one L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n >> 3;
  const int rem = n & 7;
  if (i >= n - rem) return i;  // the ragged tail keeps its position
  return (i & 7) * per + (i >> 3);
}

// Element strides of one (B,T,H,W,NH,HD) tensor along B, T, H, W and NH
// (HD is contiguous).
struct Strides {
  int64_t b, t, h, w, n;
};

// The query box: q and out hold queries [t0, t0+Tq) x [h0, h0+Hq) x
// [w0, w0+Wq) of the T x H x W grid of k and v, and every window is placed
// in that full grid (the whole grid: offsets 0, extents T, H, W).
struct Box {
  int t0, h0, w0;
  int Tq, Hq, Wq;
};

struct Problem {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, T, H, W, NH;      // k and v grid
  int KT, KH, KW;
  Box box;                 // q and out
  Strides sq, sk, sv, so;  // k and v share h, w and n
};

// Launch description chosen by the host planner.
struct Launch {
  int family;      // 1 = general (one query plane per workgroup), 2 = rolling
  int variant;     // index into the family's instantiation table
  int tile_t, tile_h, tile_w;
  int tiles_t, tiles_h, tiles_w;
  int ta, tz;      // rolling: first run [0, ta), last run [tz, T) (ta = 0 / tz = T: none)
  int nruns, rpw;  // rolling: runs along T, consecutive runs per workgroup
  int64_t wgs;
  int threads;
  int lds_rows;    // rows of each K and V staging buffer
  int lds_bytes;
  int planes;      // K/V planes staged per workgroup (maximum)
  int band_h;      // rolling: tile rows per band of the spatial visiting order
};

// Instantiations of the rolling family: index, head dim, query block
// (QH x QW queries of 16 / (QH x QW) consecutive query planes: 16 queries per
// wave), wave grid (WH block rows x WT query-plane phases), query-plane slots per wave, 16-key tiles per softmax group, most
// groups a wave's window union may need, staged plane buffers (1 or 2), the
// waves per SIMD the register allocation must leave room for (0 = the
// compiler's choice; 4 caps it at 128 VGPRs), and staging waves (0: the
// compute waves stage the K/V planes themselves; otherwise that many extra
// waves per workgroup do nothing but stage them).
#define NA3D_ROLL_VARIANTS(X)               \
  X(0, 64, 2, 8, 1, 3, 1, 7, 1, 2, 0, 0)          \
  X(1, 64, 2, 8, 2, 3, 1, 7, 1, 2, 0, 0)          \
  X(2, 64, 4, 4, 2, 3, 1, 7, 1, 2, 0, 0)          \
  X(3, 64, 2, 8, 4, 3, 1, 7, 1, 1, 0, 0)          \
  X(4, 64, 2, 8, 2, 3, 1, 7, 1, 1, 0, 0)          \
  X(5, 64, 4, 4, 1, 4, 1, 13, 1, 1, 0, 0)         \
  X(6, 64, 4, 4, 1, 8, 1, 13, 1, 1, 0, 0)         \
  X(7, 64, 4, 4, 2, 4, 1, 13, 1, 1, 0, 0)         \
  X(8, 64, 2, 8, 1, 3, 1, 4, 1, 2, 0, 0)          \
  X(9, 64, 2, 8, 1, 3, 1, 7, 2, 2, 0, 0)          \
  X(10, 64, 4, 4, 1, 4, 1, 13, 2, 1, 0, 0)        \
  X(11, 16, 2, 8, 1, 3, 1, 7, 2, 2, 0, 0)         \
  X(12, 32, 2, 8, 1, 3, 1, 7, 2, 2, 0, 0)         \
  X(13, 128, 2, 8, 1, 3, 1, 7, 1, 2, 0, 0)        \
  X(14, 128, 2, 8, 2, 3, 1, 7, 1, 1, 0, 0)        \
  X(15, 128, 2, 8, 1, 3, 1, 7, 2, 1, 0, 0)        \
  X(16, 128, 4, 4, 1, 4, 1, 13, 1, 1, 0, 0)       \
  X(17, 64, 2, 8, 2, 4, 1, 4, 1, 2, 4, 0)         \
  X(18, 64, 2, 8, 4, 3, 1, 7, 1, 2, 0, 0)         \
  X(19, 64, 4, 4, 4, 3, 1, 7, 1, 2, 0, 0)         \
  X(20, 64, 2, 8, 1, 4, 1, 7, 1, 2, 0, 0)         \
  X(21, 64, 2, 8, 1, 4, 1, 7, 1, 1, 0, 0)         \
  X(22, 64, 4, 4, 1, 4, 1, 7, 2, 1, 0, 0)         \
  X(23, 64, 4, 4, 1, 4, 1, 7, 2, 2, 0, 0)         \
  X(24, 64, 4, 4, 2, 4, 1, 7, 2, 1, 0, 0)         \
  X(25, 128, 2, 8, 1, 4, 1, 7, 1, 1, 0, 0)        \
  X(26, 64, 2, 8, 2, 2, 2, 7, 1, 2, 0, 0)         \
  X(27, 64, 2, 8, 4, 1, 3, 4, 2, 1, 0, 0)         \
  X(28, 64, 2, 8, 2, 1, 3, 4, 2, 2, 0, 0)         \
  X(29, 128, 2, 8, 2, 2, 2, 4, 2, 1, 0, 0)        \
  X(30, 64, 2, 8, 1, 4, 1, 4, 2, 1, 0, 0)         \
  X(31, 64, 2, 8, 1, 4, 1, 4, 2, 2, 0, 0)         \
  X(32, 64, 4, 4, 1, 4, 1, 4, 2, 1, 0, 0)         \
  X(33, 128, 2, 8, 1, 4, 1, 4, 2, 1, 0, 0) \
  X(34, 64, 2, 8, 1, 4, 1, 7, 1, 1, 4, 0)  \
  X(35, 64, 4, 4, 1, 4, 1, 4, 2, 1, 4, 0)  \
  X(36, 64, 2, 8, 1, 4, 1, 4, 2, 1, 4, 0)  \
  X(37, 64, 4, 4, 1, 4, 1, 7, 1, 1, 4, 0)  \
  X(38, 64, 4, 4, 2, 4, 1, 7, 1, 1, 4, 0)  \
  X(39, 64, 4, 4, 2, 4, 1, 4, 2, 1, 4, 0)  \
  X(40, 64, 2, 8, 2, 4, 1, 7, 1, 1, 4, 0)  \
  X(41, 64, 2, 8, 4, 4, 1, 7, 1, 1, 4, 0)  \
  X(42, 64, 2, 8, 2, 4, 1, 7, 1, 2, 4, 0)  \
  X(43, 64, 4, 4, 2, 4, 1, 7, 1, 2, 4, 0)  \
  X(44, 64, 4, 4, 4, 4, 1, 7, 1, 1, 4, 0)  \
  X(45, 64, 4, 4, 3, 4, 1, 13, 1, 1, 3, 0) \
  X(46, 64, 4, 4, 3, 4, 1, 13, 1, 2, 3, 0) \
  X(47, 128, 2, 8, 2, 4, 1, 7, 1, 2, 0, 0) \
  X(48, 128, 2, 8, 2, 4, 1, 7, 1, 1, 0, 0) \
  X(49, 64, 2, 8, 1, 4, 1, 13, 1, 1, 0, 0) \
  X(50, 64, 2, 8, 2, 4, 1, 13, 1, 1, 0, 0) \
  X(51, 64, 2, 8, 2, 4, 1, 13, 1, 2, 0, 0) \
  X(52, 256, 2, 8, 1, 4, 1, 7, 1, 1, 0, 0) \
  X(53, 256, 4, 4, 1, 4, 1, 7, 1, 1, 0, 0) \
  X(54, 64, 2, 8, 2, 4, 1, 9, 2, 1, 0, 0) \
  X(55, 64, 2, 8, 2, 4, 1, 7, 3, 1, 0, 0) \
  X(56, 64, 2, 8, 2, 4, 1, 7, 4, 1, 0, 0) \
  X(57, 128, 2, 8, 1, 4, 1, 9, 2, 1, 0, 0) \
  X(58, 64, 2, 8, 1, 4, 1, 9, 2, 1, 0, 0) \
  X(59, 64, 2, 4, 2, 2, 1, 11, 1, 1, 0, 0) \
  X(60, 128, 2, 4, 2, 2, 1, 11, 1, 1, 0, 0) \
  X(61, 128, 2, 4, 4, 2, 1, 5, 1, 2, 0, 0) \
  X(62, 64, 4, 4, 2, 4, 1, 8, 4, 1, 0, 0) \
  X(63, 64, 4, 4, 2, 4, 1, 4, 1, 2, 4, 0) \
  X(64, 64, 2, 8, 2, 4, 1, 2, 1, 2, 4, 0) \
  X(65, 32, 4, 4, 1, 4, 1, 13, 1, 1, 0, 0) \
  X(66, 32, 2, 8, 1, 4, 1, 13, 1, 1, 0, 0) \
  X(67, 32, 4, 4, 2, 4, 1, 8, 4, 1, 0, 0) \
  X(68, 32, 2, 8, 2, 4, 1, 7, 1, 2, 4, 0) \
  X(69, 32, 2, 4, 2, 2, 1, 11, 1, 1, 0, 0) \
  X(70, 16, 4, 4, 1, 4, 1, 13, 1, 1, 0, 0) \
  X(71, 16, 2, 8, 1, 4, 1, 13, 1, 1, 0, 0) \
  X(72, 16, 4, 4, 2, 4, 1, 8, 4, 1, 0, 0) \
  X(73, 16, 2, 8, 2, 4, 1, 7, 1, 2, 4, 0) \
  X(74, 16, 2, 4, 2, 2, 1, 11, 1, 1, 0, 0) \
  X(75, 128, 2, 4, 4, 2, 1, 5, 1, 2, 3, 4) \
  X(76, 64, 2, 4, 6, 2, 1, 11, 1, 2, 3, 0) \
  X(77, 128, 2, 4, 4, 2, 1, 11, 1, 1, 0, 0) \
  X(78, 128, 2, 8, 1, 8, 1, 9, 2, 1, 0, 0)

struct RollVariant {
  int hd, qh, qw, wh, wt, ns, nk, ng, nbuf, occ, pw;
};

constexpr RollVariant kRollVariants[] = {
#define NA3D_ROLL_ENTRY(i, HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW) \
  {HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW},
    NA3D_ROLL_VARIANTS(NA3D_ROLL_ENTRY)
#undef NA3D_ROLL_ENTRY
};
constexpr int kNumRollVariants = sizeof(kRollVariants) / sizeof(kRollVariants[0]);

// One tile of a batched rolling launch: contiguous (B,T,H,W,NH,HD) tensors,
// every query of the grid, and the tile's own run layout.
struct BatchTile {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, T, H, W;
  int wg_off;  // the tile's first workgroup in the launch
  int tiles_t, tiles_h, tiles_w;
  int tc, ta, tz, nruns, rpw;
  int lds_rows;  // the tile's own buffer rows (the launch allocates the largest)
};

constexpr int kMaxBatch = 16;  // tiles per launch (kernel arguments stay < 2 KiB)

struct RollBatch {
  int n;
  BatchTile t[kMaxBatch];
};

// Raise kernel KERN's dynamic LDS limit above the 64 KiB default, once per
// device and size (the largest size set so far is remembered; one cache per
// kernel, since KERN is a template argument), so that launches, also under
// graph capture, make no other runtime call.
template <auto KERN>
int set_lds(int lds_bytes) {
  if (lds_bytes <= 64 * 1024) return 0;
  static std::atomic<int> done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  if (done[dev].load(std::memory_order_relaxed) >= lds_bytes) return 0;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(KERN),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess)
    return -1;
  int prev = done[dev].load(std::memory_order_relaxed);
  while (prev < lds_bytes &&
         !done[dev].compare_exchange_weak(prev, lds_bytes, std::memory_order_relaxed)) {
  }
  return 0;
}

int launch_general(const Problem& p, const Launch& l, int hd, hipStream_t s);
int launch_roll(const Problem& p, const Launch& l, int hd, hipStream_t s);
// p supplies NH and the window; l the variant, grid, threads and LDS size
int launch_roll_batch(const Problem& p, const Launch& l, const RollBatch& bt, int hd,
                      hipStream_t s);

// RMSNorm (kernel_rmsnorm.hip): 16-byte pieces held per lane for a row of
// `dim` bf16, and the launch (wgs = 0: automatic grid; 0 on success).
constexpr int kRmsMaxDim = 8192;
int rms_norm_pieces_per_lane(int dim);
int launch_rms_norm(const void* x, const void* w, void* y, int rows, int dim, float eps, int wgs,
                    hipStream_t s);

}  // namespace na3d
