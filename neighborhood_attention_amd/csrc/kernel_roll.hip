// kernel_roll.hip -- the "rolling" NA3D forward family (gfx950).
//
// Operation: ROCm/aiter PR "Add 3D neighborhood flash attention (na3d_flash)",
// Motivation and Technical Details: every query (t,h,w) attends to the
// KT x KH x KW box of keys starting at clamp(i - K/2, 0, L - K) per axis;
// Q arrives pre-scaled by head_dim^-0.5; softmax is taken online in log2 space.
//
// Workgroup (WG) = batch b, head n, a (WH*QH) x QW spatial tile and a run of
// consecutive query planes [t0, t1).  The WG is a WH x WT grid of waves: wave
// (ih, it) owns the QH x QW block of 16 queries in block row ih, for the query
// planes t0 + it, t0 + it + WT, ... of the run.  With QH x QW = 8 a block
// holds QH x QW queries on each of two consecutive planes (wave it owns the
// plane pairs starting at t0 + 2 it, t0 + 2 (it + WT), ...); both planes read
// the same key planes except the first and the last of the pair's windows,
// where the other plane's queries are masked, and the smaller spatial block
// has a smaller window union per plane.  All waves share the same query
// columns, so the union of a block's windows is one contiguous range of the
// staged halo rows, and every K/V operand address is a lane constant plus a
// compile-time tile offset.
//
// The WG streams the key planes of its runs in order.  Each plane's K/V halo
// is staged in LDS once, with direct global->LDS loads (global_load_lds
// dwordx4), into one or two plane buffers (with two, plane t'+1 is in flight
// while plane t' is computed).  Staged rows are unpadded and XOR-swizzled in
// 16-byte chunks (see swz), which keeps both operand reads free of bank
// conflicts.  A wave keeps the online-softmax state of up to NS of its query
// planes (admitted when the stream reaches their window start, retired after
// their last key plane) and reuses every K/V fragment it reads for all of them.
//
// Runs: the first query planes of an axis share the window [0, KT), and so do
// the last ones.  The host may give those planes runs of their own, so that
// in the middle runs a wave's consecutive query planes (WT apart) have
// disjoint windows and WT = KT keeps every wave busy on every key plane.
//
// Per key plane a wave reads a window of 16*NK*NG staged rows that covers
// its union (shifted down where it would pass the end of the buffer), as NG
// groups of NK 16-key tiles.  A (group, query plane) unit takes three steps;
// units run as a software pipeline, so one unit's exponentials share a
// branch-free region with the next unit's score MFMAs and the previous
// unit's P.V MFMAs:
//   S^T = K . Q^T + mask    bf16 MFMA 16x16x32 whose accumulator starts at the
//                           window mask (0 or -2^100): a register table that is
//                           the first MFMA's accumulator input when a wave
//                           reads at most 7 tiles per plane, else one MFMA
//                           per tile of masks kept as bf16 pairs against
//                           the identity
//   softmax                 one exact max over the group's scores, a
//                           rescale of the running output only when the max
//                           rises by more than kRescale, then exp2
//   O^T += V^T . P^T        bf16 MFMA 16x16x32 per pair of tiles (an odd
//                           last tile is paired with zero weights); the S^T
//                           accumulator layout is already the P^T operand,
//                           V^T comes from the transpose read
// Rows past the staged halo are zeroed once, so every row read holds finite
// values and masked keys contribute exactly zero.
//
// The kernel body (roll_body) serves two entry kernels: one grid per launch,
// and many independent grids per launch (tiles of a decoder's tile grid),
// where each workgroup first looks up its tile in a table passed with the
// kernel arguments.
//
// Global memory traffic is arranged so that compute never waits on it:
// a query plane's Q is fetched one key plane ahead into spare registers, and
// a retired plane's output is packed into registers and stored after the
// next barrier, so the one wait per key plane (for the staged plane) does
// not also wait for fresh stores.
#include "common.h"

namespace na3d {
namespace {

constexpr float kNegInf = -__builtin_inff();
// Natural-log headroom before the reference max is moved: unnormalised
// weights stay below e^8 (about 3000), far inside bf16 and fp32 range.
constexpr float kRescale = 8.f;
// Score of a key outside a query's window: -2^100, finite so that the mask
// MFMA against the identity has no -inf * 0 terms, and far below any real
// score, so exp2 of it relative to a real reference max is exactly 0.
constexpr uint32_t kMaskBits = 0xf180u;   // bf16 -2^100
constexpr float kRealScore = -1.0e27f;    // scores below this are masked ones
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left free (gfx9 layout)
constexpr int kWaitVm0 = 0x0f70;

// Division of a 32-bit unsigned value by a divisor fixed for the launch,
// by multiplication: the round-up method of Granlund and Montgomery
// ("Division by invariant integers using multiplication", 1994, section 4).
// With l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (the host
// derives them), n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0) with
// t = mulhi(m, n), exact for every 32-bit n: a few scalar instructions where
// a plain division of uniform values takes a reciprocal sequence on the
// vector unit.  FAST = false divides plainly (the batch kernel, whose tiles
// are described on the device).
struct UDiv {
  uint32_t d, m;
  int s1, s2;
};
UDiv make_udiv(uint32_t d) {
  UDiv v;
  v.d = d;
  int l = 0;
  while (l < 32 && ((uint64_t)1 << l) < d) ++l;
  v.m = (uint32_t)(((((uint64_t)1 << l) - d) << 32) / d + 1);
  v.s1 = l < 1 ? l : 1;
  v.s2 = l > 1 ? l - 1 : 0;
  return v;
}
__host__ __device__ inline UDiv plain_udiv(uint32_t d) { return UDiv{d, 0u, 0, 0}; }
template <bool FAST>
__device__ __forceinline__ uint32_t udiv(uint32_t n, const UDiv& v) {
  if constexpr (!FAST) return n / v.d;
  const uint32_t t = __umulhi(v.m, n);
  return (t + ((n - t) >> v.s1)) >> v.s2;
}

struct RollArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, T, H, W, NH;  // k and v grid
  int KT, KH, KW;
  int t_off, h_off, w_off;  // query box: q/out plane t is grid plane t_off + t, ...
  int Tq, Hq, Wq;           // ... and its extents
  int tiles_t, tiles_h, tiles_w;
  int tc;        // query planes per middle run
  int ta;        // first run [0, ta); 0 = none
  int tz;        // last run [tz, T); T = none
  int nruns;     // runs along T
  int rpw;       // consecutive runs streamed by one workgroup
  int lds_rows;  // rows of each K and V staging buffer
  int band_h;    // spatial tiles are visited in bands of this many tile rows
  Strides sq, sk, sv, so;  // element strides; k and v share h, w and n
  // the workgroup-index divisors: tiles_t, tiles_h * tiles_w, band_h *
  // tiles_w, band_h, the last band's tile rows, NH
  UDiv dv_tt, dv_nt, dv_br, dv_bh, dv_bl, dv_nh;
};

// Max over the 4 lanes (l, l^16, l^32, l^48) that hold one query,
// with the gfx950 row-swap permutes (VALU only, no LDS round trip).  After
// v_permlane16_swap a, b (both holding x), a and b hold x of lanes l and
// l^16 in some order; v_permlane32_swap does the same for l^32.  Written as
// inline assembly: the compiler folds the builtin's two results into one
// when both inputs are the same value.  The s_nop covers the VALU-write ->
// permlane-read hazard.
__device__ __forceinline__ void swap16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float xmax4(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = fmaxf(a, b);
  a = x;
  b = x;
  swap32(a, b);
  return fmaxf(a, b);
}

template <int HD>
struct Slot {
  static constexpr int KSTEPS = (HD + 31) / 32;
  static constexpr int MT = HD / 16;
  bf16x8 qf[KSTEPS];  // Q^T operand: lane (q16, g) holds head dims [32ks + 8g, +8)
  f32x4 acc[MT];      // O^T: lane (q16, g) holds head dims 16mt + 4g + r
  f32x4 accl;         // softmax denominator: the same P^T against a V^T row of ones
  float m;            // reference max (natural units), -inf before any key
};

// Q of one query plane: `base` is the wave-uniform address of the plane in
// the head, `off` this lane's token offset in bytes (32-bit: the host keeps
// one head's spatial plane of q and of out below 4 GiB for this family).
template <int HD>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[Slot<HD>::KSTEPS], const uint16_t* base, uint32_t off,
                                       int g) {
  const unsigned char* const qp = reinterpret_cast<const unsigned char*>(base) + off;
#pragma unroll
  for (int ks = 0; ks < Slot<HD>::KSTEPS; ++ks) {
    const int d = 32 * ks + 8 * g;
    qf[ks] = d < HD ? *reinterpret_cast<const bf16x8*>(qp + 2 * d) : bf16x8{};
  }
}

// A slot admits a query plane with m = -inf and whatever its accumulators
// hold from the plane it served before: the first real score of the new
// plane always moves the reference max, and that rescale multiplies the
// accumulators by 0 (units before it add only exact zero weights).
template <int HD>
__device__ __forceinline__ void reset_state(Slot<HD>& S) {
  S.m = kNegInf;
}

__device__ __forceinline__ void swap16u(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32u(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Normalised output of a retired query plane, packed as bf16 (RNE).  Lane
// (q16, g) holds head dims 16mt + 4g .. +3 (8 bytes) of query q16 for each mt.
// For HD >= 32 the 8-byte pieces of each pair of tiles (2j, 2j+1) are then
// regrouped among the four lanes of the query (lane groups g, all exchanges
// stay within one query) so that lane g holds head dims 32j + 8g .. +7: each
// 16-byte store then writes 64 contiguous bytes of every query row (half as
// many store instructions, whole 64-byte segments instead of 32-byte ones).
// Start: group g holds A = piece (g, 2j), B = piece (g, 2j+1).  The 32-lane
// swap exchanges groups {2,3} of A with groups {0,1} of B; the 16-lane swap
// then exchanges group 1 of A with group 0 of B and group 3 of A with group 2
// of B, leaving group g with the pieces at dims 32j + 8g and 32j + 8g + 4.
template <int HD>
__device__ __forceinline__ void pack_out(const Slot<HD>& S, uint32_t (&pk)[2 * Slot<HD>::MT]) {
  constexpr int MT = Slot<HD>::MT;
  const float inv = 1.f / S.accl[0];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const bf16x2 lo = {(__bf16)(S.acc[mt][0] * inv), (__bf16)(S.acc[mt][1] * inv)};
    const bf16x2 hi = {(__bf16)(S.acc[mt][2] * inv), (__bf16)(S.acc[mt][3] * inv)};
    pk[2 * mt] = __builtin_bit_cast(uint32_t, lo);
    pk[2 * mt + 1] = __builtin_bit_cast(uint32_t, hi);
  }
  if constexpr (MT >= 2) {
#pragma unroll
    for (int j = 0; j < MT / 2; ++j) {
      swap32u(pk[4 * j], pk[4 * j + 2]);
      swap32u(pk[4 * j + 1], pk[4 * j + 3]);
      swap16u(pk[4 * j], pk[4 * j + 2]);
      swap16u(pk[4 * j + 1], pk[4 * j + 3]);
    }
  }
}

// Stores of a packed output (layout of pack_out).
template <int MT>
__device__ __forceinline__ void store_out(uint16_t* base, uint32_t off, const uint32_t (&pk)[2 * MT], int g) {
  unsigned char* const op = reinterpret_cast<unsigned char*>(base) + off;
  if constexpr (MT >= 2) {
#pragma unroll
    for (int j = 0; j < MT / 2; ++j)
      *reinterpret_cast<uint4*>(op + 2 * (32 * j + 8 * g)) =
          make_uint4(pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]);
  } else {
    *reinterpret_cast<uint2*>(op + 2 * (4 * g)) = make_uint2(pk[0], pk[1]);
  }
}

// V^T operand through the transpose read: lane (4j + a) of a 16-lane group
// addresses key row j of the group's 4 keys, head dims [16mt + 4a, +4); lane
// (4a + b) receives column 16mt + 4a + b of those 4 rows.
__device__ __forceinline__ s16x4 load_vt(const unsigned char* lds, int ofs) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + ofs));
}

__device__ __forceinline__ bf16x8 cat8(s16x4 lo, s16x4 hi) {
  const bf16x4 a = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 b = __builtin_bit_cast(bf16x4, hi);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// K operand chunk c of staged row r, and V operand bytes for transpose-read
// lane (q16 & 3) of head-dim tile mt, in the swizzled layout.
template <int HD>
__device__ __forceinline__ int k_addr(int r, int c) {
  return r * (HD * 2) + ((c ^ swz(HD, r)) << 4);
}
template <int HD>
__device__ __forceinline__ int v_addr(int r, int mt, int q16) {
  return r * (HD * 2) + (((2 * mt + ((q16 & 3) >> 1)) ^ swz(HD, r)) << 4) + ((q16 & 1) << 3);
}

// Direct global->LDS load of 16 bytes per lane: lane L's bytes land at LDS
// address lds + 16 L.  Written as inline assembly so that the compiler does
// not see an LDS write in flight: it would otherwise wait for it (vmcnt(0))
// before every transpose read, stalling compute on the next plane's
// staging.  The kernel waits for these loads itself, before the barrier that
// hands a staged plane to compute.  M0 (the LDS base operand) is restored;
// the s_nop keeps the wait state the hardware needs between an M0 write and
// an LDS DMA (the compiler inserts the same one for its own sequence).
// The source address is a wave-uniform base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16(const void* base, uint32_t ofs, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(ofs), "s"(base), "s"(lds)
      : "memory");
}

// The same for a K row chunk and the V row chunk at the same source offset,
// landing vgap bytes apart in LDS: one M0 save/restore for the pair.
__device__ __forceinline__ void dma16_kv(const void* kbase, const void* vbase, uint32_t ofs, uint32_t lds,
                                         uint32_t vgap) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_add_u32 m0, m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(ofs), "s"(kbase), "s"(vbase), "s"(lds), "s"(vgap)
      : "memory", "scc");
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// The whole kernel for workgroup `wg` of the problem in `a` (one grid, or
// one tile of a batch).
template <int HD, int QH, int QW, int WH, int WT, int NS, int NK, int NG, int NBUF, int OCC, int PW,
          bool FASTDIV>
__device__ __forceinline__ void roll_body(const RollArgs& a, int wg) {
  // A wave owns 16 queries: a QH x QW block of PT consecutive query planes
  // (PT = 2 for 8-query spatial blocks: the union of their windows is
  // smaller per plane, and a key plane is shared by both planes' queries).
  constexpr int BQ = QH * QW;  // queries of one plane in a block
  constexpr int PT = 16 / BQ;
  static_assert(BQ * PT == 16 && (PT == 1 || PT == 2), "a wave owns 16 queries");
  static_assert(NBUF == 1 || NBUF == 2, "one or two plane buffers");
  constexpr int KSTEPS = Slot<HD>::KSTEPS;
  constexpr int MT = Slot<HD>::MT;
  constexpr int CPR = HD / 8;  // 16-byte chunks per staged row
  constexpr int RB = HD * 2;   // staged row bytes
  constexpr int BH = WH * QH;
  // With PW > 0 the workgroup has PW staging waves after its WH x WT compute
  // waves: they issue every K/V plane's loads and compute nothing, so the
  // compute waves never wait behind the plane's burst of loads at the CU's
  // address unit (with one workgroup per CU, every wave otherwise spends a
  // large part of each step there).  NT = the threads that stage.
  constexpr int NTC = kWave * WH * WT;
  constexpr int NT = PW > 0 ? kWave * PW : NTC;
  constexpr int NTA = NTC + kWave * PW;
  constexpr int RSTEP = NT / CPR;  // staged rows per DMA round
  constexpr int GK = 16 * NK;      // keys per softmax group
  constexpr int NP = NK / 2;       // 32-key tile pairs per group
  constexpr bool ODD = (NK & 1) != 0;
  // window masks as an fp32 accumulator-input table (see below) when a wave
  // reads at most 7 tiles per key plane, else as bf16 pairs applied by MFMA
  constexpr bool kMaskTable = NG * NK <= 7;
  // two-plane blocks apply their per-plane window along T per key plane (see
  // the compute step), with one slot per wave
  static_assert(PT == 1 || NS == 1, "two-plane blocks: one slot");
  // V^T operands of all ones (bf16 1.0): the MFMA against P^T sums the
  // weights of each query, already reduced over its four lanes
  const bf16x8 kOnes8 = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int buf_bytes = a.lds_rows * RB;  // one K or V plane buffer

  const int tid = threadIdx.x;
  // the wave index is uniform across the wave: keep it (and everything that
  // depends only on it) in scalar registers, so per-wave decisions are
  // scalar branches rather than exec-masked code
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int q16 = lane & 15;
  const int g = lane >> 4;
  const bool stager = PW > 0 && wave >= WH * WT;  // a staging wave
  const bool computes = !stager;
  const int ih = wave % WH;
  const int it = wave / WH;
  // the thread's (and wave's) place among the threads that stage
  const int stid = PW > 0 ? tid - NTC : tid;
  const int swave = PW > 0 ? wave - WH * WT : wave;

  // ---- workgroup -> (b, n, tile_h, tile_w, run group); run groups vary
  // fastest.  Within a head the spatial tiles are visited in bands of band_h
  // tile rows, down each band's column of tiles before the next column, so
  // the workgroups in flight on one XCD (consecutive indices, see xcd_remap)
  // cover a compact block of the grid and read the halo rows they share
  // from that XCD's L2 rather than from HBM.
  const int wq1 = (int)udiv<FASTDIV>((uint32_t)wg, a.dv_tt);
  const int tt = wg - wq1 * a.tiles_t;
  const int ntile = a.tiles_h * a.tiles_w;
  const int wq2 = (int)udiv<FASTDIV>((uint32_t)wq1, a.dv_nt);
  const int j = wq1 - wq2 * ntile;
  const int band_rows = a.band_h * a.tiles_w;
  const int band = (int)udiv<FASTDIV>((uint32_t)j, a.dv_br);
  const int jb = j - band * band_rows;
  const int gh = min(a.band_h, a.tiles_h - band * a.band_h);  // rows in this band
  const int tw = (int)udiv<FASTDIV>((uint32_t)jb, gh == a.band_h ? a.dv_bh : a.dv_bl);
  const int th = band * a.band_h + jb - tw * gh;
  const int b = (int)udiv<FASTDIV>((uint32_t)wq2, a.dv_nh);
  const int n = wq2 - b * a.NH;

  const int T = a.T, H = a.H, W = a.W, KT = a.KT, KH = a.KH, KW = a.KW;
  const int Hq = a.Hq, Wq = a.Wq;
  // Queries are indexed in the box (q, out, tiles, runs); windows, halos and
  // K/V in the grid: the window of box plane t starts at key plane wst(t),
  // of box row h at grid row wsh(h), of box column w at grid column wsw(w).
  auto wst = [&](int t) { return win_start(a.t_off + t, KT, T); };
  auto wsh = [&](int h) { return win_start(a.h_off + h, KH, H); };
  auto wsw = [&](int w) { return win_start(a.w_off + w, KW, W); };
  // query planes [t0, t1) of run ri
  auto run_bounds = [&](int ri, int& t0, int& t1) {
    const int mid = ri - (a.ta > 0 ? 1 : 0);
    if (a.ta > 0 && ri == 0) {
      t0 = 0;
      t1 = a.ta;
    } else if (a.tz < a.Tq && ri == a.nruns - 1) {
      t0 = a.tz;
      t1 = a.Tq;
    } else {
      t0 = a.ta + mid * a.tc;
      t1 = min(t0 + a.tc, a.tz);
    }
  };
  const int r_lo = tt * a.rpw, r_hi = min(r_lo + a.rpw, a.nruns);
  const int h0 = th * BH, w0 = tw * QW;  // tile origin in the box
  const int h1 = min(h0 + BH, Hq) - 1, w1 = min(w0 + QW, Wq) - 1;
  // halo of the tile (grid coordinates): rows [hh0, hh0 + hhn) x columns
  // [hw0, hw0 + hwd)
  const int hh0 = wsh(h0);
  const int hhn = wsh(h1) + KH - hh0;
  const int hw0 = wsw(w0);
  const int hwd = wsw(w1) + KW - hw0;
  const int halo_rows = hhn * hwd;
  const int total_chunks = halo_rows * CPR;

  // ---- this wave's block of 16 queries
  const int bh0 = h0 + ih * QH;
  const bool active = computes && bh0 < Hq;
  const int pt = q16 / BQ;  // this lane's plane within the block (PT > 1)
  const int qr = q16 % BQ;  // and its query within that plane's block
  const int qh = bh0 + qr / QW;
  const int qw = w0 + qr % QW;
  const bool qvalid = active && qh < Hq && qw < Wq;  // spatially
  const int qhc = min(qh, Hq - 1), qwc = min(qw, Wq - 1);
  // union of the block's windows = staged rows [base, base + un); the wave
  // reads rows [rb, rb + NG * GK), which hold the union (the host checks
  // NG * GK >= un) and stay in the buffer (lds_rows >= NG * GK)
  const int uh0 = active ? wsh(bh0) : hh0;
  const int base = (uh0 - hh0) * hwd;
  const int rb = max(0, min(base, a.lds_rows - NG * GK));

  // ---- window masks.  For tile c of group gi, lane (q16, g) holds the A
  // operand of a 16x16x16 MFMA against the identity: for the key in MFMA row
  // q16 (the same key its K operand row holds) and the block's queries
  // 4g .. 4g+3, 0 (in window) or -2^100 (out), as bf16 pairs.  The product
  // lands in the S^T accumulator layout and seeds the score MFMAs.
  int ah[4], aw[4];  // window starts of queries 4g + j, relative to the halo
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int qi = (4 * g + j) % BQ;
    const int qhj = bh0 + qi / QW, qwj = w0 + qi % QW;
    const bool ok = active && qhj < Hq && qwj < Wq;
    ah[j] = ok ? wsh(qhj) - hh0 : -(1 << 20);
    aw[j] = wsw(min(qwj, Wq - 1)) - hw0;
  }
  const int kp = key_perm(HD, q16);
  constexpr int NKP = (NK + 1) / 2;  // tile pairs per group
  uint4 mk[kMaskTable ? 1 : NG][NKP];  // tiles 2p (x, y) and 2p + 1 (z, w)
  if constexpr (!kMaskTable) {
    // halo coordinates of this lane's key row, advanced 16 rows per tile
    int r = rb + kp;
    int uh = r / hwd, uw = r - (r / hwd) * hwd;
    const int dh = 16 / hwd, dw = 16 % hwd;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        uint32_t bits[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool in = r < halo_rows && (unsigned)(uh - ah[j]) < (unsigned)KH &&
                          (unsigned)(uw - aw[j]) < (unsigned)KW;
          bits[j] = in ? 0u : kMaskBits;
        }
        const uint32_t w0 = bits[0] | (bits[1] << 16), w1 = bits[2] | (bits[3] << 16);
        if (c & 1) {
          mk[gi][c >> 1].z = w0;
          mk[gi][c >> 1].w = w1;
        } else {
          mk[gi][c >> 1].x = w0;
          mk[gi][c >> 1].y = w1;
          if (c == NK - 1) mk[gi][c >> 1].z = mk[gi][c >> 1].w = 0u;
        }
        r += 16;
        uh += dh;
        uw += dw;
        if (uw >= hwd) {
          uw -= hwd;
          ++uh;
        }
      }
  }
  // With few tiles per wave the masks are kept instead in the S^T
  // accumulator layout, as the accumulator input of each tile's first score
  // MFMA, so masking costs no instruction per tile: for tile c of group gi,
  // lane (q16, g) holds query q16 of the block against the keys
  // key_perm(4g + r) of the tile, r = 0..3, as 0 or -2^100 (fp32).  The
  // key-to-row map is the same on every key plane, so the table is built once
  // per wave.  It takes 4 registers per tile (the bf16 pairs above take 2,
  // plus the identity), so it is used where it leaves the register budget of
  // the variant intact.
  f32x4 mc[kMaskTable ? NG : 1][kMaskTable ? NK : 1];
  if constexpr (kMaskTable) {
    const int qhm = bh0 + qr / QW, qwm = w0 + qr % QW;
    const bool okm = active && qhm < Hq && qwm < Wq;
    // window start of this lane's query, relative to the halo
    const int ahm = okm ? wsh(qhm) - hh0 : -(1 << 20);
    const int awm = wsw(min(qwm, Wq - 1)) - hw0;
    const float kMaskF = __builtin_bit_cast(float, kMaskBits << 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // halo coordinates of key row key_perm(4g + r), advanced 16 rows per tile
      int row = rb + key_perm(HD, 4 * g + r);
      int uh = row / hwd, uw = row - (row / hwd) * hwd;
      const int dh = 16 / hwd, dw = 16 % hwd;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int c = 0; c < NK; ++c) {
          const bool in = row < halo_rows && (unsigned)(uh - ahm) < (unsigned)KH &&
                          (unsigned)(uw - awm) < (unsigned)KW;
          mc[gi][c][r] = in ? 0.f : kMaskF;
          row += 16;
          uh += dh;
          uw += dw;
          if (uw >= hwd) {
            uw -= hwd;
            ++uh;
          }
        }
    }
  }
  // B operands of the mask MFMA (16x16x32): lane (q16, g) holds rows
  // 8g .. 8g+7 of column q16.  Row 8g + i carries query 4g + (i & 3) of the
  // even tile of a pair (i < 4) or of the odd one (i >= 4); the identity
  // picks one of the two
  bf16x8 ident_e, ident_o;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool hit = 4 * g + (i & 3) == q16;
    ident_e[i] = (__bf16)((hit && i < 4) ? 1.f : 0.f);
    ident_o[i] = (__bf16)((hit && i >= 4) ? 1.f : 0.f);
  }

  // ---- operand offsets inside one plane buffer; tiles add multiples of 16
  // rows, which leave the swizzle unchanged
  // K operand: lane (q16, g) holds key kp of a tile; V operand (transpose
  // read): lane (4j + a) of group g addresses key vp = key_perm(4g + j)
  const int vp = key_perm(HD, 4 * g + (q16 >> 2));
  int kofs[KSTEPS], vofs[MT];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) kofs[ks] = k_addr<HD>(rb + kp, 4 * ks + g);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) vofs[mt] = v_addr<HD>(rb + vp, mt, q16);

  // (b, n) of q and out (wave-uniform; plane t adds t * sT), and this
  // lane's query token within a plane, in bytes
  const uint16_t* const qbase = a.q + (int64_t)b * a.sq.b + (int64_t)n * a.sq.n;
  uint16_t* const obase = a.o + (int64_t)b * a.so.b + (int64_t)n * a.so.n;
  const uint32_t qoff = (uint32_t)(2 * ((int64_t)qhc * a.sq.h + (int64_t)qwc * a.sq.w));
  const uint32_t ooff = (uint32_t)(2 * ((int64_t)qhc * a.so.h + (int64_t)qwc * a.so.w));
  // with two-plane blocks, the same for the lane's plane pt of a block
  // (32-bit: the host keeps one plane step plus one spatial plane below
  // 4 GiB for these variants); qoff alone where that plane is past the box
  const uint32_t qoff_pt = qoff + (uint32_t)pt * (uint32_t)(2 * a.sq.t);
  const uint32_t ooff_pt = ooff + (uint32_t)pt * (uint32_t)(2 * a.so.t);
  // Q of the block at plane t (lanes whose plane is past the box keep stale
  // registers: their queries are masked and never stored)
  auto load_q_block = [&](bf16x8 (&qf)[KSTEPS], int t) __attribute__((always_inline)) {
    if (PT == 1 || t + pt < a.Tq) load_q<HD>(qf, qbase + (int64_t)t * a.sq.t, qoff_pt, g);
  };

  // ---- DMA staging walk: round k moves chunks [k*NT, (k+1)*NT); lane P of a
  // wave lands at chunk P of the buffer (row P / CPR, physical chunk P % CPR).
  // A thread's source offsets (bytes within a plane) advance by RSTEP halo
  // rows per round; they are the same for every plane.
  const int pc = stid % CPR;
  const int row0 = stid / CPR;
  const int step_h = RSTEP / hwd, step_w = RSTEP % hwd;
  // byte steps of K/V along W and H (32-bit: the host keeps one head's
  // spatial plane below 4 GiB for this family; wrapping arithmetic is exact)
  const uint32_t sw_b = (uint32_t)(a.sk.w * 2), sh_b = (uint32_t)(a.sk.h * 2);
  const uint32_t dstep = (uint32_t)step_h * sh_b + (uint32_t)step_w * sw_b;  // one round
  const uint32_t dwrap = sh_b - (uint32_t)hwd * sw_b;                       // halo row carry
  const int rw0 = row0 % hwd;
  const uint32_t d0 = (uint32_t)(hh0 + row0 / hwd) * sh_b + (uint32_t)(hw0 + rw0) * sw_b;
  const uint16_t* const kbase = a.k + (int64_t)b * a.sk.b + (int64_t)n * a.sk.n;
  const uint16_t* const vbase = a.v + (int64_t)b * a.sv.b + (int64_t)n * a.sk.n;
  // When a round advances a multiple of 16 rows, a lane's swizzled chunk is
  // the same in every round and is folded into its start offset.
  constexpr bool kFixedSwz = RSTEP % 16 == 0;
  const uint32_t d0s = d0 + (kFixedSwz ? (uint32_t)((pc ^ swz(HD, row0)) << 4) : 0u);
  const int full_rounds = total_chunks / NT;  // rounds in which every lane has a chunk
  // With the swizzle folded in, a lane's offset only advances: by dstep per
  // round, plus dwrap where its halo column wraps to the next row.  Which
  // rounds wrap is the same for every plane, so it is worked out once, as a
  // bit per round (the host keeps every plan within 32 rounds; LDS capacity
  // alone bounds them by 27).
  constexpr bool kWrapBits = kFixedSwz;
  uint32_t wbits = 0;
  if (kWrapBits) {
    int rw = rw0;
    for (int r = 0; r < full_rounds; ++r) {
      rw += step_w;
      if (rw >= hwd) {
        rw -= hwd;
        wbits |= 1u << r;
      }
    }
  }
  auto issue_stage = [&](int tp, int bufi) {
    const uint16_t* kpl = kbase + (int64_t)tp * a.sk.t;
    const uint16_t* vpl = vbase + (int64_t)tp * a.sv.t;
    const uint32_t dk = lds_addr(smem + bufi * 2 * buf_bytes + swave * kWave * 16);
    if constexpr (kWrapBits) {
      uint32_t d = d0s;
      int r = 0;
      for (; r < full_rounds; ++r) {
        dma16_kv(kpl, vpl, d, dk + r * NT * 16, buf_bytes);
        d += dstep + (dwrap & (uint32_t)__builtin_amdgcn_sbfe((int)wbits, r, 1));
      }
      if (r * NT + stid < total_chunks) dma16_kv(kpl, vpl, d, dk + r * NT * 16, buf_bytes);
      return;
    }
    uint32_t d = d0s;
    int rw = rw0, row = row0;
    auto advance = [&]() {
      d += dstep;
      rw += step_w;
      row += RSTEP;
      if (rw >= hwd) {
        rw -= hwd;
        d += dwrap;
      }
    };
    auto lane_ofs = [&]() { return kFixedSwz ? d : d + (uint32_t)((pc ^ swz(HD, row)) << 4); };
    int r = 0;
    for (; r < full_rounds; ++r) {
      dma16_kv(kpl, vpl, lane_ofs(), dk + r * NT * 16, buf_bytes);
      advance();
    }
    if (r * NT + stid < total_chunks) dma16_kv(kpl, vpl, lane_ofs(), dk + r * NT * 16, buf_bytes);
  };

  // The same walk by a subset of the waves: the wave of rank `rank` among
  // `nst` staging waves moves chunks rank*64 + lane + k*nst*64.  Used with
  // two buffers and HD >= 128, where the waves that have no query plane in
  // flight at a key plane stage the next one while the others compute (the
  // compute of a key plane is long enough to cover the slower issue; at
  // smaller HD the plane then lands late and this measured slower).
  constexpr bool kIdleStaging = NBUF == 2 && HD >= 128 && PT == 1 && PW == 0;
  auto issue_stage_by = [&](int tp, int bufi, int rank, int nst) {
    const uint16_t* kpl = kbase + (int64_t)tp * a.sk.t;
    const uint16_t* vpl = vbase + (int64_t)tp * a.sv.t;
    const uint32_t dk = lds_addr(smem + bufi * 2 * buf_bytes);
    const int c_first = rank * kWave + lane;
    const int rs = nst * (kWave / CPR);        // halo rows per round
    const int rs_h = rs / hwd, rs_w = rs - rs_h * hwd;
    int row = c_first / CPR;
    const int pcs = c_first - row * CPR;
    int rw = row % hwd;
    uint32_t d = (uint32_t)(hh0 + row / hwd) * sh_b + (uint32_t)(hw0 + rw) * sw_b;
    const uint32_t ds = (uint32_t)rs_h * sh_b + (uint32_t)rs_w * sw_b;
    for (int c0 = rank * kWave; c0 < total_chunks; c0 += nst * kWave) {
      if (c0 + lane < total_chunks)
        dma16_kv(kpl, vpl, d + (uint32_t)((pcs ^ swz(HD, row)) << 4), dk + c0 * 16, buf_bytes);
      d += ds;
      row += rs;
      rw += rs_w;
      if (rw >= hwd) {
        rw -= hwd;
        d += dwrap;
      }
    }
  };

  // zero the rows past the halo in every buffer (never staged; read only as
  // masked keys); the first barrier of the stream orders these stores
  {
    const int pad16 = (a.lds_rows - halo_rows) * (RB / 16);
    for (int i = tid; i < 2 * NBUF * pad16; i += NTA) {
      const int region = i / pad16;
      *reinterpret_cast<uint4*>(smem + region * buf_bytes + halo_rows * RB + (i - region * pad16) * 16) =
          make_uint4(0, 0, 0, 0);
    }
  }

  // the workgroup streams the key planes of runs [r_lo, r_hi) one after the
  // other; within a run, this wave's query planes are t0 + it + WT * j,
  // j = 0, 1, ..., held in slot j % NS
  Slot<HD> S[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) S[s].qf[ks] = bf16x8{};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) S[s].acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    S[s].accl = f32x4{0.f, 0.f, 0.f, 0.f};
    reset_state(S[s]);
  }
  bf16x8 qn[KSTEPS];          // Q of query plane qn_t, fetched one key plane early
  int qn_t = -1;
  uint32_t pend[2 * MT];      // packed output of a retired query plane ...
  uint16_t* pend_p = a.o;     // ... and its plane (wave-uniform)
  bool pend_on = false;
  bool pend_ok = false;       // ... and whether this lane's query is stored
  int t0, t1;
  run_bounds(r_lo, t0, t1);
  if (PW == 0 || stager) issue_stage(wst(t0), 0);  // step st uses buffer st % NBUF
  int st = 0;
  for (int ri = r_lo; ri < r_hi; ++ri) {
    if (ri > r_lo) run_bounds(ri, t0, t1);
    const int p0 = wst(t0), p1 = wst(t1 - 1) + KT;  // the run's key planes
    int nt0 = 0, nt1 = 0, np0 = -1;  // the next run, whose first plane follows p1 - 1
    if (ri + 1 < r_hi) {
      run_bounds(ri + 1, nt0, nt1);
      np0 = wst(nt0);
    }
    // this wave's blocks: block j covers query planes [tq(j), tq_last(j)]
    auto tq = [&](int j) { return t0 + PT * (it + WT * j); };
    auto tq_last = [&](int j) { return min(tq(j) + PT - 1, t1 - 1); };
    int jlo = 0, jhi = -1;  // blocks j in [jlo, jhi] are in flight
    // query planes [alo, ahi] of the run (any wave) are in flight
    int alo = t0, ahi = t0 - 1;
    for (int tp = p0; tp < p1; ++tp, ++st) {
      if (kIdleStaging) {
        while (ahi + 1 < t1 && wst(ahi + 1) <= tp) ++ahi;
        while (alo <= ahi && wst(alo) + KT - 1 < tp) ++alo;
      }
      // admit this wave's query planes whose window starts here
      while (computes && tq(jhi + 1) < t1 && wst(tq(jhi + 1)) <= tp) {
        ++jhi;
        const int sl = jhi % NS;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          if (s == sl) {
            if (qn_t == tq(jhi)) {
#pragma unroll
              for (int ks = 0; ks < KSTEPS; ++ks) S[s].qf[ks] = qn[ks];
            } else {
              load_q_block(S[s].qf, tq(jhi));
            }
            reset_state(S[s]);
          }
      }
      // plane tp has landed (with every earlier load and store of this wave);
      // with two buffers every wave is also done with the previous step,
      // whose buffer is refilled next
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (pend_on) {
        if (pend_ok) store_out<MT>(pend_p, ooff_pt, pend, g);
        pend_on = false;
      }
      const int nxt = tp + 1 < p1 ? tp + 1 : np0;  // plane of the next step, -1 = none
      if (NBUF == 2 && nxt >= 0 && !kIdleStaging) {
        if (PW == 0 || stager) issue_stage(nxt, (st + 1) & 1);
      } else if (NBUF == 2 && nxt >= 0) {
        // waves with nothing to compute at this key plane stage the next one
        // (all waves when none is idle): a wave of phase i is busy when one of
        // the in-flight planes [alo, ahi] is congruent to t0 + i mod WT
        const int nin = ahi - alo + 1;
        const int ph = (alo - t0) % WT;
        uint32_t busy_ph = nin >= WT ? (1u << WT) - 1u
                                     : ((((1u << nin) - 1u) << ph) | (((1u << nin) - 1u) >> (WT - ph))) &
                                           ((1u << WT) - 1u);
        uint32_t idle = 0;
#pragma unroll
        for (int w = 0; w < WH * WT; ++w) {
          const bool blk = h0 + (w % WH) * QH < Hq;
          if (!blk || !((busy_ph >> (w / WH)) & 1u)) idle |= 1u << w;
        }
        if (idle == 0) {
          issue_stage(nxt, (st + 1) & 1);
        } else if ((idle >> wave) & 1u) {
          issue_stage_by(nxt, (st + 1) & 1, __builtin_popcount(idle & ((1u << wave) - 1u)),
                         __builtin_popcount(idle));
        }
      }
      // fetch Q of the query plane (if any) this wave admits at the next step
      if (computes) {
        int tn = -1;
        if (tp + 1 < p1) {
          if (tq(jhi + 1) < t1 && wst(tq(jhi + 1)) == tp + 1) tn = tq(jhi + 1);
        } else if (np0 >= 0 && nt0 + PT * it < nt1 && wst(nt0 + PT * it) == np0) {
          tn = nt0 + PT * it;
        }
        if (tn >= 0) {
          load_q_block(qn, tn);
          qn_t = tn;
        }
      }

      if (active && jhi >= jlo) {
        // two-plane blocks: key plane tp is outside the window of a lane
        // whose query plane does not reach it (or lies past the run).  With
        // the mask MFMA its scores then start at -2^100 on top of the spatial
        // mask; with the mask table its max is left out (the reference max
        // stays) and its weights are computed against +2^100, i.e. are 0
        f32x4 tb4 = {0.f, 0.f, 0.f, 0.f};
        bool tout = false;
        if constexpr (PT > 1) {
          const int tl = tq(jlo) + pt;
          tout = !(tl < t1 && wst(tl) <= tp && tp < wst(tl) + KT);
          const float tb = tout ? __builtin_bit_cast(float, kMaskBits << 16) : 0.f;
          tb4 = f32x4{tb, tb, tb, tb};
        }
        const unsigned char* lk = smem + (NBUF == 2 ? (st & 1) : 0) * 2 * buf_bytes;
        const unsigned char* lv = lk + buf_bytes;
        // Work unit u = (group u / NS, slot u % NS).  Units run as a software
        // pipeline: while unit u's weights are exponentiated (VALU), the
        // scores of unit u+1 and the P.V products of unit u-1 (MFMA) are in
        // flight, all in one branch-free region.  Free slots run too (on
        // stale Q; admission resets the slot), so the regions stay
        // branch-free; only the rare rescale of the running output branches.
        constexpr int NU = NG * NS;
        constexpr int NPP = (NK + 1) / 2;  // P operands (tile pairs) per unit
        f32x4 sc[2][NK];
        bf16x8 pf[2][NPP];
        // S^T = K . Q^T + mask for every tile of unit u
        auto unit_scores = [&](int u, f32x4 (&out)[NK]) __attribute__((always_inline)) {
          const int gi = u / NS, sl = u % NS;
          const int gofs = GK * gi * RB;
          auto load_k = [&](int c, bf16x8 (&kf)[KSTEPS]) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
              kf[ks] = (32 * ks + 8 * g < HD)
                           ? *reinterpret_cast<const bf16x8*>(lk + kofs[ks] + gofs + 16 * c * RB)
                           : bf16x8{};
          };
          // The chains of two tiles at a time, interleaved, so one tile's
          // dependent MFMA never waits directly on the previous one; one tile
          // at a time where a second K fragment set would not fit the register
          // cap of the variant.
          constexpr int kPair = (OCC > 0 && (NG > 1 || PT > 1)) ? 1 : 2;
          if constexpr (kPair == 1) {
#pragma unroll
            for (int c = 0; c < NK; ++c) {
              bf16x8 kf[KSTEPS];
              load_k(c, kf);
              if constexpr (kMaskTable) {
                out[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], S[sl].qf[0], mc[gi][c], 0, 0, 0);
              } else {
                out[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, mk[gi][c >> 1]), (c & 1) ? ident_o : ident_e, tb4, 0, 0, 0);
                out[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], S[sl].qf[0], out[c], 0, 0, 0);
              }
#pragma unroll
              for (int ks = 1; ks < KSTEPS; ++ks)
                out[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], S[sl].qf[ks], out[c], 0, 0, 0);
            }
          } else {
#pragma unroll
            for (int c0 = 0; c0 < NK; c0 += kPair) {
              bf16x8 kf[kPair][KSTEPS];
#pragma unroll
              for (int t = 0; t < kPair; ++t)
                if (c0 + t < NK) load_k(c0 + t, kf[t]);
              if constexpr (!kMaskTable) {
                // the window mask of tile c: the pair's mask against the
                // identity half that selects tile c (same MFMA kind as the
                // score chain, whose accumulator it seeds)
#pragma unroll
                for (int t = 0; t < kPair; ++t)
                  if (c0 + t < NK)
                    out[c0 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, mk[gi][(c0 + t) >> 1]),
                        ((c0 + t) & 1) ? ident_o : ident_e, tb4, 0, 0, 0);
              }
#pragma unroll
              for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
                for (int t = 0; t < kPair; ++t) {
                  const int c = c0 + t;
                  if (c >= NK) continue;
                  f32x4 acc_in;
                  if constexpr (kMaskTable)
                    acc_in = ks == 0 ? mc[gi][c] : out[c];
                  else
                    acc_in = out[c];
                  out[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][ks], S[sl].qf[ks], acc_in, 0, 0, 0);
                }
            }
          }
        };
        // max of unit u's scores; the reference max moves (and the running
        // output is rescaled) only when a real score (not a mask value)
        // exceeds it by more than kRescale
        auto unit_max = [&](int u, const f32x4 (&in)[NK]) __attribute__((always_inline)) {
          const int sl = u % NS;
          // a chain of three-input maxes: two new scores per instruction
          float mx = __builtin_fmaxf(__builtin_fmaxf(in[0][0], in[0][1]), in[0][2]);
#pragma unroll
          for (int i = 3; i + 1 < 4 * NK; i += 2)
            mx = __builtin_fmaxf(__builtin_fmaxf(mx, in[i >> 2][i & 3]), in[(i + 1) >> 2][(i + 1) & 3]);
          if ((4 * NK - 3) & 1) mx = __builtin_fmaxf(mx, in[NK - 1][3]);
          mx = xmax4(mx);
          if constexpr (PT > 1 && kMaskTable) mx = tout ? kNegInf : mx;
          if (__builtin_amdgcn_ballot_w64(mx > S[sl].m + kRescale && mx > kRealScore) != 0) {
            const float mn = mx > kRealScore ? fmaxf(S[sl].m, mx) : S[sl].m;
            const float alpha = S[sl].m == kNegInf ? 0.f : __builtin_amdgcn_exp2f((S[sl].m - mn) * kLog2e);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) S[sl].acc[mt] *= alpha;
            S[sl].accl *= alpha;
            S[sl].m = mn;
          }
        };
        // weights of unit u as bf16 P^T operands (an odd last tile padded
        // with zero weights)
        auto unit_exp = [&](int u, const f32x4 (&in)[NK], bf16x8 (&out)[NPP]) __attribute__((always_inline)) {
          const int sl = u % NS;
          float mb = S[sl].m == kNegInf ? 0.f : S[sl].m * kLog2e;
          if constexpr (PT > 1 && kMaskTable) mb = tout ? 0x1p100f : mb;
#pragma unroll
          for (int c = 0; c < NK; ++c) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              out[c >> 1][4 * (c & 1) + r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(in[c][r], kLog2e, -mb));
          }
          if (ODD) {
#pragma unroll
            for (int r = 4; r < 8; ++r) out[NPP - 1][r] = (__bf16)0.f;
          }
        };
        // O^T += V^T . P^T and the denominator for unit u
        auto unit_pv = [&](int u, const bf16x8 (&in)[NPP]) __attribute__((always_inline)) {
          const int gi = u / NS, sl = u % NS;
          const int gofs = GK * gi * RB;
#pragma unroll
          for (int pi = 0; pi < NPP; ++pi) {
            bf16x8 vf[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const s16x4 lo = load_vt(lv, vofs[mt] + gofs + 32 * pi * RB);
              // the padded half of an odd last tile re-reads the same rows
              const s16x4 hi = (ODD && pi == NPP - 1) ? lo : load_vt(lv, vofs[mt] + gofs + (32 * pi + 16) * RB);
              vf[mt] = cat8(lo, hi);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              S[sl].acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[mt], in[pi], S[sl].acc[mt], 0, 0, 0);
            S[sl].accl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes8, in[pi], S[sl].accl, 0, 0, 0);
          }
        };
        // keeps unit u's weights computed where they stand in the pipeline
        // (the compiler would otherwise sink them past the next branch)
        auto pin = [&](bf16x8 (&w)[NPP]) __attribute__((always_inline)) {
#pragma unroll
          for (int pi = 0; pi < NPP; ++pi) asm volatile("" : "+v"(w[pi]));
        };
        unit_scores(0, sc[0]);
        unit_max(0, sc[0]);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          unit_exp(u, sc[u & 1], pf[u & 1]);
          if (u + 1 < NU) unit_scores(u + 1, sc[(u + 1) & 1]);
          if (NS >= 2) {
            // unit u + 1 belongs to another query plane: the previous unit's
            // products can share this region
            if (u >= 1) unit_pv(u - 1, pf[(u - 1) & 1]);
            pin(pf[u & 1]);
            if (u + 1 < NU) unit_max(u + 1, sc[(u + 1) & 1]);
          } else {
            pin(pf[u & 1]);
            // one query plane: its products must land before the next
            // unit's max may rescale the running output.  With 11- and
            // 13-tile groups the P.V phase runs at a raised wave priority, so
            // a wave entering it issues its MFMAs ahead of the co-resident
            // waves' softmax work and the MFMA and VALU phases of the waves on
            // a SIMD stay staggered (3-4% on the 11x11x11 grid; no change on
            // the 7-tile variants, where it is left out)
            if constexpr (NK >= 11) __builtin_amdgcn_s_setprio(2);
            unit_pv(u, pf[u & 1]);
            if constexpr (NK >= 11) __builtin_amdgcn_s_setprio(0);
            if (u + 1 < NU) unit_max(u + 1, sc[(u + 1) & 1]);
          }
        }
        if (NS >= 2) unit_pv(NU - 1, pf[(NU - 1) & 1]);
      }

      // retire this wave's query planes whose window ends here; the output
      // waits in registers for the next barrier (a second one in the same
      // plane is stored at once)
      while (jlo <= jhi && wst(tq_last(jlo)) + KT - 1 == tp) {
        const int sl = jlo % NS;
        if (active) {
          if (pend_on && pend_ok) store_out<MT>(pend_p, ooff_pt, pend, g);
#pragma unroll
          for (int s = 0; s < NS; ++s)
            if (s == sl) {
              // an empty asm on the accumulators keeps the normalisation here,
              // on the retiring step: hoisted out of this branch, the compiler
              // ran it on every step, waiting each time for the step's P.V
              // MFMAs to land before the wave could go on to the barrier
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) asm volatile("" : "+v"(S[s].acc[mt]));
              asm volatile("" : "+v"(S[s].accl));
              pack_out<HD>(S[s], pend);
            }
          pend_p = obase + (int64_t)tq(jlo) * a.so.t;
          pend_ok = qvalid && tq(jlo) + pt < t1;
          pend_on = true;
        }
        ++jlo;
      }
      // one buffer: every wave must be done with plane tp before it is refilled
      if (NBUF == 1 && nxt >= 0) {
        __syncthreads();
        if (PW == 0 || stager) issue_stage(nxt, 0);
      }
    }
  }
  if (pend_on && pend_ok) store_out<MT>(pend_p, ooff_pt, pend, g);
}

template <int HD, int QH, int QW, int WH, int WT, int NS, int NK, int NG, int NBUF, int OCC, int PW>
__global__ void __launch_bounds__(kWave * (WH * WT + PW)) __attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1)))
na3d_fwd_roll_kernel(const RollArgs a) {
  roll_body<HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW, true>(a, xcd_remap(blockIdx.x, gridDim.x));
}

// Many grids in one launch: the launch's workgroups are the tiles' grids one
// after another; a workgroup finds its tile (the last whose first workgroup
// is not after it) and runs that tile's problem exactly as a launch of that
// tile alone would (same staging layout, so the same arithmetic), with the
// window and heads shared by all tiles and LDS sized for the largest.
template <int HD, int QH, int QW, int WH, int WT, int NS, int NK, int NG, int NBUF, int OCC, int PW>
__global__ void __launch_bounds__(kWave * (WH * WT + PW)) __attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1)))
na3d_fwd_roll_batch_kernel(const RollArgs shared, const RollBatch bt) {
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  int i = 0;
  while (i + 1 < bt.n && bt.t[i + 1].wg_off <= wg) ++i;
  const BatchTile& t = bt.t[i];
  RollArgs a = shared;
  a.q = t.q; a.k = t.k; a.v = t.v; a.o = t.o;
  a.B = t.B; a.T = t.T; a.H = t.H; a.W = t.W;
  a.t_off = 0; a.h_off = 0; a.w_off = 0;
  a.Tq = t.T; a.Hq = t.H; a.Wq = t.W;
  a.tiles_t = t.tiles_t; a.tiles_h = t.tiles_h; a.tiles_w = t.tiles_w;
  a.tc = t.tc; a.ta = t.ta; a.tz = t.tz; a.nruns = t.nruns; a.rpw = t.rpw;
  a.lds_rows = t.lds_rows;
  a.band_h = 1;
  a.dv_tt = plain_udiv((uint32_t)t.tiles_t);
  a.dv_nt = plain_udiv((uint32_t)(t.tiles_h * t.tiles_w));
  a.dv_br = plain_udiv((uint32_t)t.tiles_w);
  a.dv_bh = plain_udiv(1u);
  a.dv_bl = plain_udiv(1u);
  a.dv_nh = plain_udiv((uint32_t)a.NH);
  Strides c;
  c.n = HD;
  c.w = (int64_t)a.NH * HD;
  c.h = (int64_t)t.W * c.w;
  c.t = (int64_t)t.H * c.h;
  c.b = (int64_t)t.T * c.t;
  a.sq = a.sk = a.sv = a.so = c;
  roll_body<HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW, false>(a, wg - t.wg_off);
}

// ------------------------------------------------------------------ launch
template <int HD, int QH, int QW, int WH, int WT, int NS, int NK, int NG, int NBUF, int OCC, int PW>
int launch_cfg(const RollArgs& a, const Launch& l, hipStream_t stream) {
  constexpr auto kern = na3d_fwd_roll_kernel<HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW>;
  if (set_lds<kern>(l.lds_bytes) != 0) return -1;
  hipLaunchKernelGGL(kern, dim3((unsigned)l.wgs), dim3(l.threads), l.lds_bytes, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int HD, int QH, int QW, int WH, int WT, int NS, int NK, int NG, int NBUF, int OCC, int PW>
int launch_batch_cfg(const RollArgs& a, const RollBatch& bt, const Launch& l, hipStream_t stream) {
  constexpr auto kern = na3d_fwd_roll_batch_kernel<HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW>;
  if (set_lds<kern>(l.lds_bytes) != 0) return -1;
  hipLaunchKernelGGL(kern, dim3((unsigned)l.wgs), dim3(l.threads), l.lds_bytes, stream, a, bt);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_roll(const Problem& p, const Launch& l, int hd, hipStream_t s) {
  RollArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o;
  a.B = p.B; a.T = p.T; a.H = p.H; a.W = p.W; a.NH = p.NH;
  a.t_off = p.box.t0; a.h_off = p.box.h0; a.w_off = p.box.w0;
  a.Tq = p.box.Tq; a.Hq = p.box.Hq; a.Wq = p.box.Wq;
  a.KT = p.KT; a.KH = p.KH; a.KW = p.KW;
  a.tiles_t = l.tiles_t;
  a.tiles_h = l.tiles_h;
  a.tiles_w = l.tiles_w;
  a.tc = l.tile_t;
  a.ta = l.ta;
  a.tz = l.tz;
  a.nruns = l.nruns;
  a.rpw = l.rpw;
  a.lds_rows = l.lds_rows;
  a.band_h = l.band_h;
  {
    const int nbands = (l.tiles_h + l.band_h - 1) / l.band_h;
    a.dv_tt = make_udiv((uint32_t)l.tiles_t);
    a.dv_nt = make_udiv((uint32_t)(l.tiles_h * l.tiles_w));
    a.dv_br = make_udiv((uint32_t)(l.band_h * l.tiles_w));
    a.dv_bh = make_udiv((uint32_t)l.band_h);
    a.dv_bl = make_udiv((uint32_t)(l.tiles_h - (nbands - 1) * l.band_h));
    a.dv_nh = make_udiv((uint32_t)p.NH);
  }
  a.sq = p.sq;
  a.sk = p.sk;
  a.sv = p.sv;
  a.so = p.so;
  if (l.variant < 0 || l.variant >= kNumRollVariants || kRollVariants[l.variant].hd != hd) return -1;
  switch (l.variant) {
#define NA3D_ROLL_CASE(i, HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW) \
  case i: return launch_cfg<HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW>(a, l, s);
    NA3D_ROLL_VARIANTS(NA3D_ROLL_CASE)
#undef NA3D_ROLL_CASE
    default: return -1;
  }
}

int launch_roll_batch(const Problem& p, const Launch& l, const RollBatch& bt, int hd,
                      hipStream_t s) {
  RollArgs a;
  a.q = a.k = a.v = nullptr;
  a.o = nullptr;
  a.B = a.T = a.H = a.W = 0;
  a.NH = p.NH;
  a.t_off = a.h_off = a.w_off = 0;
  a.Tq = a.Hq = a.Wq = 0;
  a.KT = p.KT; a.KH = p.KH; a.KW = p.KW;
  a.tiles_t = a.tiles_h = a.tiles_w = 0;
  a.tc = a.ta = a.tz = a.nruns = a.rpw = 0;
  a.lds_rows = l.lds_rows;
  a.band_h = 1;
  a.sq = a.sk = a.sv = a.so = Strides{0, 0, 0, 0, 0};
  a.dv_tt = a.dv_nt = a.dv_br = a.dv_bh = a.dv_bl = a.dv_nh = plain_udiv(1u);  // set per tile
  if (l.variant < 0 || l.variant >= kNumRollVariants || kRollVariants[l.variant].hd != hd) return -1;
  if (bt.n < 1 || bt.n > kMaxBatch) return -1;
  switch (l.variant) {
#define NA3D_ROLL_BATCH_CASE(i, HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW) \
  case i: return launch_batch_cfg<HD, QH, QW, WH, WT, NS, NK, NG, NBUF, OCC, PW>(a, bt, l, s);
    NA3D_ROLL_VARIANTS(NA3D_ROLL_BATCH_CASE)
#undef NA3D_ROLL_BATCH_CASE
    default: return -1;
  }
}

}  // namespace na3d
