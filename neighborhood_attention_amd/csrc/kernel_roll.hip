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
// planes t0 + it, t0 + it + WT, ... of the run.  All waves share the same
// query columns, so the union of a block's windows is one contiguous range of
// the staged halo rows: key u of the union sits in LDS row base + u, and
// every K/V operand address is a lane constant plus a block offset.
//
// The WG streams the key planes of the run in order.  Each plane's K/V halo
// is staged in LDS once, with direct global->LDS loads (global_load_lds
// dwordx4), into one or two plane buffers (with two, plane t'+1 is in flight
// while plane t' is computed).  Staged rows are unpadded and XOR-swizzled in
// 16-byte chunks (see swz), which keeps both operand reads free of bank
// conflicts.  A wave keeps the online-softmax state of up to NS of its query
// planes (a ring: a query plane is admitted when the stream reaches its
// window start and retired, output written, after its last key plane), and
// reuses every K/V fragment it reads from LDS for all of them.
//
// Within a 16-key tile the keys feed the MFMA rows in the order key_perm
// (chosen for conflict-free LDS reads); K rows, V rows and window masks all
// use that order.
//
// Per key plane, a wave walks its union in groups of up to SB 32-key blocks;
// each group runs three phases, each over all of its blocks and all active
// query planes, so the MFMAs and exponentials of a phase are independent:
//   S^T = K . Q^T + bias    bf16 MFMA 16x16x32; bias (0 or -inf) is the
//                           window mask, computed once per wave and fed in
//                           as the accumulator input, so masking costs no VALU
//   softmax                 one exact max over the group's scores, one
//                           rescale of the running output, then exp2
//   O^T += V^T . P^T        bf16 MFMA; the S^T accumulator layout is already
//                           the P^T operand, V^T comes from the transpose read
// The union's last partial block uses a 16-key step (MFMA 16x16x16) when it
// holds at most 16 keys.  Its masked keys read staged rows past the union;
// each plane buffer carries kPadRows zeroed rows past the halo, so such rows
// always hold finite values (which the -inf bias then removes).
#include "common.h"

namespace na3d {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr uint32_t kBf16NegInf = 0xff80u;

struct RollArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, T, H, W, NH;
  int KT, KH, KW;
  int tiles_t, tiles_h, tiles_w;
  int tc;        // query planes per workgroup
  int lds_rows;  // rows of each K and V staging buffer
};

template <int HD>
struct Slot {
  static constexpr int KSTEPS = (HD + 31) / 32;
  static constexpr int MT = HD / 16;
  bf16x8 qf[KSTEPS];  // Q^T operand: lane (q16, g) holds head dims [32ks + 8g, +8)
  f32x4 acc[MT];      // O^T: lane (q16, g) holds head dims 16mt + 4g + r
  float m;            // running max (natural units), -inf before any key
  float l;            // this lane's share of the softmax denominator
};

template <int HD>
__device__ __forceinline__ void load_q(Slot<HD>& S, const uint16_t* qp, int g) {
#pragma unroll
  for (int ks = 0; ks < Slot<HD>::KSTEPS; ++ks) {
    const int d = 32 * ks + 8 * g;
    S.qf[ks] = d < HD ? *reinterpret_cast<const bf16x8*>(qp + d) : bf16x8{};
  }
}

template <int HD>
__device__ __forceinline__ void reset_state(Slot<HD>& S) {
#pragma unroll
  for (int mt = 0; mt < Slot<HD>::MT; ++mt) S.acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  S.m = kNegInf;
  S.l = 0.f;
}

template <int HD>
__device__ __forceinline__ void slot_finish(Slot<HD>& S, uint16_t* op, int g, bool qvalid) {
  float l = S.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (qvalid) {
    const float inv = 1.f / l;
#pragma unroll
    for (int mt = 0; mt < Slot<HD>::MT; ++mt) {
      const bf16x2 lo = {(__bf16)(S.acc[mt][0] * inv), (__bf16)(S.acc[mt][1] * inv)};
      const bf16x2 hi = {(__bf16)(S.acc[mt][2] * inv), (__bf16)(S.acc[mt][3] * inv)};
      *reinterpret_cast<uint2*>(op + 16 * mt + 4 * g) =
          make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
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

// Window-mask bias of 8 scores packed as bf16 pairs (0 or -inf), expanded to
// the two f32x4 accumulator inputs of a 32-key block.
__device__ __forceinline__ void unpack_bias(const uint32_t (&w)[4], f32x4& b0, f32x4& b1) {
  b0 = f32x4{__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xffff0000u),
             __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xffff0000u)};
  b1 = f32x4{__builtin_bit_cast(float, w[2] << 16), __builtin_bit_cast(float, w[2] & 0xffff0000u),
             __builtin_bit_cast(float, w[3] << 16), __builtin_bit_cast(float, w[3] & 0xffff0000u)};
}

template <int HD, int QH, int QW, int WH, int WT, int NS, int MAXB, int NBUF, int SB>
__global__ void __launch_bounds__(kWave * WH * WT) na3d_fwd_roll_kernel(const RollArgs a) {
  constexpr int NGRP = (MAXB + 1 + SB - 1) / SB;  // groups covering MAXB full blocks + a tail
  static_assert(QH * QW == 16, "a wave owns 16 queries");
  static_assert(NBUF == 1 || NBUF == 2, "one or two plane buffers");
  constexpr int KSTEPS = Slot<HD>::KSTEPS;
  constexpr int MT = Slot<HD>::MT;
  constexpr int CPR = HD / 8;  // 16-byte chunks per staged row
  constexpr int RB = HD * 2;   // staged row bytes
  constexpr int BH = WH * QH;
  constexpr int NT = kWave * WH * WT;
  constexpr int RSTEP = NT / CPR;  // staged rows per DMA round

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
  const int ih = wave % WH;
  const int it = wave / WH;

  // ---- workgroup -> (b, n, tile_h, tile_w, tile_t); tile_t varies fastest
  int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int tt = wg % a.tiles_t;
  wg /= a.tiles_t;
  const int tw = wg % a.tiles_w;
  wg /= a.tiles_w;
  const int th = wg % a.tiles_h;
  wg /= a.tiles_h;
  const int n = wg % a.NH;
  const int b = wg / a.NH;

  const int T = a.T, H = a.H, W = a.W, KT = a.KT, KH = a.KH, KW = a.KW;
  const int t0 = tt * a.tc, t1 = min(t0 + a.tc, T);
  const int h0 = th * BH, w0 = tw * QW;
  const int h1 = min(h0 + BH, H) - 1, w1 = min(w0 + QW, W) - 1;
  // halo of the tile: rows [hh0, hh0 + hhn) x columns [hw0, hw0 + hwd)
  const int hh0 = win_start(h0, KH, H);
  const int hhn = win_start(h1, KH, H) + KH - hh0;
  const int hw0 = win_start(w0, KW, W);
  const int hwd = win_start(w1, KW, W) + KW - hw0;
  const int halo_rows = hhn * hwd;
  const int total_chunks = halo_rows * CPR;

  // ---- this wave's block of 16 queries
  const int bh0 = h0 + ih * QH;
  const bool active = bh0 < H && t0 + it < t1;
  const int bh1 = min(bh0 + QH, H) - 1;
  const int qh = bh0 + q16 / QW;
  const int qw = w0 + q16 % QW;
  const bool qvalid = active && qh < H && qw < W;
  const int qhc = min(qh, H - 1), qwc = min(qw, W - 1);
  const int ash = win_start(qhc, KH, H);
  const int asw = win_start(qwc, KW, W);
  // union of the block's windows = staged rows [base, base + un)
  const int uh0 = bh0 < H ? win_start(bh0, KH, H) : hh0;
  const int un = active ? (win_start(bh1, KH, H) + KH - uh0) * hwd : 0;
  const int base = (uh0 - hh0) * hwd;
  const int nblk = (un + 31) >> 5;  // 32-key blocks, the last possibly partial

  // ---- window masks, packed as bf16 pairs (0 = in window, -inf = out)
  const float inv_hwd = 1.f / (float)hwd;
  auto key_out = [&](int u) -> uint32_t {
    if (!qvalid || u >= un) return kBf16NegInf;
    int uh = (int)((float)u * inv_hwd);
    int uw = u - uh * hwd;
    if (uw < 0) { --uh; uw += hwd; }
    if (uw >= hwd) { ++uh; uw -= hwd; }
    const bool in = (unsigned)(uh0 + uh - ash) < (unsigned)KH &&
                    (unsigned)(hw0 + uw - asw) < (unsigned)KW;
    return in ? 0u : kBf16NegInf;
  };
  auto bias_words = [&](int u0, uint32_t (&w)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // score slot r of tile ct holds key 16ct + key_perm(4g + r)
      const int r = 2 * (i & 1);
      const int u = u0 + 16 * (i >> 1);
      w[i] = key_out(u + key_perm(HD, 4 * g + r)) | (key_out(u + key_perm(HD, 4 * g + r + 1)) << 16);
    }
  };
  uint32_t bias[MAXB + 1][4];  // MAXB full blocks and the tail
#pragma unroll
  for (int bb = 0; bb <= MAXB; ++bb) bias_words(32 * bb, bias[bb]);

  // ---- operand offsets inside one plane buffer; blocks add multiples of 16
  // rows, which leave the swizzle unchanged
  // K operand: lane (q16, g) holds key kp of a tile; V operand (transpose
  // read): lane (4j + a) of group g addresses key vp = key_perm(4g + j)
  const int kp = key_perm(HD, q16);
  const int vp = key_perm(HD, 4 * g + (q16 >> 2));
  int kofs[KSTEPS], vofs[MT];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) kofs[ks] = k_addr<HD>(base + kp, 4 * ks + g);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) vofs[mt] = v_addr<HD>(base + vp, mt, q16);

  const int64_t tok = (int64_t)a.NH * HD;
  const int64_t plane = (int64_t)H * W * tok;
  const int64_t bbase = (int64_t)b * T * plane + (int64_t)n * HD;
  const int64_t qtok = ((int64_t)qhc * W + qwc) * tok;

  // ---- DMA staging walk: round k moves chunks [k*NT, (k+1)*NT); lane P of a
  // wave lands at chunk P of the buffer (row P / CPR, physical chunk P % CPR)
  const int pc = tid % CPR;
  const int row0 = tid / CPR;
  const int step_h = RSTEP / hwd, step_w = RSTEP % hwd;
  const int row0_h = row0 / hwd, row0_w = row0 % hwd;
  auto issue_stage = [&](int tp, int bufi) {
    const uint16_t* kp = a.k + bbase + (int64_t)tp * plane;
    const uint16_t* vp = a.v + bbase + (int64_t)tp * plane;
    unsigned char* dk = smem + bufi * 2 * buf_bytes + wave * kWave * 16;
    unsigned char* dv = dk + buf_bytes;
    int rh = row0_h, rw = row0_w;
    for (int c0 = 0, row = row0; c0 < total_chunks; c0 += NT, row += RSTEP) {
      if (c0 + tid < total_chunks) {
        const int64_t off = ((int64_t)(hh0 + rh) * W + (hw0 + rw)) * tok + ((pc ^ swz(HD, row)) << 3);
        __builtin_amdgcn_global_load_lds(kp + off, (__attribute__((address_space(3))) void*)(dk + c0 * 16), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp + off, (__attribute__((address_space(3))) void*)(dv + c0 * 16), 16, 0, 0);
      }
      rh += step_h;
      rw += step_w;
      if (rw >= hwd) { rw -= hwd; ++rh; }
    }
  };

  // this wave's query planes: t0 + it + WT * j, j = 0, 1, ...; slot j % NS
  auto tq = [&](int j) { return t0 + it + WT * j; };
  Slot<HD> S[NS];
  unsigned preloaded = 0;  // slots whose Q was fetched one plane early
  int jlo = 0, jhi = -1;   // query planes j in [jlo, jhi] are in flight
  const int p0 = win_start(t0, KT, T), p1 = win_start(t1 - 1, KT, T) + KT;
  // zero the rows past the halo in every buffer (never staged; read only by
  // masked tail keys); the first barrier of the stream orders these stores
  {
    const int pad16 = (a.lds_rows - halo_rows) * (RB / 16);
    for (int i = tid; i < 2 * NBUF * pad16; i += NT) {
      const int region = i / pad16;
      *reinterpret_cast<uint4*>(smem + region * buf_bytes + halo_rows * RB + (i - region * pad16) * 16) =
          make_uint4(0, 0, 0, 0);
    }
  }
  issue_stage(p0, NBUF == 2 ? (p0 & 1) : 0);  // key plane tp lives in buffer tp % NBUF
  for (int tp = p0; tp < p1; ++tp) {
    // admit this wave's query planes whose window starts here
    while (tq(jhi + 1) < t1 && win_start(tq(jhi + 1), KT, T) <= tp) {
      ++jhi;
      const int sl = jhi % NS;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (s == sl) {
          if (!((preloaded >> s) & 1)) load_q(S[s], a.q + bbase + (int64_t)tq(jhi) * plane + qtok, g);
          reset_state(S[s]);
        }
      preloaded &= ~(1u << sl);
    }
    // plane tp has landed (own DMA + Q loads); with two buffers every wave is
    // also done with plane tp - 1, whose buffer is refilled next
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (NBUF == 2 && tp + 1 < p1) issue_stage(tp + 1, (tp + 1) & 1);
    // fetch Q of query planes that start at the next key plane, where their
    // slot is already free, so the load hides behind this plane's work
    for (int j = jhi + 1; tq(j) < t1 && win_start(tq(j), KT, T) == tp + 1; ++j) {
      if (j - NS >= jlo) break;
      const int sl = j % NS;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (s == sl) load_q(S[s], a.q + bbase + (int64_t)tq(j) * plane + qtok, g);
      preloaded |= 1u << sl;
    }

    if (active && jhi >= jlo) {
      const unsigned char* lk = smem + (NBUF == 2 ? (tp & 1) : 0) * 2 * buf_bytes;
      const unsigned char* lv = lk + buf_bytes;
      bool sact[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) sact[s] = ((s - jlo % NS + NS) % NS) < (jhi - jlo + 1);
      // The union is processed in groups of SB 32-key blocks; each group runs
      // three phases over all of its blocks and all active query planes:
      // scores, softmax (one exact group max, one rescale), P.V.
#pragma unroll
      for (int grp = 0; grp < NGRP; ++grp) {
        if (grp * SB >= nblk) break;
        f32x4 sc[NS][SB][2];
        // ---- phase 1: S^T = K . Q^T + mask for every block of the group
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          const int bi = grp * SB + j;
          if (bi > MAXB || bi >= nblk) break;
          const bool half = 32 * bi + 16 >= un;  // a tail of at most 16 keys
          bf16x8 kf[2][KSTEPS];
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            const bool use = 32 * ks + 8 * g < HD;
            const unsigned char* ka = lk + kofs[ks] + 32 * bi * RB;
            kf[0][ks] = use ? *reinterpret_cast<const bf16x8*>(ka) : bf16x8{};
            kf[1][ks] = bf16x8{};
            if (!half) kf[1][ks] = use ? *reinterpret_cast<const bf16x8*>(ka + 16 * RB) : bf16x8{};
          }
          f32x4 b0, b1;
          unpack_bias(bias[bi], b0, b1);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            sc[s][j][0] = b0;
            sc[s][j][1] = b1;
            if (!sact[s]) continue;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
              sc[s][j][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], S[s].qf[ks], sc[s][j][0], 0, 0, 0);
              if (!half)
                sc[s][j][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], S[s].qf[ks], sc[s][j][1], 0, 0, 0);
            }
          }
        }
        // ---- phase 2: softmax over the group (the masked half of a 16-key
        // tail block holds -inf and contributes nothing)
        bf16x8 pf[NS][SB];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (!sact[s]) continue;
          float mx = kNegInf;
#pragma unroll
          for (int j = 0; j < SB; ++j) {
            const int bi = grp * SB + j;
            if (bi > MAXB || bi >= nblk) break;
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fmaxf(sc[s][j][0][r], sc[s][j][1][r]));
          }
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mn = fmaxf(S[s].m, mx);
          const float alpha = S[s].m == kNegInf ? 0.f : __builtin_amdgcn_exp2f((S[s].m - mn) * kLog2e);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) S[s].acc[mt] *= alpha;
          S[s].m = mn;
          const float mb = mn == kNegInf ? 0.f : mn * kLog2e;
          float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
          for (int j = 0; j < SB; ++j) {
            const int bi = grp * SB + j;
            if (bi > MAXB || bi >= nblk) break;
            float p[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[s][j][0][r], kLog2e, -mb));
              p[4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[s][j][1][r], kLog2e, -mb));
            }
            sum0 += (p[0] + p[1]) + (p[2] + p[3]);
            sum1 += (p[4] + p[5]) + (p[6] + p[7]);
#pragma unroll
            for (int r = 0; r < 8; ++r) pf[s][j][r] = (__bf16)p[r];
          }
          S[s].l = S[s].l * alpha + (sum0 + sum1);
        }
        // ---- phase 3: O^T += V^T . P^T for every block of the group
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          const int bi = grp * SB + j;
          if (bi > MAXB || bi >= nblk) break;
          const bool half = 32 * bi + 16 >= un;
          if (half) {
            s16x4 vf[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) vf[mt] = load_vt(lv, vofs[mt] + 32 * bi * RB);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              if (!sact[s]) continue;
              const bf16x4 lo = {pf[s][j][0], pf[s][j][1], pf[s][j][2], pf[s][j][3]};
              const s16x4 pb = __builtin_bit_cast(s16x4, lo);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                S[s].acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[mt], pb, S[s].acc[mt], 0, 0, 0);
            }
          } else {
            bf16x8 vf[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              vf[mt] = cat8(load_vt(lv, vofs[mt] + 32 * bi * RB), load_vt(lv, vofs[mt] + (32 * bi + 16) * RB));
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              if (!sact[s]) continue;
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                S[s].acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[mt], pf[s][j], S[s].acc[mt], 0, 0, 0);
            }
          }
        }
        // keep the scheduler from hoisting the next group's operand reads
        // above this one, which would hold every group's fragments at once
        if (NGRP > 1) __builtin_amdgcn_sched_barrier(0);
      }
    }

    // retire this wave's query planes whose window ends here
    while (jlo <= jhi && win_start(tq(jlo), KT, T) + KT - 1 == tp) {
      const int sl = jlo % NS;
      uint16_t* op = a.o + bbase + (int64_t)tq(jlo) * plane + qtok;
      if (active) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
          if (s == sl) slot_finish(S[s], op, g, qvalid);
      }
      ++jlo;
    }
    // one buffer: every wave must be done with plane tp before it is refilled
    if (NBUF == 1 && tp + 1 < p1) {
      __syncthreads();
      issue_stage(tp + 1, 0);
    }
  }
}

// ------------------------------------------------------------------ launch
template <int HD, int QH, int QW, int WH, int WT, int NS, int MAXB, int NBUF, int SB>
int launch_cfg(const RollArgs& a, const Launch& l, hipStream_t stream) {
  auto kern = na3d_fwd_roll_kernel<HD, QH, QW, WH, WT, NS, MAXB, NBUF, SB>;
  if (l.lds_bytes > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, l.lds_bytes) != hipSuccess)
    return -1;
  hipLaunchKernelGGL(kern, dim3((unsigned)l.wgs), dim3(l.threads), l.lds_bytes, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_roll(const Problem& p, const Launch& l, int hd, hipStream_t s) {
  RollArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o;
  a.B = p.B; a.T = p.T; a.H = p.H; a.W = p.W; a.NH = p.NH;
  a.KT = p.KT; a.KH = p.KH; a.KW = p.KW;
  a.tiles_t = l.tiles_t;
  a.tiles_h = l.tiles_h;
  a.tiles_w = l.tiles_w;
  a.tc = l.tile_t;
  a.lds_rows = l.lds_rows;
  if (l.variant < 0 || l.variant >= kNumRollVariants || kRollVariants[l.variant].hd != hd) return -1;
  switch (l.variant) {
#define NA3D_ROLL_CASE(i, HD, QH, QW, WH, WT, NS, MAXB, NBUF, SB) \
  case i: return launch_cfg<HD, QH, QW, WH, WT, NS, MAXB, NBUF, SB>(a, l, s);
    NA3D_ROLL_VARIANTS(NA3D_ROLL_CASE)
#undef NA3D_ROLL_CASE
    default: return -1;
  }
}

}  // namespace na3d
