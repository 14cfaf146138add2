// kernel_general.hip -- the general NA3D forward family (gfx950).
//
// Operation: ROCm/aiter PR "Add 3D neighborhood flash attention (na3d_flash)",
// Motivation (each query token attends to a KT x KH x KW box of keys) and
// Technical Details (windows shifted inward at borders so each holds exactly
// KT*KH*KW keys; Q pre-scaled by head_dim^-0.5; online softmax in log2 space).
//
// One workgroup (WG) = batch b, head n, one query plane t and an 8 x 8
// spatial tile of queries.  The WG walks the KT key planes of its window; for
// each it stages the tile's K/V halo (the union of its queries' windows) in
// LDS, in chunks when the halo exceeds the LDS budget, and every wave handles
// its 4 x 4 query block against the union of that block's windows, flattened
// and cut into 32-key blocks:
//   S^T (16 keys x 16 queries) = K . Q^T          bf16 MFMA 16x16x32
//   window mask from the per-query clamped starts  (out-of-window -> -inf)
//   online softmax per query, fp32, exp2
//   O^T (16 hd x 16 queries) += V^T . P^T          bf16 MFMA 16x16x32
// The transposed orientation keeps one query per lane, so the running max
// and sum of a query live in the 4 lanes that share it, and the score
// accumulator of S^T is already the B operand of the P.V product.  V^T
// operands come straight from row-major LDS through the gfx950 transpose read
// (ds_read_b64_tr_b16), which also gathers arbitrary key rows.
//
// This family has no static limit on window size or union shape (key
// coordinates are decoded per block); the rolling family is used wherever its
// register-resident tables fit.
#include "common.h"

namespace na3d {
namespace {

constexpr int kLdsPad = 16;  // bytes of padding per staged K/V row

struct GeneralArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, T, H, W, NH;  // k and v grid
  int KT, KH, KW;
  int t_off, h_off, w_off;  // query box: q/out plane t is grid plane t_off + t, ...
  int Tq, Hq, Wq;           // ... and its extents
  int tiles_h, tiles_w;
  int lds_rows;  // capacity of each of the K and V staging buffers, in rows
  Strides sq, sk, sv, so;  // element strides; k and v share h, w and n
};

__device__ __forceinline__ void divmod(int u, int d, int& qo, int& ro) {
  qo = u / d;
  ro = u - qo * d;
}

// Number of keys of a union box (rows [0,uhn) x cols [0,uw), placed at
// offset (oh, ow) inside a halo of width hwd) whose halo flat index is < r.
__device__ __forceinline__ int union_keys_before(int r, int oh, int ow, int uhn, int uw, int hwd) {
  int hr = r / hwd - oh;
  int wr = r % hwd - ow;
  if (hr < 0) return 0;
  if (hr >= uhn) return uhn * uw;
  wr = wr < 0 ? 0 : (wr > uw ? uw : wr);
  return hr * uw + wr;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <int HD, int QH, int QW, int WH, int WW>
__global__ void __launch_bounds__(kWave * WH * WW)
na3d_fwd_general_kernel(const GeneralArgs a) {
  static_assert(QH * QW == 16, "a wave owns 16 queries");
  constexpr int BH = WH * QH;
  constexpr int BW = WW * QW;
  constexpr int KSTEPS = (HD + 31) / 32;  // MFMA k-steps over the head dim
  constexpr int MT = HD / 16;             // 16-wide output tiles over the head dim
  constexpr int ROW = HD * 2 + kLdsPad;   // LDS row stride (bytes)
  constexpr int PARTS = HD / 8;           // 16-byte pieces per row

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* lds_k = smem;
  unsigned char* lds_v = smem + (size_t)a.lds_rows * ROW;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int q16 = lane & 15;
  const int g = lane >> 4;

  // ---- workgroup -> (b, n, tile_h, tile_w, t); t varies fastest
  int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int t = wg % a.Tq;  // query plane in the box
  wg /= a.Tq;
  const int tw = wg % a.tiles_w;
  wg /= a.tiles_w;
  const int th = wg % a.tiles_h;
  wg /= a.tiles_h;
  const int n = wg % a.NH;
  const int b = wg / a.NH;

  const int H = a.H, W = a.W, KH = a.KH, KW = a.KW, Hq = a.Hq, Wq = a.Wq;
  // queries are indexed in the box, windows and K/V in the grid
  auto wsh = [&](int h) { return win_start(a.h_off + h, KH, H); };
  auto wsw = [&](int w) { return win_start(a.w_off + w, KW, W); };
  const int h0 = th * BH, w0 = tw * BW;
  const int h1 = min(h0 + BH, Hq) - 1, w1 = min(w0 + BW, Wq) - 1;
  // halo of the whole tile (grid coordinates), [hh0, hh0+hhn) x [hw0, hw0+hwd)
  const int hh0 = wsh(h0);
  const int hhn = wsh(h1) + KH - hh0;
  const int hw0 = wsw(w0);
  const int hwd = wsw(w1) + KW - hw0;
  const int halo_rows = hhn * hwd;
  const int st = win_start(a.t_off + t, a.KT, a.T);

  // ---- this wave's 16-query block
  const int bh0 = h0 + (wave / WW) * QH;
  const int bw0 = w0 + (wave % WW) * QW;
  const bool wave_active = bh0 < Hq && bw0 < Wq;
  const int bh1 = min(bh0 + QH, Hq) - 1;
  const int bw1 = min(bw0 + QW, Wq) - 1;
  const int qh = bh0 + q16 / QW;
  const int qw = bw0 + q16 % QW;
  const bool qvalid = wave_active && qh < Hq && qw < Wq;
  const int qhc = min(qh, Hq - 1), qwc = min(qw, Wq - 1);
  const int ash = wsh(qhc);  // query window start (grid)
  const int asw = wsw(qwc);
  // union of the block's windows, in grid coordinates
  const int uh0 = wave_active ? wsh(bh0) : hh0;
  const int uhn = wave_active ? wsh(bh1) + KH - uh0 : 0;
  const int uw0 = wave_active ? wsw(bw0) : hw0;
  const int uw = wave_active ? wsw(bw1) + KW - uw0 : 1;
  const int oh = uh0 - hh0, ow = uw0 - hw0;  // union origin inside the halo


  // ---- Q^T operand (B of S^T = K.Q^T): lane (q16, g) holds hd [32ks+8g, +8)
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.sq.b + (int64_t)t * a.sq.t + (int64_t)n * a.sq.n +
                         (int64_t)qhc * a.sq.h + (int64_t)qwc * a.sq.w;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int d = 32 * ks + 8 * g;
      if (d < HD)
        qf[ks] = *reinterpret_cast<const bf16x8*>(qp + d);
      else
        qf[ks] = bf16x8{};
    }
  }

  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  const int nchunk = (halo_rows + a.lds_rows - 1) / a.lds_rows;
  for (int dt = 0; dt < a.KT; ++dt) {
    const int tp = st + dt;
    const uint16_t* kplane = a.k + (int64_t)b * a.sk.b + (int64_t)tp * a.sk.t + (int64_t)n * a.sk.n;
    const uint16_t* vplane = a.v + (int64_t)b * a.sv.b + (int64_t)tp * a.sv.t + (int64_t)n * a.sk.n;
    for (int c = 0; c < nchunk; ++c) {
      const int r0 = c * a.lds_rows;
      const int r1 = min(r0 + a.lds_rows, halo_rows);
      // ---- stage halo rows [r0, r1) of K and V into LDS
      __syncthreads();
      const int pieces = (r1 - r0) * PARTS;
      for (int i = tid; i < pieces; i += blockDim.x) {
        const int row = i / PARTS, part = i % PARTS;
        const int fr = r0 + row;
        const int hp = hh0 + fr / hwd, wp = hw0 + fr % hwd;
        const int64_t off = (int64_t)hp * a.sk.h + (int64_t)wp * a.sk.w + part * 8;
        const uint4 kv = *reinterpret_cast<const uint4*>(kplane + off);
        const uint4 vv = *reinterpret_cast<const uint4*>(vplane + off);
        *reinterpret_cast<uint4*>(lds_k + row * ROW + part * 16) = kv;
        *reinterpret_cast<uint4*>(lds_v + row * ROW + part * 16) = vv;
      }
      __syncthreads();
      if (!wave_active) continue;

      // union keys whose halo row lies in [r0, r1): a contiguous index range
      const int u_lo = union_keys_before(r0, oh, ow, uhn, uw, hwd);
      const int u_hi = union_keys_before(r1, oh, ow, uhn, uw, hwd);
      for (int ub = u_lo; ub < u_hi; ub += 32) {
        // LDS row of union key u (row 0 for keys past u_hi: always masked)
        auto lds_row = [&](int u) -> int {
          if (u >= u_hi) return 0;
          int uh, uwr;
          divmod(u, uw, uh, uwr);
          return (oh + uh) * hwd + ow + uwr - r0;
        };
        // ---- S^T = K . Q^T for the two 16-key tiles of the block
        f32x4 s[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int row = lds_row(ub + 16 * ct + q16);
          s[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            const int d = 32 * ks + 8 * g;
            bf16x8 kf = bf16x8{};
            if (d < HD) kf = *reinterpret_cast<const bf16x8*>(lds_k + row * ROW + d * 2);
            s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[ct], 0, 0, 0);
          }
        }
        // ---- window mask: lane (q16, g) holds keys ub + 16ct + 4g + r
        float mx = -__builtin_inff();
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int u = ub + 16 * ct + 4 * g + r;
            bool ok = qvalid && u < u_hi;
            if (ok) {
              int uh, uwr;
              divmod(u, uw, uh, uwr);
              ok = (unsigned)(uh0 + uh - ash) < (unsigned)KH &&
                   (unsigned)(uw0 + uwr - asw) < (unsigned)KW;
            }
            if (!ok) s[ct][r] = -__builtin_inff();
            mx = fmaxf(mx, s[ct][r]);
          }
        }
        // ---- online softmax (the 4 lanes of a query are lanes q16 + 16g)
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha =
            (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e);
        const float mb = (m_new == -__builtin_inff()) ? 0.f : m_new * kLog2e;
        m_run = m_new;
        float psum = 0.f;
        bf16x8 pf;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ct][r], kLog2e, -mb));
            const __bf16 pb = (__bf16)p;
            pf[4 * ct + r] = pb;
            psum += (float)pb;
          }
        }
        l_run = l_run * alpha + psum;
        // ---- O^T += V^T . P^T; V^T slots come from the transpose read:
        // lane (4j + a) of a 16-lane group addresses key row 16c + 4g + j,
        // columns [16mt + 4a, +4).
        const int rv0 = lds_row(ub + 4 * g + (q16 >> 2));
        const int rv1 = lds_row(ub + 16 + 4 * g + (q16 >> 2));
        const unsigned char* pv0 = lds_v + rv0 * ROW + (q16 & 3) * 8;
        const unsigned char* pv1 = lds_v + rv1 * ROW + (q16 & 3) * 8;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt] *= alpha;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pv0 + mt * 32));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pv1 + mt * 32));
          bf16x8 vf;
          const bf16x4 lob = __builtin_bit_cast(bf16x4, lo);
          const bf16x4 hib = __builtin_bit_cast(bf16x4, hi);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vf[j] = lob[j];
            vf[4 + j] = hib[j];
          }
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[mt], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: full row sum over the 4 lanes of a query, O / l, bf16 store
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (qvalid) {
    const float inv = 1.f / l_run;
    uint16_t* op = a.o + (int64_t)b * a.so.b + (int64_t)t * a.so.t + (int64_t)n * a.so.n +
                   (int64_t)qh * a.so.h + (int64_t)qw * a.so.w;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[mt][0] * inv) |
                          ((uint32_t)f32_to_bf16_rne(acc[mt][1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[mt][2] * inv) |
                          ((uint32_t)f32_to_bf16_rne(acc[mt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + 16 * mt + 4 * g) = make_uint2(lo, hi);
    }
  }
}


constexpr int kQH = 4, kQW = 4, kWH = 2, kWW = 2;  // 8 x 8 query tile, 4 waves

template <int HD>
int launch_hd(const GeneralArgs& a, const Launch& l, hipStream_t stream) {
  constexpr auto kern = na3d_fwd_general_kernel<HD, kQH, kQW, kWH, kWW>;
  if (set_lds<kern>(l.lds_bytes) != 0) return -1;
  hipLaunchKernelGGL(kern, dim3((unsigned)l.wgs), dim3(l.threads), l.lds_bytes, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int general_tile_h() { return kWH * kQH; }
int general_tile_w() { return kWW * kQW; }
int general_threads() { return kWave * kWH * kWW; }
int general_row_bytes(int hd) { return hd * 2 + kLdsPad; }

int launch_general(const Problem& p, const Launch& l, int hd, hipStream_t s) {
  GeneralArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o;
  a.B = p.B; a.T = p.T; a.H = p.H; a.W = p.W; a.NH = p.NH;
  a.t_off = p.box.t0; a.h_off = p.box.h0; a.w_off = p.box.w0;
  a.Tq = p.box.Tq; a.Hq = p.box.Hq; a.Wq = p.box.Wq;
  a.KT = p.KT; a.KH = p.KH; a.KW = p.KW;
  a.tiles_h = l.tiles_h;
  a.tiles_w = l.tiles_w;
  a.lds_rows = l.lds_rows;
  a.sq = p.sq;
  a.sk = p.sk;
  a.sv = p.sv;
  a.so = p.so;
  switch (hd) {
    case 16: return launch_hd<16>(a, l, s);
    case 32: return launch_hd<32>(a, l, s);
    case 64: return launch_hd<64>(a, l, s);
    case 128: return launch_hd<128>(a, l, s);
    case 256: return launch_hd<256>(a, l, s);
    default: return -1;
  }
}

}  // namespace na3d
