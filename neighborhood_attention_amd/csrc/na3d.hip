// na3d.hip -- MI355X (gfx950) forward pass of 3-D neighborhood attention.
//
// Operation: ROCm/aiter PR "Add 3D neighborhood flash attention (na3d_flash)",
// Motivation (each query token attends to a KT x KH x KW box of keys) and
// Technical Details (windows shifted inward at borders so each holds exactly
// KT*KH*KW keys; Q pre-scaled by head_dim^-0.5; online softmax in log2 space).
//
// Structure of one workgroup (WG): batch b, head n, query plane t and a
// BH x BW spatial tile of queries.  The WG walks the KT key planes of its
// window; for each it stages the tile's K/V halo (the union of its queries'
// windows) in LDS with 16-byte loads, then every wave processes its own
// 16-query block (QH x QW queries) against the union of that block's windows,
// flattened and cut into 32-key blocks:
//   S^T (16 keys x 16 queries) = K . Q^T          bf16 MFMA 16x16x32
//   window mask from the per-query clamped starts  (out-of-window -> -inf)
//   online softmax per query, fp32, exp2
//   O^T (16 hd x 16 queries) += V^T . P^T          bf16 MFMA 16x16x32
// The transposed orientation keeps one query per lane, so the running max
// and sum of a query live in the 4 lanes that share it, and the score
// accumulator of S^T is already the B operand of the P.V product (no shuffle).
// V^T operands come straight from row-major LDS through the gfx950 transpose
// read (ds_read_b64_tr_b16), which also gathers arbitrary key rows.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/na3d.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsPad = 16;  // bytes of padding per staged K/V row

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int B, T, H, W, NH;
  int KT, KH, KW;
  int tiles_h, tiles_w;
  int lds_rows;  // capacity of each of the K and V staging buffers, in rows
};

// clamp(i - K/2, 0, L - K)
__device__ __forceinline__ int win_start(int i, int K, int L) {
  int s = i - (K >> 1);
  s = s < 0 ? 0 : s;
  return s > L - K ? L - K : s;
}

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

// Spread consecutive logical tiles over one XCD: hardware hands workgroup i
// to XCD i % 8, so XCD x receives logical tiles [x*n/8, (x+1)*n/8) in order
// and neighbouring tiles (which share K/V halo rows) meet in the same L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n >> 3;
  const int rem = n & 7;
  if (i >= n - rem) return i;  // the ragged tail keeps its position
  return (i & 7) * per + (i >> 3);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <int HD, int QH, int QW, int WH, int WW>
__global__ void __launch_bounds__(kWave * WH * WW)
na3d_fwd_plane_kernel(const Args a) {
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
  const int t = wg % a.T;
  wg /= a.T;
  const int tw = wg % a.tiles_w;
  wg /= a.tiles_w;
  const int th = wg % a.tiles_h;
  wg /= a.tiles_h;
  const int n = wg % a.NH;
  const int b = wg / a.NH;

  const int H = a.H, W = a.W, KH = a.KH, KW = a.KW;
  const int h0 = th * BH, w0 = tw * BW;
  const int h1 = min(h0 + BH, H) - 1, w1 = min(w0 + BW, W) - 1;
  // halo of the whole tile (global coordinates), [hh0, hh0+hhn) x [hw0, hw0+hwd)
  const int hh0 = win_start(h0, KH, H);
  const int hhn = win_start(h1, KH, H) + KH - hh0;
  const int hw0 = win_start(w0, KW, W);
  const int hwd = win_start(w1, KW, W) + KW - hw0;
  const int halo_rows = hhn * hwd;
  const int st = win_start(t, a.KT, a.T);

  // ---- this wave's 16-query block
  const int bh0 = h0 + (wave / WW) * QH;
  const int bw0 = w0 + (wave % WW) * QW;
  const bool wave_active = bh0 < H && bw0 < W;
  const int bh1 = min(bh0 + QH, H) - 1;
  const int bw1 = min(bw0 + QW, W) - 1;
  const int qh = bh0 + q16 / QW;
  const int qw = bw0 + q16 % QW;
  const bool qvalid = wave_active && qh < H && qw < W;
  const int qhc = min(qh, H - 1), qwc = min(qw, W - 1);
  const int ash = win_start(qhc, KH, H);  // query window start (global)
  const int asw = win_start(qwc, KW, W);
  // union of the block's windows, in global coordinates
  const int uh0 = wave_active ? win_start(bh0, KH, H) : hh0;
  const int uhn = wave_active ? win_start(bh1, KH, H) + KH - uh0 : 0;
  const int uw0 = wave_active ? win_start(bw0, KW, W) : hw0;
  const int uw = wave_active ? win_start(bw1, KW, W) + KW - uw0 : 1;
  const int oh = uh0 - hh0, ow = uw0 - hw0;  // union origin inside the halo

  const int64_t tok_stride = (int64_t)a.NH * HD;
  const int64_t plane_stride = (int64_t)H * W * tok_stride;
  const int64_t batch_base = (int64_t)b * a.T * plane_stride + (int64_t)n * HD;

  // ---- Q^T operand (B of S^T = K.Q^T): lane (q16, g) holds hd [32ks+8g, +8)
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = a.q + batch_base + (int64_t)t * plane_stride +
                         ((int64_t)qhc * W + qwc) * tok_stride;
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
    const uint16_t* kplane = a.k + batch_base + (int64_t)tp * plane_stride;
    const uint16_t* vplane = a.v + batch_base + (int64_t)tp * plane_stride;
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
        const int64_t off = ((int64_t)hp * W + wp) * tok_stride + part * 8;
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
    uint16_t* op = a.o + batch_base + (int64_t)t * plane_stride +
                   ((int64_t)qh * W + qw) * tok_stride;
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

// ------------------------------------------------------------------ host side
constexpr int kQH = 4, kQW = 4, kWH = 2, kWW = 2;  // 8 x 8 query tile, 4 waves
constexpr int kMaxLdsBytes = 80 * 1024;            // two workgroups per CU

int head_dim_ok(int hd) { return hd == 16 || hd == 32 || hd == 64 || hd == 128 || hd == 256; }

bool overlaps(const void* a, const void* b, size_t bytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bytes && y < x + bytes;
}

struct Plan {
  int family, bt, bh, bw;
  int64_t wgs;
  int threads, lds_bytes, planes;
  int tiles_h, tiles_w, lds_rows;
};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

int make_plan(int B, int T, int H, int W, int NH, int HD, int KT, int KH, int KW, Plan* p) {
  const int BH = kWH * kQH, BW = kWW * kQW;
  p->family = 1;
  p->bt = 1;
  p->bh = BH;
  p->bw = BW;
  p->tiles_h = ceil_div(H, BH);
  p->tiles_w = ceil_div(W, BW);
  p->wgs = (int64_t)B * NH * T * p->tiles_h * p->tiles_w;
  p->threads = kWave * kWH * kWW;
  const int row = HD * 2 + kLdsPad;
  const int max_halo = (std::min(BH + KH - 1, H)) * (std::min(BW + KW - 1, W));
  const int cap = kMaxLdsBytes / (2 * row);
  p->lds_rows = std::min(max_halo, cap);
  p->lds_bytes = 2 * p->lds_rows * row;
  p->planes = KT;
  if (p->wgs > 0x7fffffff) return NA3D_ERR_SHAPE;
  return NA3D_OK;
}

int check_sizes(int B, int T, int H, int W, int NH, int HD, int KT, int KH, int KW) {
  if (B < 1 || T < 1 || H < 1 || W < 1 || NH < 1 || HD < 1) return NA3D_ERR_SHAPE;
  if (!head_dim_ok(HD)) return NA3D_ERR_HEAD_DIM;
  // element offsets of one batch entry are formed in 64-bit; grid extents
  // themselves must keep per-axis products in 32-bit range
  if ((int64_t)T * H * W > (int64_t)1 << 30) return NA3D_ERR_SHAPE;
  if ((int64_t)B * T * H * W * NH * HD > ((int64_t)1 << 62) / 2) return NA3D_ERR_SHAPE;
  if (H > (1 << 20) || W > (1 << 20)) return NA3D_ERR_SHAPE;
  if (KT < 1 || KH < 1 || KW < 1 || KT > T || KH > H || KW > W) return NA3D_ERR_WINDOW;
  return NA3D_OK;
}

template <int HD>
int launch(const Args& a, const Plan& p, hipStream_t stream) {
  auto kern = na3d_fwd_plane_kernel<HD, kQH, kQW, kWH, kWW>;
  static std::atomic<int> attr_done{0};
  if (!attr_done.load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            kMaxLdsBytes) != hipSuccess)
      return NA3D_ERR_LAUNCH;
    attr_done.store(1, std::memory_order_release);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)p.wgs), dim3(p.threads), p.lds_bytes, stream, a);
  return hipGetLastError() == hipSuccess ? NA3D_OK : NA3D_ERR_LAUNCH;
}

// gfx950 check, cached per device (0 unknown, 1 yes, -1 no)
std::atomic<int> g_arch_ok[64];

int device_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NA3D_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return NA3D_ERR_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NA3D_ERR_DEVICE;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? NA3D_OK : NA3D_ERR_DEVICE;
}

}  // namespace

extern "C" {

int na3d_abi_version(void) { return 1; }

const char* na3d_status_string(int status) {
  switch (status) {
    case NA3D_OK: return "ok";
    case NA3D_ERR_NULL: return "a tensor pointer is NULL";
    case NA3D_ERR_SHAPE: return "a dimension is < 1 or the tensor is too large";
    case NA3D_ERR_WINDOW: return "a window extent is < 1 or larger than its grid axis";
    case NA3D_ERR_HEAD_DIM: return "head dimension must be 16, 32, 64, 128 or 256";
    case NA3D_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case NA3D_ERR_OVERLAP: return "out overlaps q, k or v";
    case NA3D_ERR_DEVICE: return "the current HIP device is not gfx950";
    case NA3D_ERR_LAUNCH: return "the kernel launch failed";
    default: return "unknown status";
  }
}

int na3d_check_args(const void* q, const void* k, const void* v, const void* out, int B,
                    int T, int H, int W, int NH, int HD, int KT, int KH, int KW) {
  if (!q || !k || !v || !out) return NA3D_ERR_NULL;
  const int rc = check_sizes(B, T, H, W, NH, HD, KT, KH, KW);
  if (rc != NA3D_OK) return rc;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return NA3D_ERR_ALIGN;
  const size_t bytes = (size_t)B * T * H * W * NH * HD * 2;
  if (overlaps(out, q, bytes) || overlaps(out, k, bytes) || overlaps(out, v, bytes))
    return NA3D_ERR_OVERLAP;
  return NA3D_OK;
}

int na3d_plan(int B, int T, int H, int W, int NH, int HD, int KT, int KH, int KW, int* plan) {
  if (!plan) return NA3D_ERR_NULL;
  const int rc = check_sizes(B, T, H, W, NH, HD, KT, KH, KW);
  if (rc != NA3D_OK) return rc;
  Plan p;
  const int rp = make_plan(B, T, H, W, NH, HD, KT, KH, KW, &p);
  if (rp != NA3D_OK) return rp;
  plan[0] = p.family;
  plan[1] = p.bt;
  plan[2] = p.bh;
  plan[3] = p.bw;
  plan[4] = (int)p.wgs;
  plan[5] = p.threads;
  plan[6] = p.lds_bytes;
  plan[7] = p.planes;
  return NA3D_OK;
}

int na3d_fwd(const void* q, const void* k, const void* v, void* out, int B, int T, int H,
             int W, int NH, int HD, int KT, int KH, int KW, void* stream) {
  int rc = na3d_check_args(q, k, v, out, B, T, H, W, NH, HD, KT, KH, KW);
  if (rc != NA3D_OK) return rc;
  Plan p;
  rc = make_plan(B, T, H, W, NH, HD, KT, KH, KW, &p);
  if (rc != NA3D_OK) return rc;
  rc = device_ok();
  if (rc != NA3D_OK) return rc;
  Args a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(out);
  a.B = B; a.T = T; a.H = H; a.W = W; a.NH = NH;
  a.KT = KT; a.KH = KH; a.KW = KW;
  a.tiles_h = p.tiles_h;
  a.tiles_w = p.tiles_w;
  a.lds_rows = p.lds_rows;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (HD) {
    case 16: return launch<16>(a, p, s);
    case 32: return launch<32>(a, p, s);
    case 64: return launch<64>(a, p, s);
    case 128: return launch<128>(a, p, s);
    case 256: return launch<256>(a, p, s);
    default: return NA3D_ERR_HEAD_DIM;
  }
}

}  // extern "C"
