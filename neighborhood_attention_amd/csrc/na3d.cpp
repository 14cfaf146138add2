// na3d.cpp -- C ABI of the NA3D forward library: argument checks, launch
// planning (which kernel family and instantiation runs a given shape) and
// dispatch.  All checks run on the host before any device call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/na3d.h"
#include "common.h"

namespace na3d {

int general_tile_h();
int general_tile_w();
int general_threads();
int general_row_bytes(int hd);

namespace {

constexpr int kMaxLdsBytes = 160 * 1024;     // LDS of one CU
constexpr int kGeneralLdsBytes = 80 * 1024;  // two general workgroups per CU
constexpr int kTargetWorkgroups = 1024;      // 256 CUs x 4

bool head_dim_ok(int hd) { return hd == 16 || hd == 32 || hd == 64 || hd == 128 || hd == 256; }

// Do the byte ranges [a, a + na) and [b, b + nb) intersect?
bool overlaps2(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// *r = a * b + c without signed overflow; false when it would overflow.
bool mul_add(int64_t a, int64_t b, int64_t c, int64_t* r) {
  int64_t p;
  if (__builtin_mul_overflow(a, b, &p)) return false;
  return !__builtin_add_overflow(p, c, r);
}

int check_sizes(int B, int T, int H, int W, int NH, int HD, int KT, int KH, int KW) {
  if (B < 1 || T < 1 || H < 1 || W < 1 || NH < 1 || HD < 1) return NA3D_ERR_SHAPE;
  if (!head_dim_ok(HD)) return NA3D_ERR_HEAD_DIM;
  // per-plane and per-batch element counts stay addressable in 32/64 bit;
  // every product is overflow-checked (the factors are arbitrary ints)
  if ((int64_t)T * H * W > ((int64_t)1 << 30)) return NA3D_ERR_SHAPE;
  int64_t n = (int64_t)T * H * W;
  for (const int f : {B, NH, HD})
    if (!mul_add(n, f, 0, &n) || n > ((int64_t)1 << 61)) return NA3D_ERR_SHAPE;
  if (KT < 1 || KH < 1 || KW < 1 || KT > T || KH > H || KW > W) return NA3D_ERR_WINDOW;
  return NA3D_OK;
}

Strides contiguous(int T, int H, int W, int NH, int HD) {
  Strides s;
  s.n = HD;
  s.w = (int64_t)NH * HD;
  s.h = (int64_t)W * s.w;
  s.t = (int64_t)H * s.h;
  s.b = (int64_t)T * s.t;
  return s;
}

// Element offset of the last element of a tensor, plus one, or -1 when it
// does not fit in 62 bits (strides are >= 0 and sizes >= 1 here).
int64_t extent(const Strides& s, int B, int T, int H, int W, int NH, int HD) {
  int64_t e = HD;
  const int64_t str[5] = {s.b, s.t, s.h, s.w, s.n};
  const int ext[5] = {B, T, H, W, NH};
  for (int i = 0; i < 5; ++i)
    if (!mul_add(str[i], (int64_t)ext[i] - 1, e, &e)) return -1;
  return e < ((int64_t)1 << 62) ? e : -1;
}

// Bytes spanned by the spatial (H, W) part of one plane of one head of a
// tensor: the rolling family addresses K/V staging, Q loads and output
// stores within such a plane with 32-bit byte offsets.
int64_t kv_span_bytes(const Strides& sk, int H, int W, int HD) {
  return 2 * ((int64_t)(H - 1) * sk.h + (int64_t)(W - 1) * sk.w + HD);
}

// Everything a plan depends on: the k/v grid, heads, head dim, window, the
// query box, and the most bytes one head's spatial plane of k, v, q or out
// spans.
struct Geom {
  int B, T, H, W, NH, HD, KT, KH, KW;
  Box box;
  int64_t kv_span;
  int64_t qo_step;  // bytes of one query-plane step of q or out, the larger
};

// The T axis of the query box: local query plane tl is plane off + tl of the
// grid, and its window starts at key plane ws(tl).
struct TAxis {
  int n;  // query planes
  int off, T, KT;
  int ws(int tl) const { return win_start(off + tl, KT, T); }
};

// Query-plane runs along the box's T axis (local indices): an optional first
// run [0, ta) (the planes whose window is [0, KT)), middle runs of tc planes
// over [ta, tz), and an optional last run [tz, n) (the planes whose window is
// [T - KT, T)).
struct Runs {
  int ta, tz, tc;
};

int run_count(const TAxis& ax, const Runs& r) {
  return (r.ta > 0) + (r.tz > r.ta ? ceil_div(r.tz - r.ta, r.tc) : 0) + (r.tz < ax.n);
}

// Calls f(t0, t1) for every run.
template <class F>
void for_runs(const TAxis& ax, const Runs& r, F f) {
  if (r.ta > 0) f(0, r.ta);
  for (int t0 = r.ta; t0 < r.tz; t0 += r.tc) f(t0, std::min(t0 + r.tc, r.tz));
  if (r.tz < ax.n) f(r.tz, ax.n);
}

// Most query blocks one wave holds at a time: in a run [t0, t1) wave r of WT
// owns the blocks of pt consecutive query planes starting at t0 + pt r,
// t0 + pt (r + WT), ...; count, over all key planes of the run, the owned
// blocks with a plane whose window contains that key plane.
int max_active_per_wave(const TAxis& ax, const Runs& runs, int wt, int pt = 1) {
  int best = 0;
  for_runs(ax, runs, [&](int t0, int t1) {
    const int p0 = ax.ws(t0), p1 = ax.ws(t1 - 1) + ax.KT;
    for (int r = 0; r < wt; ++r)
      for (int tp = p0; tp < p1; ++tp) {
        int c = 0;
        for (int t = t0 + pt * r; t < t1; t += pt * wt) {
          const int s = ax.ws(t), e = ax.ws(std::min(t + pt, t1) - 1) + ax.KT;
          c += (s <= tp && tp < e);
        }
        best = std::max(best, c);
      }
  });
  return best;
}

// K/V planes staged per spatial tile over all runs, and the most in one run.
void staged_planes(const TAxis& ax, const Runs& runs, int* total, int* most) {
  *total = 0;
  *most = 0;
  for_runs(ax, runs, [&](int t0, int t1) {
    const int n = ax.ws(t1 - 1) + ax.KT - ax.ws(t0);
    *total += n;
    *most = std::max(*most, n);
  });
}

// Runs for a rolling variant with wt waves along T, ns slots per wave and
// query blocks of pt planes.
// tile_t > 0 fixes the middle run length.  Both layouts are tried: with the
// shared-window planes split off into runs of their own, and without; the
// feasible one that stages fewer planes wins.
bool choose_runs(const TAxis& ax, int wt, int ns, int tile_t, Runs* out, int pt = 1) {
  int ta = 0;
  while (ta < ax.n && ax.ws(ta) == 0) ++ta;
  int tz = ax.n;
  while (tz > 0 && ax.ws(tz - 1) == ax.T - ax.KT) --tz;
  bool found = false;
  int best_cost = 0;
  for (int split = 1; split >= 0; --split) {
    Runs r;
    r.ta = split ? ta : 0;
    r.tz = split ? std::max(tz, ta) : ax.n;
    if (split && (ta >= ax.n || r.tz <= 0)) continue;  // one shared window: nothing to split
    const int span = std::max(r.tz - r.ta, 1);
    int tc = tile_t > 0 ? std::min(tile_t, span) : span;
    r.tc = tc;
    if (tile_t <= 0)
      while (tc > 1 && max_active_per_wave(ax, r, wt, pt) > ns) r.tc = --tc;
    if (max_active_per_wave(ax, r, wt, pt) > ns) continue;
    int total, most;
    staged_planes(ax, r, &total, &most);
    if (!found || total < best_cost) {
      found = true;
      best_cost = total;
      *out = r;
    }
  }
  return found;
}

bool plan_general(const Geom& g, Launch* l) {
  const int BH = general_tile_h(), BW = general_tile_w();
  l->family = 1;
  l->variant = 0;
  l->tile_t = 1;
  l->tile_h = BH;
  l->tile_w = BW;
  l->tiles_t = g.box.Tq;
  l->ta = 0;
  l->tz = g.box.Tq;
  l->nruns = g.box.Tq;
  l->rpw = 1;
  l->tiles_h = ceil_div(g.box.Hq, BH);
  l->tiles_w = ceil_div(g.box.Wq, BW);
  l->wgs = (int64_t)g.B * g.NH * g.box.Tq * l->tiles_h * l->tiles_w;
  l->threads = general_threads();
  const int row = general_row_bytes(g.HD);
  const int max_halo = std::min(BH + g.KH - 1, g.H) * std::min(BW + g.KW - 1, g.W);
  l->lds_rows = std::min(max_halo, kGeneralLdsBytes / (2 * row));
  l->lds_bytes = 2 * l->lds_rows * row;
  l->planes = g.KT;
  l->band_h = 1;
  return l->wgs <= 0x7fffffff;
}

// Can rolling variant v run these sizes?  tile_t = 0 picks the run length;
// `target` is the number of workgroups the launch should reach (runs are
// shortened, and fewer runs given to one workgroup, until it does).
bool plan_roll(int v, const Geom& g, int tile_t, Launch* l, int target = kTargetWorkgroups) {
  if (v < 0 || v >= kNumRollVariants) return false;
  const RollVariant& rv = kRollVariants[v];
  const int HD = g.HD, KH = g.KH, KW = g.KW, H = g.H, W = g.W;
  if (rv.hd != HD) return false;
  // staging, Q and output offsets are 32-bit byte offsets within one head's
  // spatial plane
  if (g.kv_span >= ((int64_t)1 << 32)) return false;
  // blocks of pt query planes (8-query spatial blocks span two planes): a
  // lane's q and out offsets add one plane step
  const int pt = 16 / (rv.qh * rv.qw);
  if (pt > 1 && g.kv_span + g.qo_step >= ((int64_t)1 << 32)) return false;
  const int BH = rv.wh * rv.qh;
  const int hwd_max = std::min(rv.qw + KW - 1, W);
  const int un_max = std::min(rv.qh + KH - 1, H) * hwd_max;
  const int gk = 16 * rv.nk;
  if (un_max > rv.ng * gk) return false;
  const int halo_max = std::min(BH + KH - 1, H) * hwd_max;
  // every wave's read window of ng * gk rows fits in a buffer
  const int rows = std::max(halo_max, rv.ng * gk);
  // K and V rows of HD*2 bytes, in one or two plane buffers
  const int64_t lds = 2LL * rv.nbuf * rows * (HD * 2);
  if (lds > kMaxLdsBytes) return false;
  // the kernel's staging walk keeps one bit per full DMA round of a plane
  // (at most 32; the LDS limit above already bounds them by 27)
  // (a round is one 16-byte chunk per staging lane: the compute waves', or
  // the staging waves' where the variant has them)
  const int stagers = kWave * (rv.pw > 0 ? rv.pw : rv.wh * rv.wt);
  if ((int64_t)halo_max * (HD / 8) / stagers > 32) return false;
  const int tiles_h = ceil_div(g.box.Hq, BH), tiles_w = ceil_div(g.box.Wq, rv.qw);
  const int64_t spatial = (int64_t)g.B * g.NH * tiles_h * tiles_w;
  const TAxis ax{g.box.Tq, g.box.t0, g.T, g.KT};
  Runs r;
  if (!choose_runs(ax, rv.wt, rv.ns, tile_t, &r, pt)) return false;
  if (tile_t <= 0) {
    // shorter middle runs while the grid is too small to fill the chip
    while (r.tc > rv.wt * pt && spatial * run_count(ax, r) < target) {
      Runs s = r;
      s.tc = ceil_div(r.tc, 2);
      if (max_active_per_wave(ax, s, rv.wt, pt) > rv.ns) break;
      r = s;
    }
  }
  int total, most;
  staged_planes(ax, r, &total, &most);
  // a workgroup streams several consecutive runs (one set-up, and the next
  // run's first plane is fetched during the last plane of the previous one)
  // as long as the grid keeps enough workgroups
  const int nruns = run_count(ax, r);
  const int groups = (int)std::min<int64_t>(nruns, std::max<int64_t>(1, (target + spatial - 1) / spatial));
  const int rpw = ceil_div(nruns, groups);
  l->family = 2;
  l->variant = v;
  l->tile_t = r.tc;
  l->tile_h = BH;
  l->tile_w = rv.qw;
  l->tiles_t = ceil_div(nruns, rpw);
  l->nruns = nruns;
  l->rpw = rpw;
  l->tiles_h = tiles_h;
  l->tiles_w = tiles_w;
  l->ta = r.ta;
  l->tz = r.tz;
  l->wgs = spatial * l->tiles_t;
  l->threads = kWave * (rv.wh * rv.wt + rv.pw);
  l->lds_rows = rows;
  l->lds_bytes = (int)lds;
  l->planes = std::min(rpw, nruns) == 1 ? most : total;  // upper bound for run groups
  // Visiting order of the spatial tiles: bands of band_h tile rows, so that
  // the tiles in flight on one XCD (32 CUs, as many workgroups per CU as LDS
  // allows, consecutive workgroup indices) form a block about as tall as it
  // is wide in query space and share their halo rows in that XCD's L2.
  {
    const int per_cu = std::max(1, kMaxLdsBytes / std::max(1, l->lds_bytes));
    const double tiles_in_flight = 32.0 * per_cu / l->tiles_t;
    const double bh = std::sqrt(tiles_in_flight * rv.qw / BH);
    l->band_h = std::max(1, std::min(tiles_h, (int)std::lround(bh)));
  }
  return l->wgs <= 0x7fffffff;
}

// Preferred rolling instantiations, best first (from measured sweeps), by
// head dimension and by the union of one 2x8 query block's windows; the first
// whose static limits fit the sizes wins.
int pick_roll(const Geom& g, Launch* l) {
  // head dim 16: the same shapes as head dim 32 (16x64x96 (3,7,7) at 8 heads
  // 105 against 186 us; 11x11x11 233 us on 4x4 blocks and 224 us on
  // two-plane ones against 335 us; (3,5,27) at 32 heads 37 against 50 us;
  // (19,19,19) 307 against 1347 us on the general family)
  static const int p16_mid[] = {73, 11};
  static const int p16_large[] = {70, 71, 11, 72};
  // head dim 32: the head-dim-64 shapes (decoder-class 8-wave two-buffer
  // 7-tile groups; 13-tile 4x4 and 2x8 one-group; four 8-tile groups), then
  // the 2x8 two-group catch-all (16x64x96 (3,7,7) at 8 heads 105 against
  // 267 us for the catch-all; 16x48x64 (11,11,11) 253 against 434 us, and
  // 225 us on two-plane blocks (69, by the rule below); (3,5,27) on 4x8x128 at
  // 32 heads 40 against 68 us; 24x32x32 (19,19,19) 300 against 1446 us on
  // the general family)
  static const int p32_mid[] = {68, 12};
  static const int p32_large[] = {65, 66, 12, 67};
  // union <= 64 keys: first the 8-wave two-buffer 4-tile variant (two 2x8
  // blocks along H, four phases: 15-22% faster than the 3-wave variant 8 on
  // the narrow edge tiles, 16x64x96 (3,3,3) and (3,5,3), 8x32x48 (3,3,5))
  static const int p64_small[] = {17, 8, 34, 21, 26, 20, 9};
  static const int p64_mid[] = {42, 43, 40, 38, 35, 26, 34, 21, 20, 1, 9, 10};  // <= 112 keys
  // larger windows: 4x4 blocks for near-cubic ones; 2x8 blocks for windows
  // much wider along W (their union is smaller in 2x8 blocks), with one
  // 13-tile group up to a 208-key union and two to four groups beyond (the
  // windows wider than 33 that the pages' kernel refused: measured 1.9-2.8x
  // faster than the 4x4 two-group variant 10 and 3.5x faster than the
  // general family on (3,5,35) to (3,5,63))
  // and, last, four 8-tile groups (512 keys) on 4x4 blocks for unions no
  // smaller instantiation holds, one 8-wave workgroup per CU (19x19x19 on
  // 24x32x32, 4 heads: 384 us against 1687 us for the general family;
  // (5,19,19) on 8x32x64: 88 against 317 us)
  static const int p64_large[] = {5, 46, 51, 50, 49, 58, 55, 56, 10, 22, 6, 7, 9, 62};
  // head dim 128: past the 2x8 7-tile variants, two-plane blocks of 2x4
  // queries in 8-wave workgroups of 8x4-query tiles (77: one 126 KB
  // workgroup per CU, two waves per SIMD, where the 4-wave variants of
  // 100-104 KB leave one): 16x64x96, 8 heads, (3,11,11) 501 against 830 us
  // for 4x4 blocks (16), (5,9,9) 690 against 1120, (7,9,9) 842 against 1330;
  // 11x11x11 on 16x48x64 636 against 912 us for the 4-wave two-plane
  // variant (60) and 982 for 16, on 16x80x32 at 32 heads 2043 against 2984;
  // then 4x4 blocks (one 13-tile group) before the 2x8 two-group variants
  // for near-cubic windows (11x11x11 on 16x48x64, 8 heads: 1018 us against
  // 1299 us for variant 57 and 1632 us for variant 15); the 9-tile two-group
  // 2x8 variant for wide windows (3x7x19: 1004 us against 1080 us), with 8
  // phases along T in 8 waves (78: the same 147 KB of LDS, two waves per
  // SIMD instead of one, bitwise the same outputs) before its 4-wave form
  // (57): (13,13,13) on 16x32x32 at 8 heads 342 against 485 us, (3,5,27)
  // and (3,5,35) on 16x64x128 1283 and 1335 against 1327 and 1393 us,
  // (3,5,27) on 4x8x128 at 32 heads 168 against 174 us
  static const int p128[] = {47, 25, 77, 16, 78, 57, 15, 14, 13, 29};
  // head dim 256: one-buffer variants (a two-buffer plane of 512-byte rows
  // does not fit LDS; measured 548 us against 862 us for the general family
  // on 16x64x96, 4 heads, (3,7,7))
  static const int p256[] = {53, 52};
  const int un28 = std::min(2 + g.KH - 1, g.H) * std::min(8 + g.KW - 1, g.W);
  const int un44 = std::min(4 + g.KH - 1, g.H) * std::min(4 + g.KW - 1, g.W);
  // head dim 64, windows whose 4x4-block union fits 4 tiles but whose 2x8
  // union does not (e.g. (3,5,5): 64 against 72 keys): 4x4 blocks in 8-wave
  // two-buffer workgroups with 4-tile groups, where the 2x8 choice would read
  // 7 tiles (36x64x96 at 8 heads 272 against 293 us, at 32 heads 914
  // against 1106 us; 16x64x96 at 8 heads 122 against 135 us)
  if (g.HD == 64 && un28 > 64 && un44 <= 64 && plan_roll(63, g, 0, l)) return 1;
  // head dim 64, 2x8-block unions of at most 2 tiles (the W = 5 edge tile
  // with (3,5,5): 6x5 = 30 keys): the same 8-wave shape with 2-tile groups
  // (14.0 against 15.9 us for the 4-tile one)
  if (g.HD == 64 && un28 <= 32 && plan_roll(64, g, 0, l)) return 1;
  const int* pref;
  int np;
  switch (g.HD) {
    case 16:
      if (un28 <= 112) {
        pref = p16_mid; np = (int)(sizeof(p16_mid) / sizeof(int));
      } else {
        pref = p16_large; np = (int)(sizeof(p16_large) / sizeof(int));
      }
      break;
    case 32:
      if (un28 <= 112) {
        pref = p32_mid; np = (int)(sizeof(p32_mid) / sizeof(int));
      } else {
        pref = p32_large; np = (int)(sizeof(p32_large) / sizeof(int));
      }
      break;
    case 64:
      if (un28 <= 64) {
        pref = p64_small; np = (int)(sizeof(p64_small) / sizeof(int));
      } else if (un28 <= 112) {
        pref = p64_mid; np = (int)(sizeof(p64_mid) / sizeof(int));
      } else {
        pref = p64_large; np = (int)(sizeof(p64_large) / sizeof(int));
      }
      break;
    case 128: pref = p128; np = (int)(sizeof(p128) / sizeof(int)); break;
    default: pref = p256; np = (int)(sizeof(p256) / sizeof(int)); break;
  }
  // head dim 128, three-plane windows: blocks of 2x4 queries on two planes,
  // 8 waves as 4 block rows by 2 plane-pair phases (a wave's consecutive
  // pairs are four planes apart, so their windows never overlap and every
  // wave works on every key plane, where 2x8 blocks on single planes leave
  // one phase in four idle): 4653 against 4952 us on the 32x128x192,
  // 16-head grid
  // The same blocks with four staging waves added to the workgroup (75): the
  // compute waves no longer issue the plane's loads (4179 against 4591 us on
  // the same grid)
  if (g.HD == 128 && g.KT == 3 && (plan_roll(75, g, 0, l) || plan_roll(61, g, 0, l))) return 1;
  for (int i = 0; i < np; ++i) {
    if (!plan_roll(pref[i], g, 0, l)) continue;
    // windows much wider than tall, on a grid large enough that the 8-wave
    // two-buffer variant has four or more workgroups per CU: the 4-wave
    // one-buffer variant of the same blocks is faster (measured on the
    // (3,5,27) benchmark grid: 51 us against 60 us at 32 heads; equal at 16,
    // slower at 8)
    if (pref[i] == 51 && l->wgs >= 1024) {
      Launch alt;
      if (plan_roll(49, g, 0, &alt)) *l = alt;
    }
    // mid-size windows on a grid with fewer than 1024 spatial tiles of the
    // 8-wave variant: 4-wave workgroups fill the chip better (measured on
    // the 18x32x48 (3,7,7) benchmark grid: 36-51 us against 38-57 us at 4
    // and 8 heads; at 32 heads and on the decoder tile the 8-wave one wins)
    if (pref[i] == 42 && l->wgs / std::max(l->tiles_t, 1) < 1024) {
      Launch alt;
      if (plan_roll(34, g, 0, &alt)) *l = alt;
    }
    // three-plane windows on grids of 32 or more query planes with enough
    // 8x8-query tiles to fill the chip without cutting the runs along T:
    // 12-wave workgroups of those tiles (18: 4 block rows by 3 phases, one
    // workgroup per CU), whose halo is re-read by fewer workgroups.  On
    // 96x128 at 8 heads (3,7,7) 552 against 568 us at T = 32, 805 against
    // 851 at 48, 1055 against 1138 at 64; 79x192x192 4205 against 4392 us;
    // 64x96 at 32 heads equal.  Where the runs would be cut (64x96 at 8
    // heads: 768 tiles) it is far slower (T = 64: 945 against 578 us), as
    // on 16-plane grids
    if (l->variant == 42 && g.KT == 3 && g.box.Tq >= 32) {
      Launch alt;
      if (plan_roll(18, g, 0, &alt) && alt.tiles_t == 1 &&
          alt.wgs >= kTargetWorkgroups)
        *l = alt;
    }
    // query blocks over two planes (2x4 queries on each), for windows long
    // along T: where their smaller window union saves more tiles than the
    // extra key plane per block costs, i.e. (KT + 1) x 11 tiles per 16
    // queries against KT x the chosen variant's, by at least 5% (11x11x11:
    // 3% faster at head dim 64 on 16x48x64, 6% on 16x80x32 at 32 heads, 7%
    // at head dim 128)
    const int pp = g.HD == 64 ? 59 : g.HD == 128 ? 60 : g.HD == 32 ? 69 : g.HD == 16 ? 74 : -1;
    if (pp >= 0 && g.KT >= 6) {
      const RollVariant& a = kRollVariants[l->variant];
      const RollVariant& c = kRollVariants[pp];
      const int64_t ca = (int64_t)(g.KT + 16 / (a.qh * a.qw) - 1) * a.ng * a.nk;
      const int64_t cc = (int64_t)(g.KT + 16 / (c.qh * c.qw) - 1) * c.ng * c.nk;
      Launch alt;
      if (cc * 20 < ca * 19 && plan_roll(pp, g, 0, &alt)) {
        *l = alt;
        // head dim 64 on grids of 32 or more query planes: the same blocks
        // in 12-wave workgroups of 12x4-query tiles (one per CU, two plane
        // buffers), whose halo is re-read by 6.4 rather than 12.3 workgroups
        // per query (11x11x11: 79x192x192 at 32 heads 80.7 against 107.0 ms,
        // at 4 heads 10.25 against 10.72 ms; 40x96x96 at 32 heads 9.93
        // against 10.53 ms; even on 32x96x96; slower on 16- and 24-plane
        // grids, e.g. 16x48x64 at 8 heads 320 against 303 us)
        if (pp == 59 && g.box.Tq >= 32 && plan_roll(76, g, 0, &alt)) *l = alt;
      }
    }
    return 1;
  }
  return 0;
}

int make_plan(const Geom& g, Launch* l) {
  if (pick_roll(g, l)) return NA3D_OK;
  if (plan_general(g, l)) return NA3D_OK;
  return NA3D_ERR_SHAPE;
}

int make_plan_config(const Geom& g, int family, int variant, int tile_t, Launch* l) {
  if (family == 0) return make_plan(g, l);
  if (family == 1) return plan_general(g, l) ? NA3D_OK : NA3D_ERR_SHAPE;
  if (family == 2) return plan_roll(variant, g, tile_t, l) ? NA3D_OK : NA3D_ERR_CONFIG;
  return NA3D_ERR_CONFIG;
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

// Stride contract of the strided entry points; st = {q, k, v, out}.  q and
// out have the query box's extents, k and v the grid's.
int check_strides(const void* q, const void* k, const void* v, const void* out, const Geom& g,
                  const Strides* st) {
  const int64_t lim = (int64_t)1 << 56;
  for (int i = 0; i < 4; ++i) {
    const int64_t x[5] = {st[i].b, st[i].t, st[i].h, st[i].w, st[i].n};
    for (int j = 0; j < 5; ++j)
      if (x[j] < 0 || x[j] % 8 != 0 || x[j] > lim) return NA3D_ERR_STRIDE;
  }
  if (st[1].h != st[2].h || st[1].w != st[2].w || st[1].n != st[2].n) return NA3D_ERR_STRIDE;
  const Box& bx = g.box;
  // no two elements of out at one address: ordered by stride, every axis of
  // extent > 1 steps over the whole span of the smaller ones (HD first)
  {
    int64_t ext[5] = {g.B, bx.Tq, bx.Hq, bx.Wq, g.NH};
    int64_t str[5] = {st[3].b, st[3].t, st[3].h, st[3].w, st[3].n};
    int idx[5] = {0, 1, 2, 3, 4};
    std::sort(idx, idx + 5, [&](int a, int b) { return str[a] < str[b]; });
    int64_t span = g.HD;
    for (int j = 0; j < 5; ++j) {
      const int a = idx[j];
      if (ext[a] == 1) continue;
      if (str[a] < span) return NA3D_ERR_STRIDE;
      if (!mul_add(str[a], ext[a] - 1, span, &span)) return NA3D_ERR_STRIDE;
    }
  }
  // element extents (-1: beyond what any buffer can span)
  const int64_t eq = extent(st[0], g.B, bx.Tq, bx.Hq, bx.Wq, g.NH, g.HD);
  const int64_t ek = extent(st[1], g.B, g.T, g.H, g.W, g.NH, g.HD);
  const int64_t ev = extent(st[2], g.B, g.T, g.H, g.W, g.NH, g.HD);
  const int64_t eo = extent(st[3], g.B, bx.Tq, bx.Hq, bx.Wq, g.NH, g.HD);
  if (eq < 0 || ek < 0 || ev < 0 || eo < 0) return NA3D_ERR_STRIDE;
  const size_t bo = 2 * (size_t)eo;
  if (overlaps2(out, bo, q, 2 * (size_t)eq) || overlaps2(out, bo, k, 2 * (size_t)ek) ||
      overlaps2(out, bo, v, 2 * (size_t)ev))
    return NA3D_ERR_OVERLAP;
  return NA3D_OK;
}

Geom make_geom(int B, int T, int H, int W, int NH, int HD, int KT, int KH, int KW, const Box& box) {
  Geom g;
  g.B = B; g.T = T; g.H = H; g.W = W; g.NH = NH; g.HD = HD;
  g.KT = KT; g.KH = KH; g.KW = KW;
  g.box = box;
  g.kv_span = 0;
  g.qo_step = 0;
  return g;
}

Box full_box(int T, int H, int W) { return Box{0, 0, 0, T, H, W}; }

// All host checks of a call, in the order the status codes document.
int check_all(const void* q, const void* k, const void* v, const void* out, const Geom& g,
              const Strides* st) {
  if (!q || !k || !v || !out) return NA3D_ERR_NULL;
  const int rc = check_sizes(g.B, g.T, g.H, g.W, g.NH, g.HD, g.KT, g.KH, g.KW);
  if (rc != NA3D_OK) return rc;
  const Box& b = g.box;
  if (b.Tq < 1 || b.Hq < 1 || b.Wq < 1 || b.t0 < 0 || b.h0 < 0 || b.w0 < 0 ||
      b.t0 > g.T - b.Tq || b.h0 > g.H - b.Hq || b.w0 > g.W - b.Wq)
    return NA3D_ERR_BOX;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return NA3D_ERR_ALIGN;
  return check_strides(q, k, v, out, g, st);
}

int run(const void* q, const void* k, const void* v, void* out, const Geom& g, const Strides* st,
        const Launch& l, void* stream) {
  int rc = device_ok();
  if (rc != NA3D_OK) return rc;
  Problem p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(out);
  p.B = g.B; p.T = g.T; p.H = g.H; p.W = g.W; p.NH = g.NH;
  p.KT = g.KT; p.KH = g.KH; p.KW = g.KW;
  p.box = g.box;
  p.sq = st[0]; p.sk = st[1]; p.sv = st[2]; p.so = st[3];
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = l.family == 2 ? launch_roll(p, l, g.HD, s) : launch_general(p, l, g.HD, s);
  return rc == 0 ? NA3D_OK : NA3D_ERR_LAUNCH;
}

// Plans by geometry and requested configuration: the planner's run search
// costs a few microseconds per call, comparable to a small grid's kernel, so
// repeated calls with the same sizes reuse the first plan.
struct PlanKey {
  int v[19];
  int64_t span, step;
  bool operator==(const PlanKey& o) const {
    return span == o.span && step == o.step && std::memcmp(v, o.v, sizeof(v)) == 0;
  }
};
struct PlanKeyHash {
  size_t operator()(const PlanKey& k) const {
    uint64_t h = (1469598103934665603ull ^ (uint64_t)k.span) * 1099511628211ull ^ (uint64_t)k.step;
    for (int x : k.v) h = (h ^ (uint32_t)x) * 1099511628211ull;
    return (size_t)h;
  }
};
std::mutex g_plan_mu;
std::unordered_map<PlanKey, std::pair<int, Launch>, PlanKeyHash> g_plans;

int cached_plan(const Geom& g, int family, int variant, int tile_t, Launch* l) {
  const PlanKey key{{g.B, g.T, g.H, g.W, g.NH, g.HD, g.KT, g.KH, g.KW, g.box.t0, g.box.h0,
                     g.box.w0, g.box.Tq, g.box.Hq, g.box.Wq, family, variant, tile_t, 0},
                    g.kv_span, g.qo_step};
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    const auto it = g_plans.find(key);
    if (it != g_plans.end()) {
      *l = it->second.second;
      return it->second.first;
    }
  }
  const int rc = make_plan_config(g, family, variant, tile_t, l);
  std::lock_guard<std::mutex> lk(g_plan_mu);
  if (g_plans.size() >= 4096) g_plans.clear();
  g_plans.emplace(key, std::make_pair(rc, *l));
  return rc;
}

// Checks, plans and launches one call.
int fwd_impl(const void* q, const void* k, const void* v, void* out, Geom g, const Strides* st,
             int family, int variant, int tile_t, void* stream) {
  int rc = check_all(q, k, v, out, g, st);
  if (rc != NA3D_OK) return rc;
  g.kv_span = std::max({kv_span_bytes(st[1], g.H, g.W, g.HD), kv_span_bytes(st[2], g.H, g.W, g.HD),
                        kv_span_bytes(st[0], g.box.Hq, g.box.Wq, g.HD),
                        kv_span_bytes(st[3], g.box.Hq, g.box.Wq, g.HD)});
  g.qo_step = 2 * std::max(std::llabs(st[0].t), std::llabs(st[3].t));
  Launch l;
  rc = cached_plan(g, family, variant, tile_t, &l);
  if (rc != NA3D_OK) return rc;
  return run(q, k, v, out, g, st, l, stream);
}

void read_strides(const long long* strides, Strides* st) {
  for (int i = 0; i < 4; ++i)
    st[i] = Strides{strides[5 * i], strides[5 * i + 1], strides[5 * i + 2], strides[5 * i + 3],
                    strides[5 * i + 4]};
}

// Contiguous strides of q and out (box extents) and of k and v (grid extents).
void contiguous_all(const Geom& g, Strides* st) {
  st[0] = st[3] = contiguous(g.box.Tq, g.box.Hq, g.box.Wq, g.NH, g.HD);
  st[1] = st[2] = contiguous(g.T, g.H, g.W, g.NH, g.HD);
}

void fill_plan(const Launch& l, int* plan) {
  plan[0] = l.family;
  plan[1] = l.tile_t;
  plan[2] = l.tile_h;
  plan[3] = l.tile_w;
  plan[4] = (int)l.wgs;
  plan[5] = l.threads;
  plan[6] = l.lds_bytes;
  plan[7] = l.planes;
  plan[8] = l.variant;
  plan[9] = l.tiles_t;
}

// Argument contract of the RMSNorm entry points.
int rms_check(const void* x, const void* w, const void* y, int rows, int dim, float eps) {
  if (rows < 0 || dim < 8 || dim % 8 != 0 || dim > kRmsMaxDim) return NA3D_ERR_SHAPE;
  // bit test behind an opaque barrier: the library is built without NaN
  // semantics, so a float test (or a bit test the compiler can see through)
  // could be folded into an infinity-only check
  uint32_t eb;
  std::memcpy(&eb, &eps, 4);
  asm volatile("" : "+r"(eb));
  if ((eb & 0x7f800000u) == 0x7f800000u || eps < 0.f) return NA3D_ERR_VALUE;
  if (rows == 0) return NA3D_OK;  // nothing is read or written
  if (!x || !y) return NA3D_ERR_NULL;
  if (((uintptr_t)x | (uintptr_t)y | (uintptr_t)w) & 15) return NA3D_ERR_ALIGN;
  const size_t n = (size_t)rows * dim * 2;
  if (x != y && overlaps2(y, n, x, n)) return NA3D_ERR_OVERLAP;
  if (w && overlaps2(y, n, w, (size_t)dim * 2)) return NA3D_ERR_OVERLAP;
  return NA3D_OK;
}

// ---- batches of tiles (one launch for many grids)

int64_t tile_bytes(const na3d_tile& t, int NH, int HD) {
  return 2 * (int64_t)t.B * t.T * t.H * t.W * NH * HD;
}

Geom tile_geom(const na3d_tile& t, int NH, int HD, int KT, int KH, int KW) {
  Geom g = make_geom(t.B, t.T, t.H, t.W, NH, HD, KT, KH, KW, full_box(t.T, t.H, t.W));
  return g;
}

int check_batch(const na3d_tile* tiles, int n, int NH, int HD, int KT, int KH, int KW) {
  if (n < 0) return NA3D_ERR_SHAPE;
  if (n == 0) return NA3D_OK;
  if (!tiles) return NA3D_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    const na3d_tile& t = tiles[i];
    const Geom g = tile_geom(t, NH, HD, KT, KH, KW);
    Strides st[4];
    contiguous_all(g, st);
    const int rc = check_all(t.q, t.k, t.v, t.out, g, st);
    if (rc != NA3D_OK) return rc;
  }
  // every output is disjoint from every other tile's tensors
  for (int i = 0; i < n; ++i) {
    const size_t bi = (size_t)tile_bytes(tiles[i], NH, HD);
    for (int j = 0; j < n; ++j) {
      if (j == i) continue;
      const na3d_tile& u = tiles[j];
      const size_t bj = (size_t)tile_bytes(u, NH, HD);
      if (overlaps2(tiles[i].out, bi, u.q, bj) || overlaps2(tiles[i].out, bi, u.k, bj) ||
          overlaps2(tiles[i].out, bi, u.v, bj) || overlaps2(tiles[i].out, bi, u.out, bj))
        return NA3D_ERR_OVERLAP;
    }
  }
  return NA3D_OK;
}

// The launches a batch takes: tiles that the rolling instantiation of the
// largest tile can run share launches of up to kMaxBatch tiles (in the
// given order); the others get a launch of their own with their own plan.
struct BatchPlan {
  int variant = -1;                 // rolling instantiation of the shared launches
  std::vector<Launch> plan;         // per tile
  std::vector<char> shared;         // per tile: in a shared launch?
  std::vector<std::vector<int>> groups;  // tiles of each shared launch
};

int plan_batch(const na3d_tile* tiles, int n, int NH, int HD, int KT, int KH, int KW,
               BatchPlan* bp) {
  bp->plan.assign(n, Launch{});
  bp->shared.assign(n, 0);
  bp->groups.clear();
  bp->variant = -1;
  if (n == 0) return NA3D_OK;
  std::vector<Geom> geo(n);
  int lead = 0;
  for (int i = 0; i < n; ++i) {
    const na3d_tile& t = tiles[i];
    const int rc = check_sizes(t.B, t.T, t.H, t.W, NH, HD, KT, KH, KW);
    if (rc != NA3D_OK) return rc;
    geo[i] = tile_geom(t, NH, HD, KT, KH, KW);
    Strides st[4];
    contiguous_all(geo[i], st);
    geo[i].kv_span = kv_span_bytes(st[1], t.H, t.W, HD);
    geo[i].qo_step = 2 * st[0].t;
    const int64_t wi = (int64_t)t.B * t.T * t.H * t.W, wl = (int64_t)tiles[lead].B *
                                                          tiles[lead].T * tiles[lead].H * tiles[lead].W;
    if (wi > wl) lead = i;
  }
  Launch ll;
  if (make_plan(geo[lead], &ll) != NA3D_OK) return NA3D_ERR_SHAPE;
  if (ll.family == 2) bp->variant = ll.variant;
  // a tile in a shared launch needs only its share of the launch's
  // workgroups: its runs stay as long as the whole batch allows
  double total = 0;
  for (int i = 0; i < n; ++i) total += (double)tiles[i].B * tiles[i].T * tiles[i].H * tiles[i].W;
  std::vector<int> cur;
  int64_t cur_wgs = 0;
  for (int i = 0; i < n; ++i) {
    Launch l;
    const double share = (double)tiles[i].B * tiles[i].T * tiles[i].H * tiles[i].W / total;
    const int target = std::max(1, (int)(kTargetWorkgroups * share));
    if (bp->variant >= 0 && plan_roll(bp->variant, geo[i], 0, &l, target)) {
      bp->plan[i] = l;
      bp->shared[i] = 1;
      if (!cur.empty() && ((int)cur.size() == kMaxBatch || cur_wgs + l.wgs > 0x7fffffff)) {
        bp->groups.push_back(cur);
        cur.clear();
        cur_wgs = 0;
      }
      cur.push_back(i);
      cur_wgs += l.wgs;
    } else {
      if (make_plan(geo[i], &l) != NA3D_OK) return NA3D_ERR_SHAPE;
      bp->plan[i] = l;
    }
  }
  if (!cur.empty()) bp->groups.push_back(cur);
  return NA3D_OK;
}

int batch_impl(const na3d_tile* tiles, int n, int NH, int HD, int KT, int KH, int KW,
               void* stream) {
  int rc = check_batch(tiles, n, NH, HD, KT, KH, KW);
  if (rc != NA3D_OK || n == 0) return rc;
  BatchPlan bp;
  rc = plan_batch(tiles, n, NH, HD, KT, KH, KW, &bp);
  if (rc != NA3D_OK) return rc;
  rc = device_ok();
  if (rc != NA3D_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (const std::vector<int>& grp : bp.groups) {
    RollBatch bt;
    bt.n = (int)grp.size();
    Launch l = bp.plan[grp[0]];
    int64_t off = 0;
    for (int j = 0; j < bt.n; ++j) {
      const na3d_tile& t = tiles[grp[j]];
      const Launch& lt = bp.plan[grp[j]];
      BatchTile& e = bt.t[j];
      e.q = static_cast<const uint16_t*>(t.q);
      e.k = static_cast<const uint16_t*>(t.k);
      e.v = static_cast<const uint16_t*>(t.v);
      e.o = static_cast<uint16_t*>(t.out);
      e.B = t.B; e.T = t.T; e.H = t.H; e.W = t.W;
      e.wg_off = (int)off;
      e.tiles_t = lt.tiles_t; e.tiles_h = lt.tiles_h; e.tiles_w = lt.tiles_w;
      e.tc = lt.tile_t; e.ta = lt.ta; e.tz = lt.tz; e.nruns = lt.nruns; e.rpw = lt.rpw;
      e.lds_rows = lt.lds_rows;
      off += lt.wgs;
      l.lds_rows = std::max(l.lds_rows, lt.lds_rows);
      l.lds_bytes = std::max(l.lds_bytes, lt.lds_bytes);
    }
    l.wgs = off;
    Problem p;
    p.NH = NH; p.KT = KT; p.KH = KH; p.KW = KW;
    if (launch_roll_batch(p, l, bt, HD, s) != 0) return NA3D_ERR_LAUNCH;
  }
  for (int i = 0; i < n; ++i) {
    if (bp.shared[i]) continue;
    const na3d_tile& t = tiles[i];
    const Geom g = tile_geom(t, NH, HD, KT, KH, KW);
    Strides st[4];
    contiguous_all(g, st);
    rc = run(t.q, t.k, t.v, t.out, g, st, bp.plan[i], stream);
    if (rc != NA3D_OK) return rc;
  }
  return NA3D_OK;
}

int rms_impl(const void* x, const void* w, void* y, int rows, int dim, float eps, int wgs,
             void* stream) {
  int rc = rms_check(x, w, y, rows, dim, eps);
  if (rc != NA3D_OK) return rc;
  if (wgs < 0 || wgs > (1 << 24)) return NA3D_ERR_CONFIG;
  if (rows == 0) return NA3D_OK;
  rc = device_ok();
  if (rc != NA3D_OK) return rc;
  rc = launch_rms_norm(x, w, y, rows, dim, eps, wgs, static_cast<hipStream_t>(stream));
  return rc == 0 ? NA3D_OK : NA3D_ERR_LAUNCH;
}



}  // namespace
}  // namespace na3d

using namespace na3d;

extern "C" {

int na3d_abi_version(void) { return 3; }

int na3d_num_variants(void) { return kNumRollVariants; }

int na3d_variant_info(int variant, int* info) {
  if (!info) return NA3D_ERR_NULL;
  if (variant < 0 || variant >= kNumRollVariants) return NA3D_ERR_CONFIG;
  const RollVariant& v = kRollVariants[variant];
  const int vals[10] = {v.hd, v.qh, v.qw, v.wh, v.wt, v.ns, v.nk, v.ng, v.nbuf, v.occ};
  for (int i = 0; i < 10; ++i) info[i] = vals[i];
  return NA3D_OK;
}

const char* na3d_status_string(int status) {
  switch (status) {
    case NA3D_OK: return "ok";
    case NA3D_ERR_NULL: return "a tensor or stride pointer is NULL";
    case NA3D_ERR_SHAPE: return "a dimension is < 1 or the tensor is too large";
    case NA3D_ERR_WINDOW: return "a window extent is < 1 or larger than its grid axis";
    case NA3D_ERR_HEAD_DIM: return "head dimension must be 16, 32, 64, 128 or 256";
    case NA3D_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case NA3D_ERR_OVERLAP: return "an output overlaps an input it must not overlap";
    case NA3D_ERR_DEVICE: return "the current HIP device is not gfx950";
    case NA3D_ERR_LAUNCH: return "the kernel launch failed";
    case NA3D_ERR_CONFIG: return "the requested launch configuration cannot run these sizes";
    case NA3D_ERR_STRIDE:
      return "a stride is negative or not a multiple of 8, k and v differ in H/W/NH strides, "
             "or out's strides map two elements to one address";
    case NA3D_ERR_BOX: return "the query box is empty or reaches outside the grid";
    case NA3D_ERR_VALUE: return "eps is negative or not finite";
    default: return "unknown status";
  }
}

int na3d_check_args(const void* q, const void* k, const void* v, const void* out, int B,
                    int T, int H, int W, int NH, int HD, int KT, int KH, int KW) {
  const Geom g = make_geom(B, T, H, W, NH, HD, KT, KH, KW, full_box(T, H, W));
  Strides st[4];
  contiguous_all(g, st);
  return check_all(q, k, v, out, g, st);
}

int na3d_check_args_strided(const void* q, const void* k, const void* v, const void* out, int B,
                            int T, int H, int W, int NH, int HD, int KT, int KH, int KW,
                            const long long* strides) {
  if (!strides) return NA3D_ERR_NULL;
  const Geom g = make_geom(B, T, H, W, NH, HD, KT, KH, KW, full_box(T, H, W));
  Strides st[4];
  read_strides(strides, st);
  return check_all(q, k, v, out, g, st);
}

int na3d_check_args_subgrid(const void* q, const void* k, const void* v, const void* out, int B,
                            int T, int H, int W, int NH, int HD, int KT, int KH, int KW,
                            const int* box, const long long* strides) {
  if (!box) return NA3D_ERR_NULL;
  const Geom g = make_geom(B, T, H, W, NH, HD, KT, KH, KW,
                           Box{box[0], box[1], box[2], box[3], box[4], box[5]});
  Strides st[4];
  if (strides)
    read_strides(strides, st);
  else
    contiguous_all(g, st);
  return check_all(q, k, v, out, g, st);
}

int na3d_plan(int B, int T, int H, int W, int NH, int HD, int KT, int KH, int KW, int* plan) {
  return na3d_plan_config(B, T, H, W, NH, HD, KT, KH, KW, 0, 0, 0, plan);
}

int na3d_plan_config(int B, int T, int H, int W, int NH, int HD, int KT, int KH, int KW,
                     int family, int variant, int tile_t, int* plan) {
  if (!plan) return NA3D_ERR_NULL;
  int rc = check_sizes(B, T, H, W, NH, HD, KT, KH, KW);
  if (rc != NA3D_OK) return rc;
  Geom g = make_geom(B, T, H, W, NH, HD, KT, KH, KW, full_box(T, H, W));
  g.kv_span = kv_span_bytes(contiguous(T, H, W, NH, HD), H, W, HD);
  g.qo_step = 2 * contiguous(T, H, W, NH, HD).t;
  Launch l;
  rc = make_plan_config(g, family, variant, tile_t, &l);
  if (rc != NA3D_OK) return rc;
  fill_plan(l, plan);
  return NA3D_OK;
}

int na3d_fwd(const void* q, const void* k, const void* v, void* out, int B, int T, int H,
             int W, int NH, int HD, int KT, int KH, int KW, void* stream) {
  return na3d_fwd_config(q, k, v, out, B, T, H, W, NH, HD, KT, KH, KW, 0, 0, 0, stream);
}

int na3d_fwd_config(const void* q, const void* k, const void* v, void* out, int B, int T,
                    int H, int W, int NH, int HD, int KT, int KH, int KW, int family,
                    int variant, int tile_t, void* stream) {
  const Geom g = make_geom(B, T, H, W, NH, HD, KT, KH, KW, full_box(T, H, W));
  Strides st[4];
  contiguous_all(g, st);
  return fwd_impl(q, k, v, out, g, st, family, variant, tile_t, stream);
}

int na3d_fwd_strided(const void* q, const void* k, const void* v, void* out, int B, int T,
                     int H, int W, int NH, int HD, int KT, int KH, int KW,
                     const long long* strides, void* stream) {
  return na3d_fwd_strided_config(q, k, v, out, B, T, H, W, NH, HD, KT, KH, KW, strides, 0, 0,
                                 0, stream);
}

int na3d_fwd_strided_config(const void* q, const void* k, const void* v, void* out, int B,
                            int T, int H, int W, int NH, int HD, int KT, int KH, int KW,
                            const long long* strides, int family, int variant, int tile_t,
                            void* stream) {
  if (!strides) return NA3D_ERR_NULL;
  const Geom g = make_geom(B, T, H, W, NH, HD, KT, KH, KW, full_box(T, H, W));
  Strides st[4];
  read_strides(strides, st);
  return fwd_impl(q, k, v, out, g, st, family, variant, tile_t, stream);
}

int na3d_fwd_subgrid(const void* q, const void* k, const void* v, void* out, int B, int T,
                     int H, int W, int NH, int HD, int KT, int KH, int KW, const int* box,
                     const long long* strides, void* stream) {
  return na3d_fwd_subgrid_config(q, k, v, out, B, T, H, W, NH, HD, KT, KH, KW, box, strides, 0,
                                 0, 0, stream);
}

int na3d_fwd_subgrid_config(const void* q, const void* k, const void* v, void* out, int B,
                            int T, int H, int W, int NH, int HD, int KT, int KH, int KW,
                            const int* box, const long long* strides, int family, int variant,
                            int tile_t, void* stream) {
  if (!box) return NA3D_ERR_NULL;
  const Geom g = make_geom(B, T, H, W, NH, HD, KT, KH, KW,
                           Box{box[0], box[1], box[2], box[3], box[4], box[5]});
  Strides st[4];
  if (strides)
    read_strides(strides, st);
  else
    contiguous_all(g, st);
  return fwd_impl(q, k, v, out, g, st, family, variant, tile_t, stream);
}

int na3d_check_args_rms_norm(const void* x, const void* weight, const void* y, int rows,
                             int dim, float eps) {
  return rms_check(x, weight, y, rows, dim, eps);
}

int na3d_rms_norm(const void* x, const void* weight, void* y, int rows, int dim, float eps,
                  void* stream) {
  return rms_impl(x, weight, y, rows, dim, eps, 0, stream);
}

int na3d_rms_norm_config(const void* x, const void* weight, void* y, int rows, int dim,
                         float eps, int workgroups, void* stream) {
  return rms_impl(x, weight, y, rows, dim, eps, workgroups, stream);
}

int na3d_check_args_batch(const na3d_tile* tiles, int n, int NH, int HD, int KT, int KH,
                          int KW) {
  return check_batch(tiles, n, NH, HD, KT, KH, KW);
}

int na3d_plan_batch(const na3d_tile* tiles, int n, int NH, int HD, int KT, int KH, int KW,
                    int* plan) {
  if (!plan) return NA3D_ERR_NULL;
  if (n < 0) return NA3D_ERR_SHAPE;
  if (n > 0 && !tiles) return NA3D_ERR_NULL;
  BatchPlan bp;
  const int rc = plan_batch(tiles, n, NH, HD, KT, KH, KW, &bp);
  if (rc != NA3D_OK) return rc;
  int solo = 0, shared = 0;
  for (int i = 0; i < n; ++i) (bp.shared[i] ? shared : solo) += 1;
  plan[0] = (int)bp.groups.size() + solo;
  plan[1] = bp.groups.empty() ? -1 : bp.variant;
  plan[2] = shared;
  int64_t w = 0;
  if (!bp.groups.empty())
    for (int i : bp.groups[0]) w += bp.plan[i].wgs;
  plan[3] = (int)w;
  return NA3D_OK;
}

int na3d_fwd_batch(const na3d_tile* tiles, int n, int NH, int HD, int KT, int KH, int KW,
                   void* stream) {
  return batch_impl(tiles, n, NH, HD, KT, KH, KW, stream);
}

}  // extern "C"
