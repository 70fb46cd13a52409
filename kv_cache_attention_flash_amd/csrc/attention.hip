// Scheduled attention over the paged cache for gfx950, with the two-view
// (Flash-Verify) visibility rule and the exact attention mass.
//
// Sources: [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for
// Fast, Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary):
// para 1 (attention scheduled through a block table over sequences whose cached
// lengths differ inside one batch), para 2 (most-attended tokens select the
// tracking set), para 3 (draft and mask views at the same positions, isolated
// by a mask inside the fused kernel; draft rows causal among themselves).
//
// Pass 1 (attn_fwd): one workgroup per (sequence, 64-row tile, head, KV split);
// 4 waves, each owning 16 query rows.  Keys stream in 32-slot tiles: the tile's
// K (row-major) and V (transposed) are staged in double-buffered LDS and shared
// by the 4 waves; the next tile's loads are in flight while a tile is used.
// Per wave S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys along M) so that each
// lane holds one query row: row maxima and sums are in-lane plus two shuffles,
// and the fp32 probabilities convert in-register into the B operand of
// O^T += V^T P^T.  The K rows feeding the two 16-key M tiles are permuted so
// that lane group g ends up holding the 8 consecutive keys 8g..8g+7, which
// makes each V^T operand one 16-byte LDS read.  Online softmax in base 2.
// With several KV splits the unnormalised partials are merged in a fixed split
// order: by attn_merge, or, when the mass is requested, by attn_finish.
//
// Mass: m[b][j] = sum_h sum_r exp(s_rj - LSE_r) needs every row's final
// log-sum-exp, known only after all keys, so the mass is a second pass over K
// (attn_mass) that first forms each row's LSE from the pass-1 maxima and
// normalisers; per-(sequence, head) partial sums are added over heads in head
// order by attn_finish, which also merges the split outputs.
// Nothing uses floating atomics: results are bitwise reproducible.
#include "device_common.h"
#include "internal.h"

namespace fdl {

namespace {

constexpr int KT = 32;  // keys per tile
#ifndef FDL_ATTN_NPF
#define FDL_ATTN_NPF 2
#endif
#ifndef FDL_ATTN_MNPF
#define FDL_ATTN_MNPF 2
#endif
#ifndef FDL_ATTN_ROWS_KLDS
#define FDL_ATTN_ROWS_KLDS 1  // row-group path: K through a wave-private LDS tile
#endif
#ifndef FDL_ATTN_ROWS_BUF
#define FDL_ATTN_ROWS_BUF 1  // row-group path: tiles read through range-checked buffer views
#endif
#if FDL_ATTN_ROWS_BUF && !FDL_ATTN_ROWS_KLDS
#error "buffer-view tile loads use the coalesced K layout"
#endif
constexpr float kNegInf = -__builtin_huge_valf();

struct SeqInfo {
  int r0, nrows, L, w0, wl, d0;
};

__device__ __forceinline__ SeqInfo seq_info(const AttnArgs &a, int b) {
  SeqInfo si;
  si.r0 = a.cu_rows[b];
  si.nrows = a.cu_rows[b + 1] - si.r0;
  si.L = min(a.kv_len[b], a.max_kv_len);  // a length past the stated bound is clamped
  if (a.views) {
    si.w0 = a.views[3 * b];
    si.wl = a.views[3 * b + 1];
    si.d0 = a.views[3 * b + 2];
  } else {
    si.w0 = si.wl = si.d0 = 0;
  }
  return si;
}

// Rows at or past cu_rows[batch] are inactive (num_rows is then a capacity):
// no output is written for them.
__device__ __forceinline__ int active_rows(const AttnArgs &a) {
  return max(0, min(a.rows, a.cu_rows[a.batch]));
}

// The slots local row t of a sequence may see, as intervals: slot j is visible
// iff (j < lim and not x0 <= j < x1) or y0 <= j <= y1.
//   plain row:        [0, L)
//   draft row i:      context [0, min(d0, L)) minus the window [w0, w0 + W),
//                     plus the draft slots d0 .. d0 + i (causal)
//   mask row:         [0, min(d0, L))  (context and the whole window)
//   missing row:      nothing
struct Vis {
  int lim, x0, x1, y0, y1;
  // Non-short-circuit operators: compares and mask logic, no branches.
  __device__ __forceinline__ bool operator()(int j) const {
    return ((j < lim) & ((j < x0) | (j >= x1))) | ((j >= y0) & (j <= y1));
  }
  // Every slot of [k0, k0 + n) visible.
  __device__ __forceinline__ bool all(int k0, int n) const {
    return (k0 + n <= lim) & ((k0 + n <= x0) | (k0 >= x1));
  }
  // No slot of [k0, k0 + n) visible.
  __device__ __forceinline__ bool none(int k0, int n) const {
    return ((k0 >= lim) | ((k0 >= x0) & (k0 + n <= x1))) &
           ((y1 < k0) | (y0 >= k0 + n) | (y0 > y1));
  }
};

// Whole-wave visibility of one 32-key tile: 2 = every lane sees every key,
// 0 = no lane sees any key, 1 = mixed (test key by key).
__device__ __forceinline__ int tile_vis(const Vis &vis, int key0) {
  if (__all(vis.all(key0, 32))) return 2;
  if (__all(vis.none(key0, 32))) return 0;
  return 1;
}

// Online-softmax step for one 32-key tile held as S^T fragments (lane: query
// row lane % 16, keys key0 + 8g + 4mt + e).  Updates the row's running max m
// (log2 units) and normaliser l, writes the scaled scores to xs (-inf where
// not visible), rescales o by the change of max and returns the bf16 P^T
// operand of the PV product.  exp2(-inf) is 0, so hidden keys need no select.
template <int NO>
__device__ __forceinline__ u32x4 tile_softmax(const f32x4 s[2], const Vis &vis, int tv, int key0,
                                              int g, float scale, float &m, float &l, f32x4 *o,
                                              float *xs) {
  if (tv == 2) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[mt * 4 + e] = s[mt][e] * scale;
  } else {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        xs[mt * 4 + e] = vis(key0 + 8 * g + 4 * mt + e) ? s[mt][e] * scale : kNegInf;
  }
  float tmax = fmaxf(fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3])),
                     fmaxf(fmaxf(xs[4], xs[5]), fmaxf(xs[6], xs[7])));
  tmax = rows4_max(tmax);
  const float mnew = fmaxf(m, tmax);
  const float msafe = mnew == kNegInf ? 0.f : mnew;  // a row that has seen nothing keeps zeros
  const float alpha = fast_exp2(m - msafe);
  float pv[8], rs = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pv[e] = fast_exp2(xs[e] - msafe);
    rs += pv[e];
  }
  rs = rows4_sum(rs);
  l = l * alpha + rs;
  m = mnew;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int dm = 0; dm < NO; ++dm) o[dm] *= alpha;
  }
  u32x4 pb;
  pb[0] = cvt_pk_bf16(pv[0], pv[1]);
  pb[1] = cvt_pk_bf16(pv[2], pv[3]);
  pb[2] = cvt_pk_bf16(pv[4], pv[5]);
  pb[3] = cvt_pk_bf16(pv[6], pv[7]);
  return pb;
}

__device__ __forceinline__ Vis row_vis(const SeqInfo &si, int t, bool row_ok) {
  Vis v{0, 0, 0, 1, 0};
  if (!row_ok) return v;
  if (si.wl == 0) {
    v.lim = si.L;
  } else {
    v.lim = min(si.d0, si.L);
    if (t < si.wl) {
      v.x0 = si.w0;
      v.x1 = si.w0 + si.wl;
      v.y0 = si.d0;
      v.y1 = min(si.d0 + t, si.L - 1);
    }
  }
  return v;
}

// One 32-key tile of head h moves global -> registers -> LDS, K and V both
// row-major ([key][D + pad]), by one group of 256 threads (NCH 16-byte chunks
// of K and of V per thread).
template <int D>
struct Tile {
  static constexpr int CH = D / 8;                  // 16-byte chunks per key
  static constexpr int NCH = KT * CH / 256;         // chunks per thread
  u32x4 k[NCH], v[NCH];
};
template <int D> constexpr int kVPad = D + 16;  // V row stride: conflict-free transposed reads

// Slot (in 16-byte chunks) of chunk ch of key row key in a K tile held in LDS.
// One MFMA operand read gathers one chunk of the 16 keys 8a + b + 4m (a, b
// < 4): the chunk index is XORed with the key bits that vary over that set,
// so the 16 reads land in distinct banks.  D = 128: bits 0, 1, 3, 4 of the
// key; D = 64 (two rows per 256-byte bank line, told apart by bit 0): bits 1,
// 3, 4.  A row's chunks stay a permutation of its slots, so the coalesced
// writes are conflict-free too.
template <int D>
__device__ __forceinline__ int kslot(int key, int ch) {
  static_assert(D == 64 || D == 128, "head size");
  if constexpr (D == 128) return key * 16 + (ch ^ ((key & 3) | ((key >> 1) & 12)));
  else return key * 8 + (ch ^ (((key >> 1) & 1) | ((key >> 2) & 6)));
}


// Physical pages of the tiles a workgroup visits, staged once in LDS so that a
// tile's address never waits on a block-table load.
constexpr int kMaxPages = 1024;

__device__ __forceinline__ void stage_pages(const AttnArgs &a, int b, int tb, int te, int *s_page) {
  const int sh = a.c.bs_shift;
  const int p0 = (tb * KT) >> sh, p1 = te > tb ? ((te * KT - 1) >> sh) + 1 : p0;
  for (int i = threadIdx.x; i < p1 - p0; i += blockDim.x)
    s_page[i] = a.c.block_table[(size_t)b * a.c.max_blocks + p0 + i];
}

template <int D>
__device__ __forceinline__ void load_tile(Tile<D> &t, const AttnArgs &a, const int *s_page, int tb,
                                          int h, int key0, bool want_v, int gtid) {
  const int sh = a.c.bs_shift;
  const int page = s_page[(key0 >> sh) - ((tb * KT) >> sh)];
  const size_t base = ((((size_t)page * a.c.H + h) << sh) + (key0 & (a.c.bs - 1))) * D;
#pragma unroll
  for (int i = 0; i < Tile<D>::NCH; ++i) {
    const int c = gtid + 256 * i;
    t.k[i] = ld16(a.c.k + base + (size_t)c * 8);
    if (want_v) t.v[i] = ld16(a.c.v + base + (size_t)c * 8);
  }
}

// V rows at or past the cached length (vkeys valid keys in the tile) are
// stored as zeros: those slots' contents are unspecified, and a zero weight
// times a NaN would still poison the product.
template <int D>
__device__ __forceinline__ void store_tile(const Tile<D> &t, u32x4 *klds,
                                           uint16_t (*vlds)[kVPad<D>], bool want_v, int gtid,
                                           int vkeys = KT) {
  const bool part = vkeys < KT;
#pragma unroll
  for (int i = 0; i < Tile<D>::NCH; ++i) {
    const int c = gtid + 256 * i;
    const int key = c / Tile<D>::CH, dc = c % Tile<D>::CH;
    klds[kslot<D>(key, dc)] = t.k[i];
    if (want_v)
      st16(&vlds[key][dc * 8], part && key >= vkeys ? u32x4{0u, 0u, 0u, 0u} : t.v[i]);
  }
}

// V^T operand of O^T += V^T P^T for features 16*dm .. 16*dm+15: lane l needs
// keys 8g .. 8g+7 (g = l / 16) of feature 16*dm + l % 16.  ds_read_tr16_b64
// gives lane i of a 16-lane group element k = position i % 4 of the 8-byte
// chunk addressed by lane 4k + i / 4; addressing V[kb + a/4][d0 + 4*(a%4)] from
// lane a therefore hands lane i the keys kb .. kb+3 of feature d0 + i.
template <int D>
__device__ __forceinline__ u32x4 vt_operand(uint16_t (*vlds)[kVPad<D>], int dm, int lane) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int g = lane >> 4, i = lane & 15;
  const uint16_t *p0 = &vlds[8 * g + (i >> 2)][16 * dm + 4 * (i & 3)];
  const uint16_t *p1 = &vlds[8 * g + 4 + (i >> 2)][16 * dm + 4 * (i & 3)];
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p0));
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p1));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// S^T tile (32 keys x 16 rows) for one wave: s[mt][e] is key 8g + 4mt + e for
// query row (lane & 15).
template <int D>
__device__ __forceinline__ void scores(const u32x4 *klds, const u32x4 *qf,
                                       int lane, f32x4 s[2]) {
  const int g = lane >> 4, j = lane & 15;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int key = 8 * (j >> 2) + 4 * mt + (j & 3);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      u32x4 kf = klds[kslot<D>(key, 4 * ks + g)];
      acc = mfma16(kf, qf[ks], acc);
    }
    s[mt] = acc;
  }
}

template <int D>
__device__ __forceinline__ void load_q(const AttnArgs &a, int r, int h, bool ok, int g,
                                       u32x4 *qf) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = ok ? ld16(a.q + ((size_t)r * a.c.H + h) * D + 32 * ks + 8 * g)
                : u32x4{0u, 0u, 0u, 0u};
}

// Pass 1.  8 waves: key group kg = wave / 4 takes the unit's even or odd
// tiles, row group wave % 4 owns 16 query rows; the two key groups keep their
// own online-softmax state and are combined through LDS at the end (group 0
// first), so two waves per SIMD hide each other's latency.
template <int D>
__global__ __launch_bounds__(512) void attn_fwd_kernel(AttnArgs a, AttnPlan p) {
  constexpr int NPF = FDL_ATTN_NPF;  // tiles in flight per key group
  // K tiles (swizzled chunks); 8 chunks more per tile make room for the
  // merge scratch that reuses them.
  __shared__ u32x4 klds[2][2][KT * D / 8 + 8];
  __shared__ uint16_t vlds[2][2][KT][kVPad<D>];

  int u = blockIdx.x;
  const int split = u % p.splits; u /= p.splits;
  const int h = u % a.c.H; u /= a.c.H;
  const int rt = u % p.row_tiles;
  const int b = u / p.row_tiles;
  const SeqInfo si = seq_info(a, b);
  const int t0 = rt * 64;
  if (t0 >= si.nrows) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kg = wave >> 2, wr = wave & 3, gtid = threadIdx.x & 255;
  const int g = lane >> 4, j = lane & 15;
  const int t = t0 + wr * 16 + j;  // local row of this lane
  const bool row_ok = t < si.nrows;
  const int r = si.r0 + (row_ok ? t : 0);
  const Vis vis = row_vis(si, t, row_ok);

  const int tiles = (si.L + KT - 1) / KT;
  const int tps = (tiles + p.splits - 1) / p.splits;
  const int tb = split * tps, te = min(tiles, tb + tps);
  const int niter = (te - tb + 1) / 2;  // iterations per key group (group 1 may idle in the last)

  __shared__ int s_page[kMaxPages];
  stage_pages(a, b, tb, te, s_page);
  lds_barrier();
  // Loads are unconditional (tile index clamped to the unit's last tile; the
  // repeats hit L2) so the compiler keeps the other stage in flight.
  const int tlast = max(te - 1, tb);
  Tile<D> pf[NPF];
  if (te > tb) {
#pragma unroll
    for (int i = 0; i < NPF; ++i)
      load_tile<D>(pf[i], a, s_page, tb, h, min(tb + kg + 2 * i, tlast) * KT, true, gtid);
  }
  u32x4 qf[D / 32];
  load_q<D>(a, r, h, row_ok, g, qf);

  f32x4 o[D / 16];
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) o[dm] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;

  // Every iteration has the same shape: one ring stage stored to LDS, the
  // same stage reloaded, a barrier, then the tile's math only if the tile
  // exists.  With no branch around a load, the compiler waits for exactly
  // the stage it needs and keeps the other stages in flight.
  const int niter_r = (niter + NPF - 1) / NPF * NPF;
  for (int it0 = 0; it0 < niter_r; it0 += NPF) {
#pragma unroll
    for (int ii = 0; ii < NPF; ++ii) {
      const int it = it0 + ii;
      const int tile = tb + kg + 2 * it;
      const bool have = it < niter && tile < te;
      const int buf = it & 1;  // alternates across iterations for any NPF
      store_tile<D>(pf[ii], klds[kg][buf], vlds[kg][buf], true, gtid, si.L - tile * KT);
      load_tile<D>(pf[ii], a, s_page, tb, h, min(tile + 2 * NPF, tlast) * KT, true, gtid);
      lds_barrier();
      const int key0 = tile * KT;
      const int tv = have ? tile_vis(vis, key0) : 0;
      if (tv != 0) {
        f32x4 s[2];
        scores<D>(klds[kg][buf], qf, lane, s);
        float xs[8];
        const u32x4 pb = tile_softmax<D / 16>(s, vis, tv, key0, g, a.scale_log2, m, l, o, xs);
#pragma unroll
        for (int dm = 0; dm < D / 16; ++dm)
          o[dm] = mfma16(vt_operand<D>(vlds[kg][buf], dm, lane), pb, o[dm]);
      }
    }
  }

  // Combine the two key groups (group 1's state through LDS, reusing the tiles).
  lds_barrier();
  float *mo = reinterpret_cast<float *>(&klds[0][0][0]);  // [4 row groups][16 rows][D]
  float *mml = mo + 64 * D;                                   // [64 rows][2]
  static_assert((64 * D + 128) * 4 <= (int)sizeof(klds), "merge scratch");
  const int rl = wr * 16 + j;
  if (kg == 1) {
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm)
      *reinterpret_cast<f32x4 *>(&mo[rl * D + 16 * dm + 4 * g]) = o[dm];
    if (g == 0) {
      mml[2 * rl] = m;
      mml[2 * rl + 1] = l;
    }
  }
  lds_barrier();
  if (kg == 1 || !row_ok) return;
  {
    const float m1 = mml[2 * rl], l1 = mml[2 * rl + 1];
    const float mx = fmaxf(m, m1);
    const float f0 = m == kNegInf ? 0.f : exp2f(m - mx);
    const float f1 = m1 == kNegInf ? 0.f : exp2f(m1 - mx);
    l = l * f0 + l1 * f1;
    m = mx;
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm)
      o[dm] = o[dm] * f0 + *reinterpret_cast<const f32x4 *>(&mo[rl * D + 16 * dm + 4 * g]) * f1;
  }
  // o[dm][e] = O[row][16 dm + 4 g + e]
  if (p.splits == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *dst = a.out + ((size_t)r * a.c.H + h) * D + 4 * g;
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) {
      f32x4 val = o[dm] * inv;
      *reinterpret_cast<f32x4 *>(dst + 16 * dm) = val;
    }
    if (p.mass_splits && g == 0) {
      float *lse = reinterpret_cast<float *>(a.ws + p.off_lse);
      lse[(size_t)r * a.c.H + h] = l > 0.f ? m + log2f(l) : kNegInf;
    }
  } else {
    float *po = reinterpret_cast<float *>(a.ws + p.off_part_o);
    float *pml = reinterpret_cast<float *>(a.ws + p.off_part_ml);
    const size_t rh = ((size_t)split * a.rows + r) * a.c.H + h;
    float *dst = po + rh * D + 4 * g;
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) *reinterpret_cast<f32x4 *>(dst + 16 * dm) = o[dm];
    if (g == 0) {
      pml[2 * rh] = m;
      pml[2 * rh + 1] = l;
    }
  }
}

// Combine the KV-split partials of row r, head h: the global maximum, the
// rescaled normaliser and, when asked, the DW output features starting at d0.
template <int DW>
__device__ __forceinline__ float merge_row(const AttnArgs &a, const AttnPlan &p, size_t rh,
                                           int D, int d0, float *out_or_null) {
  const float *po = reinterpret_cast<const float *>(a.ws + p.off_part_o);
  const float *pml = reinterpret_cast<const float *>(a.ws + p.off_part_ml);
  const size_t stride = (size_t)a.rows * a.c.H;
  float mx = kNegInf;
#pragma unroll 8
  for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, pml[2 * (s * stride + rh)]);
  f32x4 acc[DW / 4];
#pragma unroll
  for (int i = 0; i < DW / 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (mx != kNegInf) {
#pragma unroll 4
    for (int s = 0; s < p.splits; ++s) {
      const size_t k = s * stride + rh;
      const float ms = pml[2 * k];
      const float f = ms == kNegInf ? 0.f : exp2f(ms - mx);
      l += pml[2 * k + 1] * f;
      if (out_or_null) {
#pragma unroll
        for (int i = 0; i < DW / 4; ++i)
          acc[i] += *reinterpret_cast<const f32x4 *>(po + k * D + d0 + 4 * i) * f;
      }
    }
  }
  if (out_or_null) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < DW / 4; ++i)
      *reinterpret_cast<f32x4 *>(out_or_null + rh * D + d0 + 4 * i) = acc[i] * inv;
  }
  return l > 0.f ? mx + log2f(l) : kNegInf;
}

// Merge KV-split partials (no mass requested): one thread per (row, head, 4 features).
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, AttnPlan p) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t rh = idx / (D / 4);
  const int d4 = (int)(idx % (D / 4)) * 4;
  if (rh >= (size_t)active_rows(a) * a.c.H) return;
  merge_row<4>(a, p, rh, D, d4, a.out);
}

// Attention mass pass: one workgroup per (sequence, head, key chunk).  Each
// lane first forms its row's LSE (from pass 1 directly, or by combining the
// KV-split maxima and normalisers, loaded with the first K tile), then K
// tiles stream through double-buffered LDS and P = exp2(s - LSE) is summed over
// the rows: in-wave by a reduce-scatter over the 16 row lanes, across the
// 4 waves in wave order.
template <int D>
__global__ __launch_bounds__(256) void attn_mass_kernel(AttnArgs a, AttnPlan p) {
  constexpr int MAXK = 32 * KT;  // keys per chunk (bounded by the host plan)
  __shared__ u32x4 klds[2][KT * D / 8];
  __shared__ float wsum[4][KT];
  __shared__ float macc[MAXK];

  // Reverse order, blocks and tiles alike: pass 1 read the last units' last
  // tiles most recently, so they are the likeliest still to sit in the
  // last-level cache.  Per-key sums do not depend on this order.
  int u = gridDim.x - 1 - blockIdx.x;
  const int chunk = u % p.mass_splits; u /= p.mass_splits;
  const int h = u % a.c.H;
  const int b = u / a.c.H;
  const SeqInfo si = seq_info(a, b);
  const int tiles = (si.L + KT - 1) / KT;
  const int tpc = (tiles + p.mass_splits - 1) / p.mass_splits;
  const int tb = chunk * tpc, te = min(tiles, tb + tpc);
  const int nrt = (si.nrows + 63) / 64;
  if (tb >= te) return;
  const int nkeys = max(0, te - tb) * KT;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const float *lse_ws = reinterpret_cast<const float *>(a.ws + p.off_lse);

  __shared__ int s_page[kMaxPages];
  stage_pages(a, b, tb, te, s_page);
  for (int k = threadIdx.x; k < nkeys; k += blockDim.x) macc[k] = 0.f;
  lds_barrier();

  for (int rt = 0; rt < nrt; ++rt) {
    const int t = rt * 64 + wave * 16 + j;
    const bool row_ok = t < si.nrows;
    const int r = si.r0 + (row_ok ? t : 0);
    const size_t rh = (size_t)r * a.c.H + h;
    const Vis vis = row_vis(si, t, row_ok);
    constexpr int MNPF = FDL_ATTN_MNPF;  // K tiles in flight
    Tile<D> pf[MNPF];
#pragma unroll
    for (int i = 0; i < MNPF; ++i)
      load_tile<D>(pf[i], a, s_page, tb, h, max(te - 1 - i, tb) * KT, false, threadIdx.x);
    u32x4 qf[D / 32];
    load_q<D>(a, r, h, row_ok, g, qf);
    float lr = kNegInf;
    if (row_ok) lr = p.splits == 1 ? lse_ws[rh] : merge_row<4>(a, p, rh, D, 0, nullptr);
    // A row that sees no key has LSE -inf; subtracting +inf instead sends
    // every exp2 to 0.
    const float lsafe = lr == kNegInf ? __builtin_huge_valf() : lr;

    // Same uniform ring as pass 1: no branch around a load.
    const int nt_r = (te - tb + MNPF - 1) / MNPF * MNPF;
    for (int it0 = 0; it0 < nt_r; it0 += MNPF) {
#pragma unroll
    for (int ii = 0; ii < MNPF; ++ii) {
      const int tile = te - 1 - (it0 + ii);  // descending
      const bool have = tile >= tb;
      const int buf = ii & 1;
      store_tile<D>(pf[ii], klds[buf], nullptr, false, threadIdx.x);
      load_tile<D>(pf[ii], a, s_page, tb, h, max(tile - MNPF, tb) * KT, false, threadIdx.x);
      lds_barrier();
      if (have) {
      const int key0 = tile * KT;
      const int tv = tile_vis(vis, key0);
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = 0.f;
      if (tv != 0) {
        f32x4 s[2];
        scores<D>(klds[buf], qf, lane, s);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = fast_exp2(s[mt][e] * a.scale_log2 - lsafe);
            pv[mt * 4 + e] = (tv == 2 || vis(key0 + 8 * g + 4 * mt + e)) ? x : 0.f;
          }
      }
      // Reduce over the 16 rows of the wave (lanes sharing g): reduce-scatter.
      const int b3 = (j >> 3) & 1, b2 = (j >> 2) & 1, b1 = (j >> 1) & 1;
      float q4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float give = b3 ? pv[i] : pv[i + 4];
        const float keep = b3 ? pv[i + 4] : pv[i];
        q4[i] = keep + lane_xor8(give);
      }
      float q2[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float give = b2 ? q4[i] : q4[i + 2];
        const float keep = b2 ? q4[i + 2] : q4[i];
        q2[i] = keep + lane_xor4(give);
      }
      float q1;
      {
        const float give = b1 ? q2[0] : q2[1];
        const float keep = b1 ? q2[1] : q2[0];
        q1 = keep + lane_xor2(give);
      }
      // Lanes l and l^1 now hold the same key; add them in a fixed order.
      const float other = lane_xor1(q1);
      const float tot = (j & 1) ? other + q1 : q1 + other;
      if ((j & 1) == 0) wsum[wave][8 * g + 4 * b3 + 2 * b2 + b1] = tot;
      }
      lds_barrier();
      if (have && threadIdx.x < KT) {
        const int k = threadIdx.x;
        const float sum = ((wsum[0][k] + wsum[1][k]) + wsum[2][k]) + wsum[3][k];
        macc[(tile - tb) * KT + k] += sum;
      }
    }
    }
    lds_barrier();
  }
  float *mp = reinterpret_cast<float *>(a.ws + p.off_mass_part) +
              ((size_t)b * a.c.H + h) * a.mass_stride;
  for (int k = threadIdx.x; k < nkeys; k += blockDim.x) {
    const int jj = tb * KT + k;
    if (jj < si.L) mp[jj] = macc[k];
  }
}

// Last launch of a mass-requesting call: blocks [0, nb_mass) add the per-head
// partial masses in head order (mass[b][j]; the loads of 32 heads are issued
// before their sum), blocks after that merge the KV-split partial outputs
// (one thread per row, head and 4 features), when there are splits.
template <int D>
__global__ __launch_bounds__(256) void attn_finish_kernel(AttnArgs a, AttnPlan p, int nb_mass) {
  if ((int)blockIdx.x >= nb_mass) {
    const size_t idx = (size_t)(blockIdx.x - nb_mass) * blockDim.x + threadIdx.x;
    const size_t rh = idx / (D / 4);
    const int d4 = (int)(idx % (D / 4)) * 4;
    if (rh < (size_t)active_rows(a) * a.c.H) merge_row<4>(a, p, rh, D, d4, a.out);
    return;
  }
  const int per_b = (a.mass_stride + 255) / 256;
  const int b = blockIdx.x / per_b;
  const int jj = (blockIdx.x % per_b) * blockDim.x + threadIdx.x;
  if (jj >= a.mass_stride) return;
  const int L = min(a.kv_len[b], a.max_kv_len);
  float sum = 0.f;
  if (jj < L) {
    const float *mp = reinterpret_cast<const float *>(a.ws + p.off_mass_part) +
                      (size_t)b * a.c.H * a.mass_stride + jj;
    for (int h0 = 0; h0 < a.c.H; h0 += 32) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = h0 + i < a.c.H ? mp[(size_t)(h0 + i) * a.mass_stride] : 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (h0 + i < a.c.H) sum += v[i];
    }
  }
  a.mass[(size_t)b * a.mass_stride + jj] = sum;
}


// Row-group attention: one workgroup per (sequence, head, 16-row group) over
// the whole cached length.  The workgroup therefore ends with every row's
// final log-sum-exp and needs no split merge; with the mass requested it also
// needs no second pass over K.  8 waves = 8 key groups, wave w taking tiles
// w, w + 8, ...  A wave loads its K and V tiles with coalesced 16-byte loads
// and passes both through wave-private LDS tiles, so the key loop has no
// workgroup barrier: K is read back in the MFMA operand layout (lane j of
// M-tile mt takes key 8(j/4) + 4mt + j%4, the permutation that leaves lane
// group g holding keys 8g .. 8g+7 of S^T), V transposed.  Two tiles per wave
// are in flight.
// With the mass requested each wave keeps its scaled scores (at most MAXT
// tiles) in registers and, once the workgroup has combined the waves' maxima
// and normalisers, sums exp2(s - LSE) over its 16 rows for each of its keys.
constexpr int kRowWaves = 8;

// LDS of one row-group workgroup.
template <int D>
struct RowsLds {
#if FDL_ATTN_ROWS_KLDS
  u32x4 kbuf[kRowWaves][KT * D / 8];
#endif
  uint16_t vbuf[kRowWaves][KT][kVPad<D>];
  int s_page[kMaxPages];
  float s_ml[kRowWaves][16][2];
  float s_inv[16];
};

// The workgroup body: item bid of nb (LDS from the caller, so a fused kernel
// can share one buffer across phases).
template <int D, int MAXT, bool MASS>
__device__ __forceinline__ void attn_rows_body(const AttnArgs &a, const AttnPlan &p, int bid,
                                               int nb, RowsLds<D> &L) {
  constexpr int KS = D / 32;            // MFMA k-steps per key row
  constexpr int CH = D / 8;             // 16-byte chunks per key row
  constexpr int VLD = KT * CH / 64;     // V chunks per lane per tile
  constexpr int NST = 2;                // tiles in flight per wave
  static_assert(kRowWaves * 16 * D * 4 <= kRowWaves * KT * kVPad<D> * 2, "merge scratch");
  auto &vbuf = L.vbuf;
  auto &s_page = L.s_page;
  auto &s_ml = L.s_ml;
  auto &s_inv = L.s_inv;

  // Blocks are dealt to the 8 XCDs round-robin; map them so that the row
  // groups of one (sequence, head) run on one XCD and share its L2.
  int u = bid;
  if ((nb & 7) == 0) u = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int rg = u % p.rgroups;
  u /= p.rgroups;
  const int h = u % a.c.H;
  const int b = u / a.c.H;
  const SeqInfo si = seq_info(a, b);
  const int t0 = rg * 16;
  if (t0 >= si.nrows) return;

  // The wave index in a scalar register: the tile schedule and the tile
  // descriptors derived from it are then wave-uniform to the compiler too.
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int t = t0 + j;  // local row of this lane
  const bool row_ok = t < si.nrows;
  const int r = si.r0 + (row_ok ? t : 0);
  const Vis vis = row_vis(si, t, row_ok);
  const int tiles = (si.L + KT - 1) / KT;
  const int n_w = tiles > w ? (tiles - 1 - w) / kRowWaves + 1 : 0;  // this wave's tiles

  stage_pages(a, b, 0, tiles, s_page);
  u32x4 qf[KS];
  load_q<D>(a, r, h, row_ok, g, qf);
  lds_barrier();

  struct Stage {
    u32x4 k[2 * KS];
    u32x4 v[VLD];
  };
  // Loads of the wave's kk-th tile.  Past the wave's last tile the same number
  // of load instructions is issued at one fixed 16-byte address (every lane
  // alike), so the count of loads in flight never depends on the data.
#if FDL_ATTN_ROWS_BUF
  // Wave-uniform descriptors per tile: the tile's keys are one contiguous run
  // of a page; keys at or past the cached length (and every key of a padding
  // tile) lie outside the view and load as zeros, so V needs no masking and
  // the per-lane addresses are the same for every tile.
  const int bs_log2 = __builtin_ctz(a.c.bs);
  auto issue = [&](Stage &st, int kk) {
    const int key0 = (w + kRowWaves * kk) * KT;
    size_t off = 0;
    int bytes = 0;
    if (kk < n_w) {
      const int page = __builtin_amdgcn_readfirstlane(s_page[key0 >> bs_log2]);
      off = (((size_t)page * a.c.H + h) * a.c.bs + (key0 & (a.c.bs - 1))) * D;
      bytes = min(KT, si.L - key0) * D * 2;
    }
    const auto rk = buffer_view(a.c.k + off, bytes), rv = buffer_view(a.c.v + off, bytes);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) st.k[i] = buffer_ld16(rk, (lane + 64 * i) * 16);
#pragma unroll
    for (int i = 0; i < VLD; ++i) st.v[i] = buffer_ld16(rv, (lane + 64 * i) * 16);
  };
#else
  auto issue = [&](Stage &st, int kk) {
    const bool real = kk < n_w;
    const int key0 = (w + kRowWaves * kk) * KT;
    size_t base = 0;
    if (real) {
      const int page = s_page[key0 / a.c.bs];
      base = (((size_t)page * a.c.H + h) * a.c.bs + (key0 % a.c.bs)) * D;
    }
#if FDL_ATTN_ROWS_KLDS
    // A tile's keys are one contiguous run of its page: whole 128-byte lines
    // per 8 lanes, the operand layout being formed in LDS.
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i)
      st.k[i] = ld16(a.c.k + (real ? base + (size_t)(lane + 64 * i) * 8 : (size_t)0));
#else
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int key = 8 * (j >> 2) + 4 * mt + (j & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        st.k[mt * KS + ks] =
            ld16(a.c.k + (real ? base + (size_t)key * D + 32 * ks + 8 * g : (size_t)0));
    }
#endif
#pragma unroll
    for (int i = 0; i < VLD; ++i)
      st.v[i] = ld16(a.c.v + (real ? base + (size_t)(lane + 64 * i) * 8 : (size_t)0));
  };
#endif

  f32x4 o[D / 16];
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) o[dm] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;
  uint16_t(*vb)[kVPad<D>] = vbuf[w];

  // One tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  xs receives the
  // scaled scores (-inf where not visible).
  auto process = [&](const Stage &st, int kk, float *xs) {
    const int key0 = (w + kRowWaves * kk) * KT;
    const int tv = tile_vis(vis, key0);
    if (tv == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[e] = kNegInf;
      return;
    }
#if FDL_ATTN_ROWS_KLDS
    u32x4 *kb = L.kbuf[w];
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      const int c = lane + 64 * i;
      kb[kslot<D>(c / CH, c % CH)] = st.k[i];
    }
#endif
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#if FDL_ATTN_ROWS_KLDS
      const int key = 8 * (j >> 2) + 4 * mt + (j & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16(kb[kslot<D>(key, 4 * ks + g)], qf[ks], acc);
#else
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16(st.k[mt * KS + ks], qf[ks], acc);
#endif
      s[mt] = acc;
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int c = lane + 64 * i;
      const int key = c / CH;
#if FDL_ATTN_ROWS_BUF
      st16(&vb[key][(c % CH) * 8], st.v[i]);  // zeros past the length
#else
      const bool part = key0 + KT > si.L;
      st16(&vb[key][(c % CH) * 8],
           part && key0 + key >= si.L ? u32x4{0u, 0u, 0u, 0u} : st.v[i]);
#endif
    }
    const u32x4 pb = tile_softmax<D / 16>(s, vis, tv, key0, g, a.scale_log2, m, l, o, xs);
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) o[dm] = mfma16(vt_operand<D>(vb, dm, lane), pb, o[dm]);
  };

  Stage st[NST];
  float sc[MASS ? MAXT : 1][8];
  if (n_w > 0) {
#pragma unroll
    for (int i = 0; i < NST; ++i) issue(st[i], i);
    if constexpr (MASS) {
      // No wave has more than MAXT tiles: loads for tiles past it would only
      // be waited for (before their registers are reused) at the merge.
#pragma unroll
      for (int kk = 0; kk < MAXT; ++kk) {
        if (kk < n_w) process(st[kk % NST], kk, sc[kk]);
        if (kk + NST < MAXT) issue(st[kk % NST], kk + NST);
      }
    } else {
      for (int kk0 = 0; kk0 < n_w; kk0 += NST) {
#pragma unroll
        for (int i = 0; i < NST; ++i) {
          if (kk0 + i < n_w) process(st[i], kk0 + i, sc[0]);
          issue(st[i], kk0 + i + NST);
        }
      }
    }
  }

  // Combine the 8 waves (fixed wave order): maxima and normalisers per row,
  // then the rescaled partial outputs through LDS (reusing the V buffers).
  if (g == 0) {
    s_ml[w][j][0] = m;
    s_ml[w][j][1] = l;
  }
  lds_barrier();
  float mws[kRowWaves], lws[kRowWaves];  // read once, then combined without branches
#pragma unroll
  for (int ww = 0; ww < kRowWaves; ++ww) {
    mws[ww] = s_ml[ww][j][0];
    lws[ww] = s_ml[ww][j][1];
  }
  float mx = kNegInf;
#pragma unroll
  for (int ww = 0; ww < kRowWaves; ++ww) mx = fmaxf(mx, mws[ww]);
  float lsum = 0.f;
#pragma unroll
  for (int ww = 0; ww < kRowWaves; ++ww) {
    const float e = exp2f(mws[ww] - mx);
    lsum += mws[ww] == kNegInf ? 0.f : lws[ww] * e;
  }
  const float fself = m == kNegInf ? 0.f : exp2f(m - mx);
  const float lse = lsum > 0.f ? mx + log2f(lsum) : kNegInf;
  float *ob = reinterpret_cast<float *>(&vbuf[0][0][0]);  // [8 waves][16 rows][D]
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm)
    *reinterpret_cast<f32x4 *>(&ob[(w * 16 + j) * D + 16 * dm + 4 * g]) = o[dm] * fself;
  if (w == 0 && g == 0) s_inv[j] = lsum > 0.f ? 1.f / lsum : 0.f;
  lds_barrier();
  if (threadIdx.x < 16 * D / 4) {
    const int row = threadIdx.x / (D / 4), f4 = (threadIdx.x % (D / 4)) * 4;
    f32x4 acc = *reinterpret_cast<const f32x4 *>(&ob[row * D + f4]);
#pragma unroll
    for (int ww = 1; ww < kRowWaves; ++ww)
      acc += *reinterpret_cast<const f32x4 *>(&ob[(ww * 16 + row) * D + f4]);
    if (t0 + row < si.nrows)
      *reinterpret_cast<f32x4 *>(a.out + ((size_t)(si.r0 + t0 + row) * a.c.H + h) * D + f4) =
          acc * s_inv[row];
  }

  if constexpr (MASS) {
    // Mass of the wave's keys over its 16 rows: a reduce-scatter over the
    // 16 row lanes leaves lanes j, j^1 with one key each.
    float *mp = reinterpret_cast<float *>(a.ws + p.off_mass_part) +
                (((size_t)b * a.c.H + h) * p.rgroups + rg) * a.mass_stride;
    const int b3 = (j >> 3) & 1, b2 = (j >> 2) & 1, b1 = (j >> 1) & 1;
#pragma unroll
    for (int kk = 0; kk < MAXT; ++kk) {
      if (kk >= n_w) break;
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pv[e] = (sc[kk][e] != kNegInf && lse != kNegInf) ? fast_exp2(sc[kk][e] - lse) : 0.f;
      float q4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float give = b3 ? pv[i] : pv[i + 4];
        const float keep = b3 ? pv[i + 4] : pv[i];
        q4[i] = keep + lane_xor8(give);
      }
      float q2[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float give = b2 ? q4[i] : q4[i + 2];
        const float keep = b2 ? q4[i + 2] : q4[i];
        q2[i] = keep + lane_xor4(give);
      }
      const float give = b1 ? q2[0] : q2[1];
      const float keep = b1 ? q2[1] : q2[0];
      const float q1 = keep + lane_xor2(give);
      const float other = lane_xor1(q1);
      const float tot = (j & 1) ? other + q1 : q1 + other;
      const int jj = (w + kRowWaves * kk) * KT + 8 * g + 4 * b3 + 2 * b2 + b1;
      if ((j & 1) == 0 && jj < si.L) mp[jj] = tot;
    }
  }
}

template <int D, int MAXT, bool MASS>
__global__ __launch_bounds__(512) void attn_rows_kernel(AttnArgs a, AttnPlan p) {
  __shared__ RowsLds<D> lds;
  attn_rows_body<D, MAXT, MASS>(a, p, blockIdx.x, gridDim.x, lds);
}

// Mass of the row-group path: mass[b][j] = sum over heads and row groups of the
// partial sums, zero from kv_len to the stride.  A block covers 32 keys with
// 8 lanes per key: lane group g adds partials g, g + 8, g + 16, ... in order,
// then the 8 group sums are added in group order (a fixed order throughout).
// Body for 256 threads (tid = thread index in the 256, item bid).  With
// valid false the body only takes part in the barrier (a fused caller runs
// two items per 512-thread workgroup and one half may have none).
__device__ __forceinline__ void attn_rows_mass_body(const AttnArgs &a, const AttnPlan &p, int bid,
                                                    int tid, bool valid, float (*part)[32]) {
  const int per_b = (a.mass_stride + 31) / 32;
  const int b = valid ? bid / per_b : 0;
  const int k = tid & 31, grp = tid >> 5;
  const int jj = valid ? (bid % per_b) * 32 + k : a.mass_stride;
  // Partial loads are issued with the length loads (every entry read lies in
  // the workspace; entries no workgroup wrote are selected away, not added).
  const int jc = min(jj, a.mass_stride - 1);
  const float *mp = reinterpret_cast<const float *>(a.ws + p.off_mass_part) +
                    (size_t)b * a.c.H * p.rgroups * a.mass_stride + jc;
  const int n = a.c.H * p.rgroups;
  const int L = min(a.kv_len[b], a.max_kv_len);
  const int nrows = a.cu_rows[b + 1] - a.cu_rows[b];
  const int nrg = min(p.rgroups, (nrows + 15) / 16);
  float sum = 0.f;
  for (int hr0 = grp; hr0 < n; hr0 += 8 * 16) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hr = min(hr0 + 8 * i, n - 1);
      v[i] = mp[(size_t)hr * a.mass_stride];
    }
    if (nrg == p.rgroups) {  // every row group of the sequence exists: no per-entry test
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += (hr0 + 8 * i < n && jj < L) ? v[i] : 0.f;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hr = hr0 + 8 * i;
        sum += (hr < n && hr % p.rgroups < nrg && jj < L) ? v[i] : 0.f;
      }
    }
  }
  part[grp][k] = sum;
  __syncthreads();
  if (grp == 0 && jj < a.mass_stride) {
    float t = part[0][k];
#pragma unroll
    for (int g = 1; g < 8; ++g) t += part[g][k];
    a.mass[(size_t)b * a.mass_stride + jj] = t;
  }
}

__global__ __launch_bounds__(256) void attn_rows_mass_kernel(AttnArgs a, AttnPlan p) {
  __shared__ float part[8][32];
  attn_rows_mass_body(a, p, blockIdx.x, threadIdx.x, true, part);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// The externally visible launchers (left out of a unit that compiles this
// file only for its device bodies: FDL_DEVICE_ONLY).
#ifndef FDL_DEVICE_ONLY
// Row-group path only when the split path cannot fill the GPU (few
// sequences x heads) and the mass is asked for: there it saves the split
// merge and the second pass over K, which at that size cost more than the
// row groups' repeated reads of the head's keys (served from L2).
#ifndef FDL_ATTN_ROWS_MAX_GRID
#define FDL_ATTN_ROWS_MAX_GRID 256
#endif

AttnPlan plan_attention(int batch, int rows, int H, int D, int max_kv_len,
                        int max_rows_per_seq, int mass_stride) {
  AttnPlan p{};
  const int max_tiles = max(1, (max_kv_len + KT - 1) / KT);
  // Row-group path: with the mass, while each wave's scores fit in registers
  // (at most 4 tiles per wave, 1024 keys) and the grid is small.
  const bool mass = mass_stride > 0;
  const int rgroups = max(1, (max_rows_per_seq + 15) / 16);
  if (mass && max_tiles <= kRowWaves * 4 && (long)batch * H * rgroups <= FDL_ATTN_ROWS_MAX_GRID) {
    p.rows_path = 1;
    p.rgroups = rgroups;
    p.maxt = max_tiles <= kRowWaves ? 1 : max_tiles <= 2 * kRowWaves ? 2 : 4;
    if (mass) {
      p.off_mass_part = 0;
      p.bytes = align256((size_t)batch * H * p.rgroups * mass_stride * sizeof(float));
    }
    return p;
  }
  p.row_tiles = max(1, (max_rows_per_seq + 63) / 64);
  const long base = (long)batch * p.row_tiles * H;
#ifndef FDL_ATTN_UNITS
#define FDL_ATTN_UNITS 128
#endif
  int splits = (int)((FDL_ATTN_UNITS + base - 1) / max(base, 1L));
  splits = max(1, min(splits, (max_tiles + 1) / 2));
  p.splits = splits;
  if (mass_stride > 0) {
    const long mb = (long)batch * H;
    int ms = (int)((1024 + mb - 1) / max(mb, 1L));
    ms = max(ms, (max_tiles + 31) / 32);  // at most 32 tiles per chunk (LDS accumulator)
    p.mass_splits = max(1, min(ms, max_tiles));
  }
  size_t off = 0;
  if (p.splits > 1) {
    p.off_part_o = off;
    off = align256(off + (size_t)p.splits * rows * H * D * sizeof(float));
    p.off_part_ml = off;
    off = align256(off + (size_t)p.splits * rows * H * 2 * sizeof(float));
  }
  if (p.mass_splits) {
    p.off_lse = off;
    off = align256(off + (size_t)rows * H * sizeof(float));
    p.off_mass_part = off;
    off = align256(off + (size_t)batch * H * mass_stride * sizeof(float));
  }
  p.bytes = off;
  return p;
}

template <int D>
hipError_t launch_rows(const AttnArgs &a, const AttnPlan &p, hipStream_t s) {
  const dim3 grid(a.batch * a.c.H * p.rgroups), block(kRowWaves * 64);
  if (!a.mass) {
    hipLaunchKernelGGL((attn_rows_kernel<D, 1, false>), grid, block, 0, s, a, p);
    return hipGetLastError();
  }
  if (p.maxt == 1)
    hipLaunchKernelGGL((attn_rows_kernel<D, 1, true>), grid, block, 0, s, a, p);
  else if (p.maxt == 2)
    hipLaunchKernelGGL((attn_rows_kernel<D, 2, true>), grid, block, 0, s, a, p);
  else
    hipLaunchKernelGGL((attn_rows_kernel<D, 4, true>), grid, block, 0, s, a, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = a.batch * ((a.mass_stride + 31) / 32);
  hipLaunchKernelGGL(attn_rows_mass_kernel, dim3(nb), dim3(256), 0, s, a, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, const AttnPlan &p, hipStream_t s) {
  if (p.rows_path) return a.c.D == 128 ? launch_rows<128>(a, p, s) : launch_rows<64>(a, p, s);
  const int units = a.batch * p.row_tiles * a.c.H * p.splits;
  if (a.c.D == 128) {
    hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(units), dim3(512), 0, s, a, p);
  } else {
    hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(units), dim3(512), 0, s, a, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits > 1 && !p.mass_splits) {
    const size_t threads = (size_t)a.rows * a.c.H * (a.c.D / 4);
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (blocks) {
      if (a.c.D == 128)
        hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(blocks), dim3(256), 0, s, a, p);
      else
        hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(blocks), dim3(256), 0, s, a, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (p.mass_splits) {
    const int mu = a.batch * a.c.H * p.mass_splits;
    if (a.c.D == 128)
      hipLaunchKernelGGL(attn_mass_kernel<128>, dim3(mu), dim3(256), 0, s, a, p);
    else
      hipLaunchKernelGGL(attn_mass_kernel<64>, dim3(mu), dim3(256), 0, s, a, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int nb_mass = a.batch * ((a.mass_stride + 255) / 256);
    const size_t mthreads = p.splits > 1 ? (size_t)a.rows * a.c.H * (a.c.D / 4) : 0;
    const int nb = nb_mass + (int)((mthreads + 255) / 256);
    if (a.c.D == 128)
      hipLaunchKernelGGL(attn_finish_kernel<128>, dim3(nb), dim3(256), 0, s, a, p, nb_mass);
    else
      hipLaunchKernelGGL(attn_finish_kernel<64>, dim3(nb), dim3(256), 0, s, a, p, nb_mass);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

#endif  // FDL_DEVICE_ONLY

}  // namespace fdl
