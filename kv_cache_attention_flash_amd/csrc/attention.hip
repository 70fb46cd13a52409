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

constexpr int KT = 32;   // keys per tile
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

// The same step handing back, instead of the scaled scores, the fp32
// probabilities pv[e] = exp2(x - mt) of the tile's keys and the maximum mt they
// are taken against (the row's running maximum after this tile; 0 while the
// row has seen nothing, when every pv is 0).  exp2(x - LSE) = pv * exp2(mt -
// LSE): one exponential per row and tile forms the mass once the LSE is known.
template <int NO>
__device__ __forceinline__ u32x4 tile_softmax_pv(const f32x4 s[2], const Vis &vis, int tv,
                                                 int key0, int g, float scale, float &m, float &l,
                                                 f32x4 *o, float *pv, float &mt) {
  float xs[8];
  if (tv == 2) {
#pragma unroll
    for (int mt_ = 0; mt_ < 2; ++mt_)
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[mt_ * 4 + e] = s[mt_][e] * scale;
  } else {
#pragma unroll
    for (int mt_ = 0; mt_ < 2; ++mt_)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        xs[mt_ * 4 + e] = vis(key0 + 8 * g + 4 * mt_ + e) ? s[mt_][e] * scale : kNegInf;
  }
  float tmax = fmaxf(fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3])),
                     fmaxf(fmaxf(xs[4], xs[5]), fmaxf(xs[6], xs[7])));
  tmax = rows4_max(tmax);
  const float mnew = fmaxf(m, tmax);
  const float msafe = mnew == kNegInf ? 0.f : mnew;
  const float alpha = fast_exp2(m - msafe);
  float rs = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pv[e] = fast_exp2(xs[e] - msafe);
    rs += pv[e];
  }
  rs = rows4_sum(rs);
  l = l * alpha + rs;
  m = mnew;
  mt = msafe;
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

template <int D>
__device__ __forceinline__ void load_q(const AttnArgs &a, int r, int h, bool ok, int g,
                                       u32x4 *qf) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = ok ? ld16(a.q + ((size_t)r * a.c.H + h) * D + 32 * ks + 8 * g)
                : u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// LDS ring of the split-path kernels (attn_fwd, attn_xmass).  A tile's K and
// V go from global memory straight into LDS by buffer loads that write LDS
// (`buffer_load ... lds`): no registers, no LDS store instructions.  Lane l
// of a load fills 16-byte slot 64·piece + l of the tile, so the permuted
// layouts are made on the source side: K slot s holds chunk (s % CH) ^
// kswz(key) of key s / CH (the kslot layout), V slot s chunk (s % CH) ^
// vswz(key) (rows unpadded; the permutation keeps the transposed reads free
// of bank conflicts).  Keys at or past the cached length lie outside the
// buffer view and load as zeros.

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// The XOR term of kslot: kslot(key, ch) = key·CH + (ch ^ kswz(key)).
template <int D>
__device__ __forceinline__ int kswz(int key) {
  return D == 128 ? (key & 3) | ((key >> 1) & 12) : ((key >> 1) & 1) | ((key >> 2) & 6);
}
// V rows: 16-byte chunk c of key row k sits at chunk c ^ vswz(k).
template <int D>
__device__ __forceinline__ int vswz(int key) {
  return D == 128 ? (key & 3) << 1 : key & 2;
}

// Loads of one tile (K, and V when asked) into a ring buffer by the 4 waves
// of a key group (wq = wave within the group, wave-uniform).  The tile is
// the key run [key0, key0 + KT) of one page.
template <int D>
__device__ __forceinline__ void ring_issue(const AttnArgs &a, const int *s_page, int page0,
                                           int h, int key0, int L, u32x4 *kdst,
                                           u32x4 *vdst, bool want_v, int wq, int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int CH = D / 8, PERW = KT * CH / 64 / 4;  // 1 KB loads per wave per tile
  const int sh = a.c.bs_shift;
  const int page = __builtin_amdgcn_readfirstlane(s_page[(key0 >> sh) - page0]);
  const size_t off = ((((size_t)page * a.c.H + h) << sh) + (key0 & (a.c.bs - 1))) * D;
  // readfirstlane: a clamp may be selected as a vector instruction, and a
  // descriptor word in a vector register costs a loop around each load.
  const int bytes = __builtin_amdgcn_readfirstlane(max(0, min(KT, L - key0)) * D * 2);
  const auto rk = buffer_view(a.c.k + off, bytes);
  const auto rv = buffer_view(a.c.v + off, bytes);
#pragma unroll
  for (int i = 0; i < PERW; ++i) {
    const int piece = wq * PERW + i;
    const int s = 64 * piece + lane, key = s / CH;
    const int ko = (key * CH + ((s % CH) ^ kswz<D>(key))) * 16;
    const int vo = (key * CH + ((s % CH) ^ vswz<D>(key))) * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(kdst + 64 * piece), 16, ko, 0, 0, 0);
    if (want_v)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(vdst + 64 * piece), 16, vo, 0, 0,
                                               0);
  }
}

// S^T tile (32 keys x 16 rows) for one wave from a ring K tile: s[mt][e] is
// key 8g + 4mt + e for query row (lane & 15).
template <int D>
__device__ __forceinline__ void scores_ring(const u32x4 *ktile, const u32x4 *qf, int lane,
                                            f32x4 s[2]) {
  const lds_u32x4 *kb = (const lds_u32x4 *)ktile;
  const int g = lane >> 4, j = lane & 15;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int key = 8 * (j >> 2) + 4 * mt + (j & 3);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      u32x4 kf = kb[opaque_index(kslot<D>(key, 4 * ks + g))];
      acc = mfma16(kf, qf[ks], acc);
    }
    s[mt] = acc;
  }
}

// V^T operand from a ring V tile (as vt_operand() from a padded tile, with
// the rows' chunks permuted by vswz).
template <int D>
__device__ __forceinline__ u32x4 vt_operand_ring(const u32x4 *vtile, int dm, int lane) {
  const lds_u32x4 *vb = (const lds_u32x4 *)vtile;
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const lds_u16 *v16 = reinterpret_cast<const lds_u16 *>(vb);
  const int g = lane >> 4, i = lane & 15;
  const int c = 2 * dm + ((i >> 1) & 1), half = (i & 1) * 4;
  const int k0 = 8 * g + (i >> 2), k1 = k0 + 4;
  const int e0 = k0 * D + ((c ^ vswz<D>(k0)) << 3) + half;
  const int e1 = k1 * D + ((c ^ vswz<D>(k1)) << 3) + half;
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(v16 + opaque_index(e0)));
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(v16 + opaque_index(e1)));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// Tiles a key group holds in LDS at once.  Two keep a head-128 workgroup's LDS
// near 71 KB, so two workgroups (16 waves) share a CU; a third (one more tile
// in flight per key group) needs 103 KB and fits one workgroup per CU, which
// streams the cache more slowly.
constexpr int kRingDepth = 2;

// Pass 1.  8 waves: key group kg = wave / 4 takes the unit's even or odd
// tiles, row group wave % 4 owns 16 query rows; the two key groups keep their
// own online-softmax state and are combined through LDS at the end (group 0
// first), so two waves per SIMD hide each other's latency.
//
// MASS (one unit per (sequence, row tile, head): no KV split): the same
// workgroup then forms the attention mass of its keys, m_h[j] = sum over its
// rows of exp2(x_rj - LSE_r), in a second pass over K that starts right after
// the first and visits the tiles last-first: the keys read last are the ones
// still in the last-level cache, so the second read mostly avoids HBM.  The
// per-(sequence, head, row tile) sums go to the workspace; attn_xfinish adds
// them over heads and row tiles.
template <int D, bool MASS>
__global__ __launch_bounds__(512) void attn_fwd_kernel(AttnArgs a, AttnPlan p) {
  constexpr int T = KT * D / 8;                // 16-byte slots of a K (or V) tile
  constexpr int PERW = KT * (D / 8) / 64 / 4;  // ring loads per wave per K (or V) tile
  constexpr int NB = kRingDepth;
  static_assert(NB == 2, "two ring buffers");
  // The ring buffers of [key group][K tile | V tile] (separate objects, so
  // that reading one never waits for loads into another); ring0 has room
  // after its tiles for the merge scratch (64 rows x D floats, 64 (m, l)).
  __shared__ u32x4 ring0[4 * T + 32];
  __shared__ u32x4 ring1[4 * T];

  int u = blockIdx.x;
  const int split = u % p.splits; u /= p.splits;
  const int h = u % a.c.H; u /= a.c.H;
  const int rt = u % p.row_tiles;
  const int b = u / p.row_tiles;
  const SeqInfo si = seq_info(a, b);
  const int t0 = rt * 64;
  if (t0 >= si.nrows) return;

  // The wave index in a scalar register: the ring loads' descriptors and LDS
  // destinations are then wave-uniform to the compiler too.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = wave >> 2, wr = wave & 3;
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
  const int page0 = (tb * KT) >> a.c.bs_shift;
  const int tlast = max(te - 1, tb);
  auto ring = [&](auto b_c) -> u32x4 * {
    if constexpr (decltype(b_c)::value == 0) return &ring0[0];
    else return &ring1[0];
  };

  u32x4 qf[D / 32];
  load_q<D>(a, r, h, row_ok, g, qf);
  asm volatile("" ::: "memory");  // Q's loads ahead of the ring's (in-order load counts)

  f32x4 o[D / 16];
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) o[dm] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;

  // Key group kg takes tiles tb + kg, tb + kg + 2, ...; iteration it uses ring
  // buffer it % NB.  Iteration it waits for its tile (this wave's loads, then
  // a barrier for every wave's), refills the buffer of iteration it - 1 with
  // the tile of it + NB - 1, then does the tile's math if the tile exists.
  // Every iteration issues the same number of loads (past the key group's
  // last tile, loads of an empty view: zeros, no memory traffic), so the
  // count of loads behind a tile is fixed.
  auto issue1 = [&](auto b_c, int it) {
    u32x4 *rb = ring(b_c) + kg * 2 * T;
    const bool live = tb + kg + 2 * it < te;  // else an empty view: zeros, no traffic
    const int tile = live ? tb + kg + 2 * it : tlast;
    ring_issue<D>(a, s_page, page0, h, tile * KT, live ? si.L : 0, rb, rb + T, true, wr, lane);
  };
  if (te > tb) {
    static_for<0, NB - 1>([&](auto s_c) { issue1(s_c, decltype(s_c)::value); });
    const int niter_r = (niter + NB - 1) / NB * NB;
    for (int it0 = 0; it0 < niter_r; it0 += NB) {
      static_for<0, NB>([&](auto s_c) {
        constexpr int sb = decltype(s_c)::value;
        const int it = it0 + sb;
        ring_barrier<vm_lgkm0((NB - 2) * 2 * PERW)>();
        issue1(std::integral_constant<int, (sb + NB - 1) % NB>{}, it + NB - 1);
        asm volatile("" ::: "memory");
        const int tile = tb + kg + 2 * it;
        const bool have = it < niter && tile < te;
        const int key0 = tile * KT;
        const int tv = have ? tile_vis(vis, key0) : 0;
        if (tv != 0) {
          const u32x4 *rb = ring(s_c) + kg * 2 * T;
          f32x4 sv[2];
          scores_ring<D>(rb, qf, lane, sv);
          float xs[8];
          const u32x4 pb = tile_softmax<D / 16>(sv, vis, tv, key0, g, a.scale_log2, m, l, o, xs);
#pragma unroll
          for (int dm = 0; dm < D / 16; ++dm)
            o[dm] = mfma16(vt_operand_ring<D>(rb + T, dm, lane), pb, o[dm]);
        }
      });
    }
  }
  // Ring loads past the last tile still write LDS: complete before ring0 holds
  // the merge scratch.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // Combine the two key groups (group 1's state through LDS, reusing the tiles).
  lds_barrier();
  float *mo = reinterpret_cast<float *>(&ring0[0]);  // [4 row groups][16 rows][D]
  float *mml = mo + 64 * D;                            // [64 rows][2]
  static_assert((64 * D + 128) * 4 <= (int)sizeof(ring0), "merge scratch");
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
  if constexpr (MASS) {
    __shared__ float s_lse[64];
    __shared__ float wsum[2][2][4][KT];  // [buffer][key group][row group][key]
    if (kg == 0) {
      const float m1 = mml[2 * rl], l1 = mml[2 * rl + 1];
      const float mx = fmaxf(m, m1);
      const float f0 = m == kNegInf ? 0.f : exp2f(m - mx);
      const float f1 = m1 == kNegInf ? 0.f : exp2f(m1 - mx);
      l = l * f0 + l1 * f1;
      m = mx;
      if (row_ok) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *dst = a.out + ((size_t)r * a.c.H + h) * D + 4 * g;
#pragma unroll
        for (int dm = 0; dm < D / 16; ++dm)
          *reinterpret_cast<f32x4 *>(dst + 16 * dm) =
              (o[dm] * f0 + *reinterpret_cast<const f32x4 *>(&mo[rl * D + 16 * dm + 4 * g]) * f1) *
              inv;
      }
      if (g == 0) s_lse[rl] = row_ok && l > 0.f ? m + log2f(l) : kNegInf;
    }
    lds_barrier();
    // A row that sees no key has LSE -inf; subtracting +inf instead sends
    // every exp2 to 0.
    const float lr = s_lse[rl];
    const float lsafe = lr == kNegInf ? __builtin_huge_valf() : lr;
    float *mp = reinterpret_cast<float *>(a.ws + p.off_mass_part) +
                (((size_t)b * a.c.H + h) * p.row_tiles + rt) * a.mass_stride;
    // Pass 2: key group kg takes tiles te-1-kg, te-3-kg, ... (last first), K
    // only, through the same ring (the merge scratch is no longer read).
    const int n2 = (te - tb + 1) / 2;
    const int n2r = te > tb ? (n2 + NB - 1) / NB * NB : 0;
    auto issue2 = [&](auto b_c, int it) {
      u32x4 *rb = ring(b_c) + kg * 2 * T;
      const bool live = te - 1 - kg - 2 * it >= tb;
      const int tile = live ? te - 1 - kg - 2 * it : tb;
      ring_issue<D>(a, s_page, page0, h, tile * KT, live ? si.L : 0, rb, rb, false, wr, lane);
    };
    const int b3 = (j >> 3) & 1, b2 = (j >> 2) & 1, b1 = (j >> 1) & 1;
    // The sums of the previous iteration's tile (buffer pb_) are added over
    // the row groups after the next barrier, by 64 threads (key group
    // threadIdx.x / 32, key threadIdx.x % 32).
    auto flush = [&](int it_prev) {
      if (threadIdx.x < 2 * KT) {
        const int fk = threadIdx.x / KT, key = threadIdx.x % KT, pb_ = it_prev & 1;
        const int tile = te - 1 - fk - 2 * it_prev;
        if (it_prev < n2 && tile >= tb) {
          const float *ws4 = &wsum[0][0][0][0];
          const int w0 = opaque_index((pb_ * 2 + fk) * 4 * KT + key);
          const float v = ((ws4[w0] + ws4[w0 + KT]) + ws4[w0 + 2 * KT]) + ws4[w0 + 3 * KT];
          const int jj = tile * KT + key;
          if (jj < si.L) mp[jj] = v;
        }
      }
    };
    if (n2r > 0) static_for<0, NB - 1>([&](auto s_c) { issue2(s_c, decltype(s_c)::value); });
    for (int it0 = 0; it0 < n2r; it0 += NB) {
      static_for<0, NB>([&](auto s_c) {
        constexpr int sb = decltype(s_c)::value;
        const int it = it0 + sb;
        const int tile = te - 1 - kg - 2 * it;
        const bool have = it < n2 && tile >= tb;
        const int buf = it & 1;
        ring_barrier<vm_lgkm0((NB - 2) * PERW)>();
        if (it > 0) flush(it - 1);
        issue2(std::integral_constant<int, (sb + NB - 1) % NB>{}, it + NB - 1);
        asm volatile("" ::: "memory");
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = 0.f;
        const int key0 = tile * KT;
        const int tv = have ? tile_vis(vis, key0) : 0;
        if (tv != 0) {
          f32x4 sv[2];
          scores_ring<D>(ring(s_c) + kg * 2 * T, qf, lane, sv);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = fast_exp2(sv[mt][e] * a.scale_log2 - lsafe);
              pv[mt * 4 + e] = (tv == 2 || vis(key0 + 8 * g + 4 * mt + e)) ? x : 0.f;
            }
        }
        // Reduce over the wave's 16 rows (lanes sharing g): reduce-scatter.
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
        // Opaque index: the write stays visibly inside wsum, so it need not
        // wait for the ring loads in flight.
        if ((j & 1) == 0)
          (&wsum[0][0][0][0])[opaque_index(((buf * 2 + kg) * 4 + wr) * KT + 8 * g + 4 * b3 +
                                           2 * b2 + b1)] = tot;
      });
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();
    if (n2r > 0) flush(n2r - 1);
    return;
  }
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

// Split path with the mass: pass 1 and the mass in one launch, the scores
// kept on chip.  m[b][j] = sum_h sum_r exp2(x_rj - LSE_r) needs each row's
// final log-sum-exp, which exists only once every key has been seen.  A
// workgroup covers one KV split of kXSplitTiles tiles (1024 keys) of one
// (sequence, 64-row tile, head) group, as attn_fwd does, and keeps its scaled
// scores: kXRegTiles of a wave's tiles in registers, the rest in LDS.  When a
// sequence's cache fits one split the workgroup has the LSE at the end of its
// pass.  Otherwise the splits of the group exchange their row maxima and
// normalisers: each publishes its (m, l) with device-coherent stores, waits
// for its own stores to complete, counts itself in, and waits until all S_b
// splits are in; each then forms the same LSE from the S_b pairs in split
// order.  The keys are read once.  The unnormalised split outputs go to the
// workspace and attn_xfinish merges them in split order.
// Workgroups take their units from a ticket counter (cleared by
// attn_xclear_kernel before the launch), so every unit with a lower ticket is
// held by a running workgroup: a wait is only ever for a workgroup that is
// running and does not wait for it.  Every wait is bounded; past the bound
// the error word is set and the results of the call are invalid.
constexpr int kXSplitTiles = 32;  // tiles (of KT keys) per split: 1024 keys
constexpr int kXWaveTiles = kXSplitTiles / 2;
constexpr int kXRegTiles = 13;    // of a wave's tiles, the scores held in registers
constexpr int kXRingDepth = 3;    // ring buffers (tiles a key group holds in LDS)
constexpr int kXLdsTiles = kXWaveTiles - kXRegTiles;
constexpr int kXSpinLimit = 1 << 16;  // polls: ~0.1 s, far beyond any pass
constexpr int kXSyncHead = 4;     // ticket, error word, 2 spare; then one count per group

// Completes this thread's outstanding memory operations (stores included:
// on this architecture the vector memory counter covers both), with no
// compiler motion of memory accesses across it.
__device__ __forceinline__ void wait_mem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); lgkmcnt, expcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void attn_xclear_kernel(int *sync, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    if (i != 1) sync[i] = 0;  // the error word stays as it is
}

template <int D, bool LOOP>
__global__ __launch_bounds__(512) void attn_xmass_kernel(AttnArgs a, AttnPlan p) {
  constexpr int T = KT * D / 8;                // 16-byte slots of a K (or V) tile
  constexpr int PERW = KT * (D / 8) / 64 / 4;  // ring loads per wave per K (or V) tile
  constexpr int NB = kXRingDepth;
  // NB ring buffers of [key group][K tile | V tile], as in attn_fwd.  Tile
  // iteration it of a key group uses buffer (it + 1) % NB, so that ring0 is
  // free after a unit's pass: it then holds the key-group merge and the mass
  // sums while ring1 and ring2 take the next unit's first tiles.
  __shared__ u32x4 ring0[4 * T + 32];
  __shared__ u32x4 ring1[4 * T];
  __shared__ u32x4 ring2[4 * T];
  static_assert(NB == 3, "three ring buffers");
  __shared__ float sc_lds[8][kXLdsTiles][8][64];  // [wave][tile][element][lane]
  __shared__ float s_tmax[2][kXWaveTiles][64];     // [key group][tile][row]
  constexpr int kSplitPages = kXSplitTiles * KT / 32;  // block size >= 32
  __shared__ int s_page[kSplitPages];
  __shared__ float s_lse[64];
  __shared__ int s_unit;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = wave >> 2, wr = wave & 3;
  const int g = lane >> 4, j = lane & 15;
  const int rl = wr * 16 + j;  // row of the lane inside the tile
  const int S = p.splits;
  int *sync = reinterpret_cast<int *>(a.ws + p.off_sync);
  auto ring = [&](auto b_c) -> u32x4 * {
    if constexpr (decltype(b_c)::value == 0) return &ring0[0];
    else if constexpr (decltype(b_c)::value == 1) return &ring1[0];
    else return &ring2[0];
  };

  // LOOP (every cache fits one split: no unit waits for another): a grid of
  // at most one workgroup per CU walks the units u = blockIdx.x, + gridDim.x,
  // ..., skipping empty row tiles, and starts each next unit's pages, Q and
  // first two tiles while it finishes the current one.  Otherwise one unit
  // per workgroup, taken from the ticket counter when the splits exchange.
  const int units = a.batch * p.row_tiles * a.c.H * S;
  // LOOP: the units in order of decreasing cache length (sequences ranked in
  // LDS, ties by index; a batch above kXRankMax keeps index order), dealt to
  // the workgroups in snake order (round k: workgroup w takes position
  // k G + w for even k, k G + G - 1 - w for odd k), so that every workgroup's
  // total is close to the mean.
  constexpr int kXRankMax = 128;
  __shared__ int s_order[kXRankMax];
  const bool ranked = LOOP && a.batch <= kXRankMax;
  if (ranked) {
    if ((int)threadIdx.x < a.batch) {
      const int L = min(a.kv_len[threadIdx.x], a.max_kv_len);
      int rank = 0;
      for (int i = 0; i < a.batch; ++i) {
        const int Li = min(a.kv_len[i], a.max_kv_len);
        rank += (Li > L || (Li == L && i < (int)threadIdx.x)) ? 1 : 0;
      }
      s_order[rank] = threadIdx.x;
    }
    __syncthreads();
  }
  const int per_seq = p.row_tiles * a.c.H;  // units of a sequence (LOOP: one split)
  auto unit_at = [&](int k) -> int {        // k-th position of this workgroup, or units
    const int G = gridDim.x;
    const int pos = k * G + ((k & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
    if (pos >= units) return units;
    const int rb = pos / per_seq;
    return (ranked ? s_order[rb] : rb) * per_seq + pos % per_seq;
  };
  auto live_k = [&](int k) -> int {  // first position at or after k whose row tile has rows
    for (;; ++k) {
      const int v = unit_at(k);
      if (v >= units) return k;
      const int b = v / per_seq, rt = v / a.c.H % p.row_tiles;
      if (rt * 64 < a.cu_rows[b + 1] - a.cu_rows[b]) return k;
    }
  };
  int u, kpos = 0;
  if constexpr (LOOP) {
    // (unit numbers in scalar registers: the per-unit loads are then scalar
    // loads, which do not wait behind the next unit's tiles in flight)
    kpos = __builtin_amdgcn_readfirstlane(live_k(0));
    u = __builtin_amdgcn_readfirstlane(unit_at(kpos));
  } else {
    if (S > 1) {
      if (threadIdx.x == 0)
        s_unit = __hip_atomic_fetch_add(sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
    } else if (threadIdx.x == 0) {
      s_unit = blockIdx.x;  // no waits: the launch order is enough
    }
    __syncthreads();
    u = s_unit;
  }
  bool pref = false;  // this unit's pages, Q and first two tiles are on their way
  u32x4 qf[D / 32];
  int next_page = 0;  // LOOP: this thread's block-table entry of the next unit
  // LOOP: the next unit's sequence, read before its tiles were issued (a
  // vector load at the loop top would wait behind those tiles)
  SeqInfo nsi{};

  while (!LOOP || u < units) {
    const int split = u % S;
    const int grp = u / S;  // (sequence, row tile, head)
    const int h = grp % a.c.H;
    const int rt = grp / a.c.H % p.row_tiles;
    const int b = grp / a.c.H / p.row_tiles;
    const SeqInfo si = pref ? nsi : seq_info(a, b);
    const int t0 = rt * 64;
    const int tiles = (si.L + KT - 1) / KT;
    const int Sb = max(1, (tiles + kXSplitTiles - 1) / kXSplitTiles);
    if (!LOOP && (t0 >= si.nrows || split >= Sb)) return;

    const int t = t0 + wr * 16 + j;  // local row of this lane
    const bool row_ok = t < si.nrows;
    const int r = si.r0 + (row_ok ? t : 0);
    const Vis vis = row_vis(si, t, row_ok);

    const int tb = split * kXSplitTiles, te = min(tiles, tb + kXSplitTiles);
    const int niter = (te - tb + 1) / 2;  // iterations per key group
    const int tlast = max(te - 1, tb);
    const int page0 = (tb * KT) >> a.c.bs_shift;
    auto issue = [&](auto b_c, int it) {
      u32x4 *rb = ring(b_c) + kg * 2 * T;
      const bool live = tb + kg + 2 * it < te;
      const int tile = live ? tb + kg + 2 * it : tlast;
      ring_issue<D>(a, s_page, page0, h, tile * KT, live ? si.L : 0, rb, rb + T, true, wr, lane);
    };
    if (!pref) {
      stage_pages(a, b, tb, te, s_page);
      lds_barrier();
      load_q<D>(a, r, h, row_ok, g, qf);
      if (te > tb) {
        asm volatile("" ::: "memory");  // Q's loads ahead of the ring's
        static_for<0, NB - 1>([&](auto c_) {
          issue(std::integral_constant<int, decltype(c_)::value + 1>{}, decltype(c_)::value);
        });
      }
    }

    f32x4 o[D / 16];
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) o[dm] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, l = 0.f;
    // fp32 probabilities of the wave's tiles, each against its tile's running
    // maximum (kept in s_tmax)
    float sc[kXRegTiles][8];

    // The wave's tiles, unrolled so that every probability lands in a fixed
    // register (or LDS slot) and every ring buffer index is a constant.  An
    // empty cache (no tile, no staged page) issues no load at all.
    if (te > tb) {
      static_for<0, kXWaveTiles>([&](auto it_c) {
        constexpr int it = decltype(it_c)::value;
        // Past the split's last iteration (the same for the whole workgroup)
        // there is nothing to wait for or compute; the loads already issued
        // for those iterations are drained after the loop.
        if (it >= niter) return;
        const int tile = tb + kg + 2 * it;
        const bool have = tile < te;
        ring_barrier<vm_lgkm0((NB - 2) * 2 * PERW)>();
        issue(std::integral_constant<int, (it + NB) % NB>{}, it + NB - 1);
        asm volatile("" ::: "memory");
        const u32x4 *rb = ring(std::integral_constant<int, (it + 1) % NB>{}) + kg * 2 * T;
        const int key0 = tile * KT;
        const int tv = have ? tile_vis(vis, key0) : 0;
        float pv[8], mt = 0.f;
        if (tv != 0) {
          f32x4 sv[2];
          scores_ring<D>(rb, qf, lane, sv);
          const u32x4 pb =
              tile_softmax_pv<D / 16>(sv, vis, tv, key0, g, a.scale_log2, m, l, o, pv, mt);
#pragma unroll
          for (int dm = 0; dm < D / 16; ++dm)
            o[dm] = mfma16(vt_operand_ring<D>(rb + T, dm, lane), pb, o[dm]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = 0.f;
        }
        if (g == 0) s_tmax[kg][it][rl] = mt;
        if constexpr (it < kXRegTiles) {
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[it][e] = pv[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) sc_lds[wave][it - kXRegTiles][e][lane] = pv[e];
        }
      });
    }
    // Ring loads past the last tile still write LDS: complete before ring0
    // holds the merge (and before ring1 / ring2 take the next unit's tiles).
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // LOOP: the next unit, and its block-table entries on their way (written
    // to s_page once this unit's outputs are out; the pass no longer reads it).
    int nu = units, nb_ = 0, nh = 0, nrt = 0;
    int nte = 0;
    if constexpr (LOOP) {
      kpos = __builtin_amdgcn_readfirstlane(live_k(kpos + 1));
      nu = __builtin_amdgcn_readfirstlane(unit_at(kpos));
      if (nu < units) {
        nh = nu / S % a.c.H;
        nrt = nu / S / a.c.H % p.row_tiles;
        nb_ = nu / S / a.c.H / p.row_tiles;
        nsi = seq_info(a, nb_);
        nte = min((nsi.L + KT - 1) / KT, kXSplitTiles);
        const int np = nte > 0 ? ((nte * KT - 1) >> a.c.bs_shift) + 1 : 0;
        if ((int)threadIdx.x < np)
          next_page = a.c.block_table[(size_t)nb_ * a.c.max_blocks + threadIdx.x];
      }
    }

    // Combine the two key groups: group 1's state through LDS (reusing the
    // tiles), the maxima and normalisers first so that they can be published
    // before the outputs are merged.
    lds_barrier();
    float *mo = reinterpret_cast<float *>(&ring0[0]);  // [64 rows][D]
    float *mml = mo + 64 * D;                            // [64 rows][2]
    static_assert((64 * D + 128) * 4 <= (int)sizeof(ring0), "merge scratch");
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
    float f0 = 0.f, f1 = 0.f;
    if (kg == 0) {
      const float m1 = mml[2 * rl], l1 = mml[2 * rl + 1];
      const float mx = fmaxf(m, m1);
      f0 = m == kNegInf ? 0.f : exp2f(m - mx);
      f1 = m1 == kNegInf ? 0.f : exp2f(m1 - mx);
      l = l * f0 + l1 * f1;
      m = mx;
    }
    float *po = reinterpret_cast<float *>(a.ws + p.off_part_o);
    float *pml = reinterpret_cast<float *>(a.ws + p.off_part_ml);
    const size_t stride = (size_t)a.rows * a.c.H;
    const size_t rh0 = (size_t)r * a.c.H + h;
    int *count = sync + kXSyncHead + grp;
    if (!LOOP && Sb > 1) {
      // Publish this split's (m, l) with device-coherent stores, complete them,
      // then count the split in.
      if (kg == 0 && row_ok && g == 0) {
        store_agent(&pml[2 * (split * stride + rh0)], m);
        store_agent(&pml[2 * (split * stride + rh0) + 1], l);
      }
      wait_mem();
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // The outputs, while the other splits arrive: the final (normalised) rows
    // when the cache fits one split, else this split's unnormalised partial.
    if (kg == 0 && row_ok) {
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm)
        o[dm] = o[dm] * f0 + *reinterpret_cast<const f32x4 *>(&mo[rl * D + 16 * dm + 4 * g]) * f1;
      if (Sb == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *dst = a.out + rh0 * D + 4 * g;
#pragma unroll
        for (int dm = 0; dm < D / 16; ++dm)
          *reinterpret_cast<f32x4 *>(dst + 16 * dm) = o[dm] * inv;
      } else {
        float *dst = po + (split * stride + rh0) * D + 4 * g;
#pragma unroll
        for (int dm = 0; dm < D / 16; ++dm) *reinterpret_cast<f32x4 *>(dst + 16 * dm) = o[dm];
      }
    }

    // The row's log-sum-exp over the whole cache.
    float lse = kNegInf;
    if (LOOP || Sb == 1) {
      if (kg == 0 && row_ok) lse = l > 0.f ? m + log2f(l) : kNegInf;
    } else {
      if (threadIdx.x == 0) {
        int spins = 0;
        while (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < Sb) {
          if (++spins > kXSpinLimit) {
            __hip_atomic_store(sync + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      __syncthreads();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (kg == 0 && row_ok) {
        // Eight splits' pairs at a time, all loads in flight together; the
        // chunks are combined in split order.
        float mx = kNegInf, lsum = 0.f;
        for (int s0 = 0; s0 < Sb; s0 += 8) {
          float mv[8], lv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const size_t k = (size_t)min(s0 + i, Sb - 1) * stride + rh0;
            mv[i] = load_agent(&pml[2 * k]);
            lv[i] = load_agent(&pml[2 * k + 1]);
          }
          float cm = kNegInf;
#pragma unroll
          for (int i = 0; i < 8; ++i) cm = s0 + i < Sb ? fmaxf(cm, mv[i]) : cm;
          const float nm = fmaxf(mx, cm);
          if (nm != kNegInf) {
            float cs = mx == kNegInf ? 0.f : lsum * exp2f(mx - nm);
#pragma unroll
            for (int i = 0; i < 8; ++i)
              cs += (s0 + i < Sb && mv[i] != kNegInf) ? lv[i] * exp2f(mv[i] - nm) : 0.f;
            lsum = cs;
          }
          mx = nm;
        }
        lse = lsum > 0.f ? mx + log2f(lsum) : kNegInf;
      }
    }
    if (kg == 0 && g == 0) s_lse[rl] = lse;
    if constexpr (LOOP) {
      if (nu < units && (int)threadIdx.x < kSplitPages) s_page[threadIdx.x] = next_page;
    }
    lds_barrier();
    const float lr = s_lse[rl];

    if constexpr (LOOP) {
      // The next unit's Q and first two tiles (into ring1 and ring2) go out
      // now and arrive while this unit's mass is formed.
      if (nu < units) {
        const int nt = nrt * 64 + wr * 16 + j;
        const bool nrow_ok = nt < nsi.nrows;
        load_q<D>(a, nsi.r0 + (nrow_ok ? nt : 0), nh, nrow_ok, g, qf);
        if (nte > 0) {
          asm volatile("" ::: "memory");
          const int ntlast = nte - 1;
          static_for<0, NB - 1>([&](auto c_) {
            constexpr int it = decltype(c_)::value;
            u32x4 *rb = ring(std::integral_constant<int, it + 1>{}) + kg * 2 * T;
            const bool live = kg + 2 * it < nte;
            const int tile = live ? kg + 2 * it : ntlast;
            ring_issue<D>(a, s_page, 0, nh, tile * KT, live ? nsi.L : 0, rb, rb + T, true, wr,
                          lane);
          });
        }
      }
    }

    // Mass of the wave's keys over its 16 rows: each probability rescaled by
    // its tile's factor exp2(mt - LSE), a reduce-scatter over the row lanes,
    // then the 4 row groups added in order through LDS.
    float *wsum = reinterpret_cast<float *>(&ring0[0]);  // [4 row groups][kXSplitTiles * KT]
    static_assert(4 * kXSplitTiles * KT * 4 <= (int)sizeof(ring0), "mass scratch");
    const int b3 = (j >> 3) & 1, b2 = (j >> 2) & 1, b1 = (j >> 1) & 1;
#pragma unroll
    for (int it = 0; it < kXWaveTiles; ++it) {
      const int tile = tb + kg + 2 * it;
      if (it < niter && tile < te) {
        const float f = lr == kNegInf ? 0.f : fast_exp2(s_tmax[kg][it][rl] - lr);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = it < kXRegTiles
                              ? sc[it < kXRegTiles ? it : 0][e]
                              : sc_lds[wave][it < kXRegTiles ? 0 : it - kXRegTiles][e][lane];
          pv[e] = x * f;
        }
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
        if ((j & 1) == 0)
          wsum[wr * (kXSplitTiles * KT) + (tile - tb) * KT + 8 * g + 4 * b3 + 2 * b2 + b1] = tot;
      }
    }
    // The LDS sums complete and visible; no wait for the next unit's tiles in
    // flight (a fence would wait for those loads into LDS too).
    ring_barrier<vm_lgkm0(63)>();
    float *mp = reinterpret_cast<float *>(a.ws + p.off_mass_part) +
                (((size_t)b * a.c.H + h) * p.row_tiles + rt) * a.mass_stride;
    const int nk = (te - tb) * KT;
    for (int k = threadIdx.x; k < nk; k += blockDim.x) {
      const int jj = tb * KT + k;
      constexpr int W = kXSplitTiles * KT;
      const float v = ((wsum[k] + wsum[W + k]) + wsum[2 * W + k]) + wsum[3 * W + k];
      if (jj < si.L) mp[jj] = v;
    }
    if constexpr (!LOOP) return;
    u = nu;
    pref = true;
  }
}

// Sequence of row r: the largest b with cu_rows[b] <= r.
__device__ __forceinline__ int attn_row_seq(const int32_t *cu_rows, int batch, int r) {
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_rows[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// Last launch of the split path with the mass: blocks [0, nb_mass) form
// mass[b][j], the per-(head, row tile) partials added in head, then row-tile
// order (zero from kv_len to the stride); the blocks after that merge the
// split outputs of rows whose sequence took more than one split, in split
// order (one thread per row, head and 4 features).
template <int D>
__global__ __launch_bounds__(256) void attn_xfinish_kernel(AttnArgs a, AttnPlan p, int nb_mass) {
  if ((int)blockIdx.x >= nb_mass) {
    const size_t idx = (size_t)(blockIdx.x - nb_mass) * blockDim.x + threadIdx.x;
    const size_t rh = idx / (D / 4);
    const int d4 = (int)(idx % (D / 4)) * 4;
    if (rh >= (size_t)active_rows(a) * a.c.H) return;
    const int r = (int)(rh / a.c.H);
    const int b = attn_row_seq(a.cu_rows, a.batch, r);
    const int L = min(a.kv_len[b], a.max_kv_len);
    const int Sb = max(1, ((L + KT - 1) / KT + kXSplitTiles - 1) / kXSplitTiles);
    if (Sb == 1) return;  // written by the pass itself
    const float *po = reinterpret_cast<const float *>(a.ws + p.off_part_o);
    const float *pml = reinterpret_cast<const float *>(a.ws + p.off_part_ml);
    const size_t stride = (size_t)a.rows * a.c.H;
    float mx = kNegInf;
    for (int s = 0; s < Sb; ++s) mx = fmaxf(mx, pml[2 * (s * stride + rh)]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    if (mx != kNegInf) {
      for (int s = 0; s < Sb; ++s) {
        const size_t k = s * stride + rh;
        const float ms = pml[2 * k];
        const float f = ms == kNegInf ? 0.f : exp2f(ms - mx);
        lsum += pml[2 * k + 1] * f;
        acc += *reinterpret_cast<const f32x4 *>(po + k * D + d4) * f;
      }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    *reinterpret_cast<f32x4 *>(a.out + rh * D + d4) = acc * inv;
    return;
  }
  const int per_b = (a.mass_stride + 255) / 256;
  const int b = blockIdx.x / per_b;
  const int jj = (blockIdx.x % per_b) * blockDim.x + threadIdx.x;
  if (jj >= a.mass_stride) return;
  const int L = min(a.kv_len[b], a.max_kv_len);
  const int nrt = min(p.row_tiles, (a.cu_rows[b + 1] - a.cu_rows[b] + 63) / 64);
  float sum = 0.f;
  if (jj < L) {
    const float *mp = reinterpret_cast<const float *>(a.ws + p.off_mass_part) +
                      (size_t)b * a.c.H * p.row_tiles * a.mass_stride + jj;
    for (int h0 = 0; h0 < a.c.H; h0 += 32) {
      float v[32];
      if (nrt == 1) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
          v[i] = h0 + i < a.c.H ? mp[(size_t)(h0 + i) * p.row_tiles * a.mass_stride] : 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) sum += v[i];
      } else {
        for (int i = 0; i < 32 && h0 + i < a.c.H; ++i)
          for (int q = 0; q < nrt; ++q)
            sum += mp[((size_t)(h0 + i) * p.row_tiles + q) * a.mass_stride];
      }
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
  u32x4 kbuf[kRowWaves][KT * D / 8];
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
    u32x4 *kb = L.kbuf[w];
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      const int c = lane + 64 * i;
      kb[kslot<D>(c / CH, c % CH)] = st.k[i];
    }
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int key = 8 * (j >> 2) + 4 * mt + (j & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16(kb[kslot<D>(key, 4 * ks + g)], qf[ks], acc);
      s[mt] = acc;
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int c = lane + 64 * i;
      const int key = c / CH;
      st16(&vb[key][(c % CH) * 8], st.v[i]);  // zeros past the length
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
constexpr long kRowsMaxGrid = 256;
// Split path with the mass: (sequence, row tile, head) units from which one
// workgroup per unit (attn_fwd_kernel<D, true>) fills the GPU.
constexpr long kFwdMassMinUnits = 256;

AttnPlan plan_attention(int batch, int rows, int H, int D, int max_kv_len,
                        int max_rows_per_seq, int mass_stride) {
  AttnPlan p{};
  const int max_tiles = max(1, (max_kv_len + KT - 1) / KT);
  // Row-group path: with the mass, while each wave's scores fit in registers
  // (at most 4 tiles per wave, 1024 keys) and the grid is small.
  const bool mass = mass_stride > 0;
  const int rgroups = max(1, (max_rows_per_seq + 15) / 16);
  if (mass && max_tiles <= kRowWaves * 4 && (long)batch * H * rgroups <= kRowsMaxGrid) {
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
  size_t off = 0;
  if (mass) {
    p.xmass = 1;
    const long units = (long)batch * p.row_tiles * H;
    if (max_tiles > kXSplitTiles && units >= kFwdMassMinUnits) {
      // Long caches and enough units to fill the GPU: one workgroup per
      // unit, the mass as a second pass over K right after the first
      // (attn_fwd_kernel<D, true>).
      p.fwd_mass = 1;
      p.splits = 1;
      p.off_mass_part = 0;
      p.bytes = align256((size_t)batch * H * p.row_tiles * mass_stride * sizeof(float));
      return p;
    }
    // Otherwise pass 1 and the mass in one launch with the scores on chip
    // (attn_xmass): one split per 1024 keys, the splits of a long cache
    // exchanging their row statistics.
    p.splits = (max_tiles + kXSplitTiles - 1) / kXSplitTiles;
    if (p.splits > 1) {
      p.off_sync = 0;  // first, so the error word sits at byte 4 of the workspace
      p.sync_ints = kXSyncHead + batch * p.row_tiles * H;
      off = align256((size_t)p.sync_ints * sizeof(int));
      p.off_part_o = off;
      off = align256(off + (size_t)p.splits * rows * H * D * sizeof(float));
      p.off_part_ml = off;
      off = align256(off + (size_t)p.splits * rows * H * 2 * sizeof(float));
    }
    p.off_mass_part = off;
    off = align256(off + (size_t)batch * H * p.row_tiles * mass_stride * sizeof(float));
    p.bytes = off;
    return p;
  }
  const long base = (long)batch * p.row_tiles * H;
  constexpr long kUnits = 128;  // target (sequence, row tile, head, split) units
  int splits = (int)((kUnits + base - 1) / max(base, 1L));
  splits = max(1, min(splits, (max_tiles + 1) / 2));
  p.splits = splits;
  if (p.splits > 1) {
    p.off_part_o = off;
    off = align256(off + (size_t)p.splits * rows * H * D * sizeof(float));
    p.off_part_ml = off;
    off = align256(off + (size_t)p.splits * rows * H * 2 * sizeof(float));
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

template <int D>
hipError_t launch_xmass(const AttnArgs &a, const AttnPlan &p, hipStream_t s) {
  if (p.fwd_mass) {
    const int units = a.batch * p.row_tiles * a.c.H;
    hipLaunchKernelGGL((attn_fwd_kernel<D, true>), dim3(units), dim3(512), 0, s, a, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nb_mass = a.batch * ((a.mass_stride + 255) / 256);
    hipLaunchKernelGGL(attn_xfinish_kernel<D>, dim3(nb_mass), dim3(256), 0, s, a, p, nb_mass);
    return hipGetLastError();
  }
  if (p.splits > 1) {
    int *sync = reinterpret_cast<int *>(a.ws + p.off_sync);
    hipLaunchKernelGGL(attn_xclear_kernel, dim3((p.sync_ints + 255) / 256), dim3(256), 0, s, sync,
                       p.sync_ints);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int units = a.batch * p.row_tiles * a.c.H * p.splits;
  if (p.splits == 1)  // no unit waits for another: at most one workgroup per CU, looping
    hipLaunchKernelGGL((attn_xmass_kernel<D, true>), dim3(std::min(units, device_cus())),
                       dim3(512), 0, s, a, p);
  else
    hipLaunchKernelGGL((attn_xmass_kernel<D, false>), dim3(units), dim3(512), 0, s, a, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb_mass = a.batch * ((a.mass_stride + 255) / 256);
  const size_t mthreads = p.splits > 1 ? (size_t)a.rows * a.c.H * (D / 4) : 0;
  const int nb = nb_mass + (int)((mthreads + 255) / 256);
  hipLaunchKernelGGL(attn_xfinish_kernel<D>, dim3(nb), dim3(256), 0, s, a, p, nb_mass);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, const AttnPlan &p, hipStream_t s) {
  if (p.rows_path) return a.c.D == 128 ? launch_rows<128>(a, p, s) : launch_rows<64>(a, p, s);
  if (p.xmass) return a.c.D == 128 ? launch_xmass<128>(a, p, s) : launch_xmass<64>(a, p, s);
  const int units = a.batch * p.row_tiles * a.c.H * p.splits;
  if (a.c.D == 128) {
    hipLaunchKernelGGL((attn_fwd_kernel<128, false>), dim3(units), dim3(512), 0, s, a, p);
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<64, false>), dim3(units), dim3(512), 0, s, a, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits > 1) {
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
  return hipSuccess;
}

#endif  // FDL_DEVICE_ONLY

}  // namespace fdl
