// Flash-Cache for gfx950: QKV projection of the active rows, rotary embedding,
// bf16 rounding and the paged KV-cache write, fused in one launch.
//
// Source: [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for Fast,
// Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary), para 1: the
// projection, the rotary embedding and the cache write are one kernel whose K/V
// come out of on-chip memory straight into the cache; para 2: only the window
// and the tracked rows are active.
//
// Work decomposition.  Output features are grouped in rotary PAIRS (i, i + D/2)
// of one head of one of Q, K, V, so a pair's two outputs always land in the
// same workgroup and the rotation needs no extra memory traffic.  Two kernels:
//   qkv_splitk_kernel  up to 64 active rows (the decode regime, where reading
//                      the weight dominates): each workgroup streams a slice
//                      of the weight once, staged through LDS in whole lines;
//   qkv_gemm_kernel    more rows: a 2-D tiled MFMA GEMM (32x32x16 bf16).
// Both finish in an fp32 epilogue: rotation with an fp64-reduced angle, bf16
// rounding (RNE), Q to its buffer and K/V scattered through the block table.
// Partial sums are always added in a fixed order, so results are bitwise
// reproducible.
#include "device_common.h"
#include "internal.h"

namespace fdl {

namespace {

constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

// Largest b with cu_rows[b] <= r (empty sequences are skipped over).
__device__ __forceinline__ int row_to_seq(const int32_t *cu_rows, int batch, int r) {
  int lo = 0, hi = batch;  // invariant: cu_rows[lo] <= r < cu_rows[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu_rows[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// Rows at or past cu_rows[batch] are inactive (num_rows is then a capacity):
// nothing is written for them.
__device__ __forceinline__ int active_rows(const FlashCacheArgs &a) {
  return max(0, min(a.rows, a.cu_rows[a.batch]));
}

// Rotary frequency base^(-2i/D), in turns (revolutions) per position, fp64.
__device__ __forceinline__ double rope_inv_freq(int i, int D, double log2_base) {
  return exp2(-(2.0 * (double)i / (double)D) * log2_base) * kInvTwoPi;
}

// cos/sin of the angle position * frequency: the angle in turns and its
// reduction to [-1/2, 1/2] in fp64, then the hardware sine and cosine
// (v_sin_f32 / v_cos_f32 take turns; absolute error far below the bf16
// rounding that follows).
__device__ __forceinline__ void rope_cs(int pos, double turns_per_pos, float &c, float &s) {
  double t = (double)pos * turns_per_pos;
  t -= rint(t);
  s = __builtin_amdgcn_sinf((float)t);
  c = __builtin_amdgcn_cosf((float)t);
}

// Rotation of one pair by the angle with cosine c and sine s (Q and K
// sections only) and bf16 rounding.
__device__ __forceinline__ uint32_t rotate_round_cs(float lo, float hi, bool rotate, float c,
                                                    float s) {
  if (rotate) {
    const float rlo = __builtin_fmaf(lo, c, -(hi * s));
    const float rhi = __builtin_fmaf(hi, c, lo * s);
    lo = rlo;
    hi = rhi;
  }
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// The same with the angle formed here; one helper for every epilogue and the
// unfused rotary kernel, so all of them round identically.
__device__ __forceinline__ uint32_t rotate_round(float lo, float hi, int sec, int pos,
                                                 double turns_per_pos) {
  float c = 1.f, s = 0.f;
  if (sec < 2) rope_cs(pos, turns_per_pos, c, s);
  return rotate_round_cs(lo, hi, sec < 2, c, s);
}

// The raw fp32 pair of row r, rotary pair p (the unfused ablation's output).
__device__ __forceinline__ void store_raw_pair(const FlashCacheArgs &a, int r, int p, float lo,
                                               float hi) {
  const int H = a.c.H, D = a.c.D, half = D >> 1;
  float *y = a.y_out + (size_t)r * 3 * H * D + (size_t)(p / half) * D + p % half;
  y[0] = lo;
  y[half] = hi;
}

// Where element i of rotary pair p (i, i + D/2) of row r goes: Q to its
// buffer, K and V into the cache (physical block blk, offset off).
__device__ __forceinline__ uint16_t *pair_dst(const FlashCacheArgs &a, int r, int p, int blk,
                                              int off) {
  const int H = a.c.H, D = a.c.D, half = D >> 1;
  const int sh = p / half;  // section * H + head
  const int i = p % half;
  const int sec = sh / H;
  const int h = sh % H;
  if (sec == 0) return a.q_out + ((size_t)r * H + h) * D + i;
  uint16_t *pool = sec == 1 ? a.c.k : a.c.v;
  return pool + (((size_t)blk * H + h) * a.c.bs + off) * D + i;
}

// Stores the rounded pair word v (low half: element i, high half: i + D/2).
__device__ __forceinline__ void store_word(uint16_t *dst, int half, uint32_t v) {
  dst[0] = (uint16_t)(v & 0xffffu);
  dst[half] = (uint16_t)(v >> 16);
}

// Rotate (Q and K parts), round and store one rotary pair of one row; with
// y_out set, store the raw fp32 pair instead (the unfused ablation).
__device__ __forceinline__ void store_pair(const FlashCacheArgs &a, int r, int p, float lo,
                                           float hi, int blk, int off, int pos,
                                           double inv_freq_i) {
  if (a.y_out) {
    store_raw_pair(a, r, p, lo, hi);
    return;
  }
  const int sec = p / (a.c.D >> 1) / a.c.H;
  store_word(pair_dst(a, r, p, blk, off), a.c.D >> 1,
             rotate_round(lo, hi, sec, pos, inv_freq_i));
}

// Row metadata (physical block, offset, position) of row r; also writes the
// slot mapping when asked.
__device__ __forceinline__ void row_meta(const FlashCacheArgs &a, int r, bool write_map, int &blk,
                                         int &off, int &pos) {
  const int b = row_to_seq(a.cu_rows, a.batch, r);
  const int s = a.slots[r];
  blk = a.c.block_table[(size_t)b * a.c.max_blocks + s / a.c.bs];
  off = s % a.c.bs;
  pos = a.positions[r];
  if (write_map && a.slot_mapping) a.slot_mapping[r] = (int64_t)blk * a.c.bs + off;
}

// Split-K projection for up to 64 active rows (the decode regime, where the
// weight stream dominates).  Grid = G column groups x S reduction splits.  A
// workgroup owns CW = 16*NTW*NGW output features (CW/2 rotary pairs) of 64 rows
// over hidden/S reduction elements, staged through LDS in KC-element chunks:
// every global load instruction reads whole 128-byte lines (consecutive lanes
// cover consecutive 16-byte pieces of a row), and the 64 x hidden activations are read G times in
// total instead of once per 48 features.  Chunk tiles are double-buffered in
// LDS with a 16-byte-slot XOR swizzle (slot ^ row % 16) so the 16 lanes that
// read one MFMA operand hit distinct banks; two register stages keep two
// chunks of loads in flight.  8 waves: wave w owns N-tile group w % NGW and
// reduction quarter w / NGW of each chunk.
//
// With S == 1 the workgroup runs the rotary / bf16 / cache-write epilogue
// itself.  With S > 1 it stores its fp32 partial tile and qkv_reduce_kernel
// (next launch on the stream) adds the S partials in split order, so the
// result does not depend on which workgroup finishes first.  (Finishing the
// reduction inside this kernel would need device-scope release/acquire fences,
// which on a multi-XCD part write back and invalidate the L2 that the weight
// stream is using.)
// Maps a projection item's pair index to the rotary pair it computes.  The
// separate kernels use the identity (and deal their items to the XCDs
// themselves); the single-launch step, which assigns items to XCDs by head,
// passes its own map (an index past the last pair marks a pair that does not
// exist).
struct PairIdentity {
  static constexpr bool kIdentity = true;
  __device__ int operator()(int p) const { return p; }
};

struct SplitPlan {
  int G, S, ks;     // column groups, splits, reduction elements per split
  float *partials;  // [G][S][64][CW]
};

// LDS of one split-K workgroup.
template <int NTW, int NGW, int KC>
struct SplitLds {
  static constexpr int CW = 16 * NTW * NGW, ROWS = 64, PIECES = KC / 8, TROWS = ROWS + CW;
  u32x4 lds[2][TROWS * PIECES];
  int s_blk[ROWS], s_off[ROWS], s_pos[ROWS];
  double s_freq[64];
};

// The workgroup body (item bid of the grid; LDS from the caller, so a fused
// kernel can share one buffer across phases).
template <int NTW, int NGW, int NST, int NCH, int NW, int KC, class PM = PairIdentity>
__device__ __forceinline__ void qkv_splitk_body(const FlashCacheArgs &a, const SplitPlan &sp,
                                                int bid, SplitLds<NTW, NGW, KC> &L,
                                                PM pmap = PM{}) {
  constexpr int NKQ = NW / NGW;
  constexpr int CW = 16 * NTW * NGW;
  constexpr int PW = CW / 2;
  constexpr int ROWS = 64;
  constexpr int PIECES = KC / 8;            // 16-byte pieces per row per chunk (KC per chunk)
  constexpr int KSTEPS = KC / 32;           // MFMA k-steps per chunk
  constexpr int TROWS = ROWS + CW;          // staged rows per chunk
  constexpr int LOADS = TROWS * PIECES / (NW * 64);
  static_assert(TROWS * PIECES % (NW * 64) == 0, "chunk must split evenly");
  static_assert(KSTEPS % NKQ == 0, "k-steps per chunk must split over the quarters");
  auto &lds = L.lds;
  auto &s_blk = L.s_blk;
  auto &s_off = L.s_off;
  auto &s_pos = L.s_pos;
  auto &s_freq = L.s_freq;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.c.H, D = a.c.D, half = D >> 1;
  const int total_pairs = 3 * H * half;
  const int hidden = a.hidden;

  // Block -> (group, split) so that the S splits of a group run on one XCD
  // (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
  const int nb = sp.G * sp.S;
  int idx = bid;
  if (PM::kIdentity && nb % 8 == 0) idx = (bid % 8) * (nb / 8) + bid / 8;
  const int grp = idx / sp.S, split = idx % sp.S;
  const int pair0 = grp * PW;
  // A mapped group whose first pair does not exist has none to compute.
  if constexpr (!PM::kIdentity)
    if (pmap(pair0) >= total_pairs) return;
  const int k_begin = split * sp.ks;

  // Row metadata for the epilogue (S == 1), in three steps.  Every wave
  // computes it for row `lane` (identical values; wave 0 parks them in LDS),
  // so no step sits in a branch.  Step 0 (slot, position, sequence) is issued
  // before the first chunk loads and is complete once chunk 0 is; step 1 (the
  // block-table entry) goes out behind chunk 2's loads; step 2 uses it one
  // chunk later.  A wait on a load is a wait on
  // every load issued before it, so no step waits ahead of the chunk loads it
  // would hold back.
  const bool epi = sp.S == 1;
  const int mrow = max(0, min(lane, a.rows - 1));
  int act = 0, m_end = 0, m_seq = 0, m_slot = 0, m_pos = 0, m_blk = 0;
  auto meta = [&](int step) {
    if (step == 0) {  // unconditional: a value merged from two paths would be waited for here
      m_end = a.cu_rows[a.batch];  // used in step 1 (a use here would wait for it)
      m_slot = a.slots[mrow];
      m_pos = a.positions[mrow];
      m_seq = row_to_seq(a.cu_rows, a.batch, mrow);
    } else if (!epi) {
      return;
    } else if (step == 1) {
      act = max(0, min(a.rows, m_end));  // the active-row count
      // rows past the active count may hold anything: they read entry 0
      const size_t e = lane < act ? (size_t)m_seq * a.c.max_blocks + m_slot / a.c.bs : 0;
      m_blk = a.c.block_table[e];
    } else if (wave == 0 && lane < act) {
      s_blk[lane] = m_blk;
      s_off[lane] = m_slot % a.c.bs;
      s_pos[lane] = m_pos;
    }
  };
  meta(0);

  // Global rows this thread stages: row t/16 + 32*i of the chunk tile, piece t%16.
  const int piece = tid % PIECES;
  const uint16_t *src[LOADS];
  int dst_slot[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int tr = tid / PIECES + (NW * 64 / PIECES) * i;
    dst_slot[i] = tr * PIECES + (piece ^ (tr & 15));
    static_assert(PIECES >= 16, "swizzle needs 16 pieces per row");
    if (tr < ROWS) {
      const int r = min(tr, a.rows - 1);
      src[i] = a.x + (size_t)r * hidden + k_begin + piece * 8;
    } else {
      const int c = tr - ROWS;  // column in the group: tile c/16, lane col c%16
      int p = pmap(pair0 + 8 * (c / 16) + (c & 7));
      p = p < total_pairs ? p : total_pairs - 1;
      const int lh = D == 128 ? 6 : 5;  // log2(D / 2): D is 64 or 128
      const int feat = (p >> lh) * D + (p & (half - 1)) + ((c & 8) ? half : 0);
      src[i] = a.w + (size_t)feat * hidden + k_begin + piece * 8;
    }
  }

  const int g = lane >> 4, j = lane & 15;
  const int ng = wave % NGW, kq = wave / NGW;
  f32x4 acc[4][NTW];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const u32x4 *buf) {
#pragma unroll
    for (int q = 0; q < KSTEPS / NKQ; ++q) {
      const int ks = kq * (KSTEPS / NKQ) + q;  // k-step of 32 inside the chunk
      const int pc = 4 * ks + g;               // this lane's 16-byte piece
      u32x4 af[4], bfr[NTW];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) af[mt] = buf[(16 * mt + j) * PIECES + (pc ^ j)];
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        bfr[t] = buf[(ROWS + 16 * (ng * NTW + t) + j) * PIECES + (pc ^ j)];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[mt][t] = mfma16(af[mt], bfr[t], acc[mt][t]);
    }
  };
  // Column groups visit their chunks in rotated order: at any moment the
  // groups read different 256-byte offsets of their weight rows (rows are a
  // power-of-two stride apart), spreading requests over the HBM channels.
  const int nch_rt = NCH > 0 ? NCH : sp.ks / KC;
  const int rot = grp % nch_rt;
  auto load = [&](u32x4 *reg, int c) {
    int cc = c + rot;
    cc = cc >= nch_rt ? cc - nch_rt : cc;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) reg[i] = ld16(src[i] + (size_t)cc * KC);
  };
  auto store = [&](u32x4 *buf, const u32x4 *reg) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) buf[dst_slot[i]] = reg[i];
  };

  // This thread's epilogue items (rows and pairs are fixed per thread): their
  // rotation angles, destinations and flags (bit k: item k is stored; bit
  // NIT + k: it is rotated), formed while chunks are still streaming in, so
  // the tail after the last chunk only adds, rotates and stores.  Items the
  // epilogue skips get an unused angle and destination.
  constexpr int NIT = ROWS * PW / (NW * 64);
  static_assert(ROWS * PW % (NW * 64) == 0, "epilogue items must split evenly");
  float ec[NIT], es[NIT];
  uint16_t *edst[NIT];
  unsigned eflags = 0;
  auto angles = [&]() {
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int item = tid + NW * 64 * k;
      const int rl = max(0, min(item / PW, act - 1)), p = pmap(pair0 + item % PW);
      rope_cs(s_pos[rl], s_freq[p % half], ec[k], es[k]);
      edst[k] = pair_dst(a, rl, min(p, total_pairs - 1), s_blk[rl], s_off[rl]);
      if (item / PW < act && p < total_pairs) eflags |= 1u << k;
      if (p / half < 2 * H) eflags |= 1u << (NIT + k);
    }
  };

  // NST register stages and two LDS buffers: while chunk c is multiplied out
  // of one LDS buffer, chunk c + 1 moves from registers into the other and
  // chunks c + 2 .. c + NST are in flight from HBM.  With a compile-time chunk
  // count (NCH > 0) the loop is fully unrolled, so the compiler knows exactly
  // which loads each LDS store waits for; scheduling barriers keep the load
  // groups in issue order.  Loads past the last chunk re-read it (clamped).
  static_assert(NCH == 0 || NCH >= 4, "the metadata steps need four chunks");
  const int nchunks = NCH > 0 ? NCH : sp.ks / KC;
  u32x4 r[NST][LOADS];
#pragma unroll
  for (int t = 0; t < NST; ++t) {
    load(r[t], min(t, nchunks - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  if (epi && tid < half) s_freq[tid] = rope_inv_freq(tid, D, a.log2_base);
  store(lds[0], r[0]);
  load(r[0], min(NST, nchunks - 1));
  __builtin_amdgcn_sched_barrier(0);
  meta(1);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  if constexpr (NCH > 0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      compute(lds[c & 1]);
      if (c + 1 < NCH) {
        store(lds[(c + 1) & 1], r[(c + 1) % NST]);
        if (c + 1 + NST < NCH) load(r[(c + 1) % NST], c + 1 + NST);
        __builtin_amdgcn_sched_barrier(0);
        if (c == 1) meta(2);
        if (c == 2 && epi) angles();
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
      }
    }
  } else {
    for (int c0 = 0; c0 < nchunks; c0 += 2 * NST) {
#pragma unroll
      for (int u = 0; u < 2 * NST; ++u) {
        const int c = c0 + u;
        if (c >= nchunks) break;
        compute(lds[u & 1]);
        store(lds[(u + 1) & 1], r[(u + 1) % NST]);
        load(r[(u + 1) % NST], min(c + 1 + NST, nchunks - 1));
        __syncthreads();
      }
    }
    meta(2);
  }
  __syncthreads();
  if (NCH == 0 && epi) angles();

  // Every wave parks its reduction share's partial tile Y_q[64][CW] (fp32,
  // reusing the LDS); the shares are then added in the fixed order
  // q = NKQ-1 .. 0, whichever wave finished first.
  float *Y = reinterpret_cast<float *>(&lds[0][0]);
  constexpr int YS = CW + 4;       // padded row stride
  constexpr int YQ = ROWS * YS;    // floats per share
  static_assert(NKQ * YQ * 4 <= (int)sizeof(lds), "LDS reuse");
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Y[kq * YQ + (16 * mt + 4 * g + e) * YS + 16 * (ng * NTW + t) + j] = acc[mt][t][e];
  __syncthreads();
  auto ysum = [&](int at) {
    float v = Y[(NKQ - 1) * YQ + at];
#pragma unroll
    for (int q = NKQ - 2; q >= 0; --q) v = Y[q * YQ + at] + v;
    return v;
  };

  if (!epi) {
    float *part = sp.partials + ((size_t)grp * sp.S + split) * ROWS * CW;
    for (int e = tid; e < ROWS * CW / 4; e += NW * 64) {
      const int row = (4 * e) / CW, col = (4 * e) % CW, at = row * YS + col;
      *reinterpret_cast<f32x4 *>(part + 4 * e) =
          f32x4{ysum(at), ysum(at + 1), ysum(at + 2), ysum(at + 3)};
    }
    return;
  }
  if (idx == 0 && wave == 0 && lane < act && a.slot_mapping)
    a.slot_mapping[lane] = (int64_t)m_blk * a.c.bs + m_slot % a.c.bs;
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int item = tid + NW * 64 * k;
    const int rl = item / PW, pl = item % PW;
    if (!(eflags >> k & 1u)) continue;
    const int clo = 16 * (pl >> 3) + (pl & 7);
    const float lo = ysum(rl * YS + clo), hi = ysum(rl * YS + clo + 8);
    if (a.y_out)
      store_raw_pair(a, rl, pmap(pair0 + pl), lo, hi);
    else
      store_word(edst[k], half, rotate_round_cs(lo, hi, eflags >> (NIT + k) & 1u, ec[k], es[k]));
  }
}

template <int NTW, int NGW, int NST, int NCH, int NW, int KC>
__global__ __launch_bounds__(NW * 64) void qkv_splitk_kernel(FlashCacheArgs a, SplitPlan sp) {
  __shared__ SplitLds<NTW, NGW, KC> lds;
  qkv_splitk_body<NTW, NGW, NST, NCH, NW, KC>(a, sp, blockIdx.x, lds);
}

// Adds the S split partials of qkv_splitk_kernel in split order and runs the
// epilogue.  One thread per (row, rotary pair); consecutive threads read
// consecutive partial columns.
template <int CW>
__global__ __launch_bounds__(256) void qkv_reduce_kernel(FlashCacheArgs a, SplitPlan sp) {
  constexpr int PW = CW / 2;
  const int total_pairs = 3 * a.c.H * (a.c.D / 2);
  const int item = blockIdx.x * blockDim.x + threadIdx.x;
  const int per_group = a.rows * PW;
  if (item >= sp.G * per_group) return;
  const int grp = item / per_group;
  const int rl = (item % per_group) / PW, pl = item % PW;
  const int p = grp * PW + pl;
  if (p >= total_pairs || rl >= active_rows(a)) return;
  const int clo = 16 * (pl >> 3) + (pl & 7);
  const size_t split_stride = (size_t)64 * CW;
  const float *base = sp.partials + (size_t)grp * sp.S * split_stride + rl * CW + clo;
  float lo = 0.f, hi = 0.f;
  for (int q = 0; q < sp.S; ++q) {
    lo += base[q * split_stride];
    hi += base[q * split_stride + 8];
  }
  int blk, off, pos;
  row_meta(a, rl, grp == 0 && pl == 0, blk, off, pos);
  store_pair(a, rl, p, lo, hi, blk, off, pos,
             rope_inv_freq(p % (a.c.D >> 1), a.c.D, a.log2_base));
}


// Tiled projection for many active rows (prefill-like batches), where the
// product is MFMA-bound.  A workgroup computes BM rows x
// 32*NWN rotary pairs (tile columns: the pairs' first elements, then their
// partners), with 2 x NWN waves: wave (wm, wn) owns BM/2 rows and pairs
// 32*wn .. 32*wn+31 through 32x32 accumulator columns (first elements,
// partners), so each lane holds both elements of its pairs and rotates them in
// registers.  K advances BK elements at a time through double-buffered LDS
// (BK / 8 16-byte slots per row, XOR-swizzled so that the 16 lanes served
// together hit 16 distinct bank groups); NREG register stages of global loads
// run ahead of the LDS stores, and every iteration issues the same loads
// (clamped past the end) so the compiler waits for exactly one stage.
// Workgroups of one feature tile are dealt to one XCD so the weight tile is
// shared through its L2.
// 16-byte slot swizzle of a staged row (PIECES slots per row): a 16-byte LDS
// access is served 16 lanes at a time, and 16 consecutive rows then cover all
// 16 slots of the 64 banks (no bank conflicts; checked with the LDS counters).
template <int PIECES>
__device__ __forceinline__ int gemm_swz(int row) {
  return PIECES == 4 ? (row >> 2) & 3 : (row >> 1) & 7;
}

// LDS of one tiled-projection workgroup.
template <int BM, int NWN, int BK = 32>
struct GemmLds {
  // staged rows, padded to a whole number of loads per thread (the padding
  // rows receive clamped loads and are never read)
  static constexpr int TR = BM + 64 * NWN, PIECES = BK / 8, NT = 128 * NWN;
  static constexpr int TRP = (TR * PIECES + NT - 1) / NT * NT / PIECES;
  u32x4 lds[2][TRP * PIECES];
  long long s_kvo[BM];  // element offset of the row's cache slot, (blk * H * bs + off) * D
  int s_pos[BM];
};

template <int BM, int NWN, int NREG, int BK = 32, class PM = PairIdentity>
__device__ __forceinline__ void qkv_gemm_body(const FlashCacheArgs &a, int nrow_tiles,
                                              int ncol_tiles, int bid, GemmLds<BM, NWN, BK> &L,
                                              PM pmap = PM{}) {
  constexpr int NT = 128 * NWN;                        // threads
  constexpr int BP = 32 * NWN;                         // pairs per tile
  constexpr int BN = 2 * BP;                           // output features per tile
  constexpr int PIECES = BK / 8;                       // 16-byte slots per row
  static_assert(BK == 32 || BK == 64, "K step");
  constexpr int MTW = BM / 64;                         // 32-row M tiles per wave
  constexpr int TR = BM + BN;                          // staged rows per step
  constexpr int LD = (TR * PIECES + NT - 1) / NT;      // 16-byte loads per thread per step
  static_assert(NT % PIECES == 0, "whole rows per load round");
  auto &lds = L.lds;
  auto &s_kvo = L.s_kvo;
  auto &s_pos = L.s_pos;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.c.H, D = a.c.D, half = D >> 1;
  const int total_pairs = 3 * H * half;
  const int hidden = a.hidden;
  const int nb = nrow_tiles * ncol_tiles;
  // Workgroup bid runs on XCD bid % 8 (workgroups are dealt to the XCDs
  // round-robin).  Each XCD owns a contiguous slice of the column tiles, so
  // its share of W is fetched once, and walks it row tile by row tile: the
  // column tiles that read one X row tile run side by side and share it
  // through that XCD's L2.
  int ct = bid / nrow_tiles, rtile = bid % nrow_tiles;
  if (PM::kIdentity && nb % 8 == 0 && ncol_tiles % 8 == 0) {
    const int cpx = ncol_tiles / 8, l = bid / 8;
    ct = (bid % 8) * cpx + l % cpx;
    rtile = l / cpx;
  } else if (PM::kIdentity && nb % 8 == 0) {
    const int idx = (bid % 8) * (nb / 8) + bid / 8;
    ct = idx / nrow_tiles;
    rtile = idx % nrow_tiles;
  }
  const int row0 = rtile * BM, pair0 = ct * BP;

  const int act = active_rows(a);
  for (int rl = tid; rl < BM; rl += NT) {
    const int r = row0 + rl;
    if (r < act) {
      int blk, off, pos;
      row_meta(a, r, ct == 0, blk, off, pos);
      s_kvo[rl] = ((long long)blk * H * a.c.bs + off) * D;
      s_pos[rl] = pos;
    }
  }

  // This thread's 16-byte chunks of a step: staged row tid / 4 + (NT / 4) * i, slot tid % 4.
  const int piece = tid % PIECES;
  const uint16_t *src[LD];
  int slot[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int tr = tid / PIECES + (NT / PIECES) * i;
    if (tr < BM) {
      const int r = min(row0 + tr, a.rows - 1);
      src[i] = a.x + (size_t)r * hidden + piece * 8;
    } else {
      const int c = tr - BM;  // 0..BN-1: first elements, then partners
      int p = pmap(pair0 + (c % BP));
      p = p < total_pairs ? p : total_pairs - 1;
      const int feat = (p / half) * D + (p % half) + (c >= BP ? half : 0);
      src[i] = a.w + (size_t)feat * hidden + piece * 8;
    }
    slot[i] = tr * PIECES + (piece ^ gemm_swz<PIECES>(tr));
  }
  const int nk = hidden / BK;
  u32x4 rg[NREG][LD];
  auto load = [&](u32x4 *r, int kt) {
    const int k = min(kt, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < LD; ++i) r[i] = ld16(src[i] + k);
  };
  auto store = [&](u32x4 *buf, const u32x4 *r) {
#pragma unroll
    for (int i = 0; i < LD; ++i) buf[slot[i]] = r[i];
  };

  const int wm = wave / NWN, wn = wave % NWN;
  const int l32 = lane & 31, hi = lane >> 5;
  f32x16 acc[MTW][2];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][c][e] = 0.f;

  // Prologue: step 0 in LDS, steps 1 .. NREG in registers.
  {
    u32x4 r0[LD];
    load(r0, 0);
#pragma unroll
    for (int s = 0; s < NREG; ++s) load(rg[s], 1 + s);
    store(lds[0], r0);
  }
  const int nk_r = (nk + NREG - 1) / NREG * NREG;
  for (int k0 = 0; k0 < nk_r; k0 += NREG) {
#pragma unroll
    for (int s = 0; s < NREG; ++s) {
      const int kt = k0 + s;
      lds_barrier();
      if (kt < nk) {
        const u32x4 *buf = lds[kt & 1];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          const int pc = 2 * ks + hi;
          u32x4 af[MTW], bfr[2];
#pragma unroll
          for (int mt = 0; mt < MTW; ++mt) {
            const int row = wm * (BM / 2) + 32 * mt + l32;
            af[mt] = buf[row * PIECES + (pc ^ gemm_swz<PIECES>(row))];
          }
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int row = BM + BP * c + 32 * wn + l32;
            bfr[c] = buf[row * PIECES + (pc ^ gemm_swz<PIECES>(row))];
          }
#pragma unroll
          for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int c = 0; c < 2; ++c) acc[mt][c] = mfma32(af[mt], bfr[c], acc[mt][c]);
        }
      }
      store(lds[(kt + 1) & 1], rg[s]);  // step kt + 1 (a clamped repeat past the end)
      load(rg[s], kt + 1 + NREG);
    }
  }

  // Epilogue: lane holds pair pair0 + 32 wn + l32 for 16 rows per M tile.
  // The pair's section, head and destination column are formed once; each
  // row then adds its own offset (Q row, or cache slot from s_kvo).
  const int p = pmap(pair0 + 32 * wn + l32);
  if (p >= total_pairs) return;
  if (a.y_out) {  // unfused ablation: the raw fp32 pairs
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rl = wm * (BM / 2) + 32 * mt + 8 * (e / 4) + 4 * hi + (e % 4);
        if (row0 + rl < act) store_raw_pair(a, row0 + rl, p, acc[mt][0][e], acc[mt][1][e]);
      }
    return;
  }
  const int sh = p / half, i = p % half, sec = sh / H, h = sh % H;
  const bool rot = sec < 2;
  const double freq = rope_inv_freq(i, D, a.log2_base);
  uint16_t *const base = sec == 0 ? a.q_out + (size_t)h * D + i
                                  : (sec == 1 ? a.c.k : a.c.v) + (size_t)h * a.c.bs * D + i;
  // One loop per destination kind (the section is the same for the whole
  // wave); rows past the active ones only occur in a grid's last row tile.
  const bool full = row0 + BM <= act;
  auto rows = [&](auto dst_off, auto rotate) {
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rl = wm * (BM / 2) + 32 * mt + 8 * (e / 4) + 4 * hi + (e % 4);
        if (!full && row0 + rl >= act) continue;
        float c = 1.f, sn = 0.f;
        if (rotate.value) rope_cs(s_pos[rl], freq, c, sn);
        store_word(base + dst_off(rl), half,
                   rotate_round_cs(acc[mt][0][e], acc[mt][1][e], rotate.value, c, sn));
      }
  };
  if (sec == 0) {
    const size_t qstride = (size_t)H * D;
    rows([&](int rl) { return (size_t)(row0 + rl) * qstride; }, std::true_type{});
  } else if (rot) {
    rows([&](int rl) { return (size_t)s_kvo[rl]; }, std::true_type{});
  } else {
    rows([&](int rl) { return (size_t)s_kvo[rl]; }, std::false_type{});
  }
}



template <int BM, int NWN, int NREG, int BK>
__global__ __launch_bounds__(128 * NWN) void qkv_gemm_kernel(FlashCacheArgs a, int nrow_tiles,
                                                              int ncol_tiles) {
  __shared__ GemmLds<BM, NWN, BK> lds;
  qkv_gemm_body<BM, NWN, NREG, BK>(a, nrow_tiles, ncol_tiles, blockIdx.x, lds);
}

// Unfused ablation, stage 2: rotary embedding and bf16 rounding from the fp32
// projection in HBM; Q to its buffer, K and V rows to staging buffers
// [rows][H][D].  One thread per (row, rotary pair).
__global__ __launch_bounds__(256) void rope_round_kernel(FlashCacheArgs a, const float *y,
                                                          uint16_t *k_stage, uint16_t *v_stage) {
  const int H = a.c.H, D = a.c.D, half = D >> 1;
  const int pairs = 3 * H * half;
  const size_t item = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (size_t)a.rows * pairs) return;
  const int r = (int)(item / pairs), p = (int)(item % pairs);
  if (r >= active_rows(a)) return;
  const int sh = p / half, i = p % half, sec = sh / H, h = sh % H;
  const float *yr = y + (size_t)r * 3 * H * D + (size_t)sh * D + i;
  const uint32_t v = rotate_round(yr[0], yr[half], sec, a.positions[r],
                                  rope_inv_freq(i, D, a.log2_base));
  uint16_t *dst = (sec == 0 ? a.q_out : sec == 1 ? k_stage : v_stage) + ((size_t)r * H + h) * D;
  dst[i] = (uint16_t)(v & 0xffffu);
  dst[i + half] = (uint16_t)(v >> 16);
}

// Unfused ablation, stage 3: copy the staged K and V rows into the paged cache
// and write the slot mapping.  One thread per (row, head, 16-byte chunk).
__global__ __launch_bounds__(256) void scatter_kv_kernel(FlashCacheArgs a, const uint16_t *k_stage,
                                                          const uint16_t *v_stage) {
  const int H = a.c.H, D = a.c.D, ch = D / 8;
  const size_t item = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (size_t)a.rows * H * ch) return;
  const int r = (int)(item / (H * ch)), rem = (int)(item % (H * ch));
  if (r >= active_rows(a)) return;
  const int h = rem / ch, c = rem % ch;
  int blk, off, pos;
  row_meta(a, r, h == 0 && c == 0, blk, off, pos);
  const size_t src = ((size_t)r * H + h) * D + c * 8;
  const size_t dst = (((size_t)blk * H + h) * a.c.bs + off) * D + c * 8;
  st16(a.c.k + dst, ld16(k_stage + src));
  st16(a.c.v + dst, ld16(v_stage + src));
}

}  // namespace

#ifndef FDL_DEVICE_ONLY
// Compute units of the current device (cached per device; 256 if the query
// fails, the part's count).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                           hipSuccess && n > 0
                   ? n
                   : 256;
  }
  return cus[dev];
}
#endif

// Tile shape of the split-K projection: kSplitNTW 16-feature tiles per wave,
// kSplitNGW wave groups across features, kSplitNST register stages,
// kSplitWaves waves, kSplitKC reduction elements per staged chunk; at most
// kSplitCap workgroups before the reduction is split.
namespace {
constexpr int kSplitNTW = 3, kSplitNGW = 1, kSplitNST = 2, kSplitWaves = 8, kSplitKC = 256;
constexpr int kSplitCap = 320;
constexpr int kSplitCW = 16 * kSplitNTW * kSplitNGW;  // features per column group

struct FcPlan {
  bool splitk;
  int G, S;
  size_t bytes;
};

FcPlan plan_fc(int rows, int hidden, int H, int D) {
  FcPlan p{};
  const int total_pairs = 3 * H * (D / 2);
  if (rows > 64 || hidden % kSplitKC != 0) return p;  // tiled kernel, no workspace
  p.splitk = true;
  p.G = (total_pairs + kSplitCW / 2 - 1) / (kSplitCW / 2);
  p.S = 1;
  while (p.S < 8 && p.G * 2 * p.S <= kSplitCap && hidden % (kSplitKC * 2 * p.S) == 0) p.S *= 2;
  if (p.S > 1) p.bytes = (size_t)p.G * p.S * 64 * kSplitCW * sizeof(float);
  return p;
}
}  // namespace

// The externally visible launchers; a unit that compiles this file only for
// its device bodies (the fused step) defines FDL_DEVICE_ONLY and leaves them out.
#ifndef FDL_DEVICE_ONLY
size_t flash_cache_workspace_bytes(int rows, int hidden, int H, int D) {
  return plan_fc(rows, hidden, H, D).bytes;
}

// An upper bound of flash_cache_workspace_bytes over every shape: a reduction
// is split only while groups x splits stay within kSplitCap.
size_t flash_cache_workspace_max() {
  return (size_t)kSplitCap * 64 * kSplitCW * sizeof(float);
}

hipError_t launch_flash_cache(const FlashCacheArgs &a, void *ws, size_t ws_bytes, hipStream_t s) {
  const FcPlan fp = plan_fc(a.rows, a.hidden, a.c.H, a.c.D);
  if (fp.splitk) {
    if (ws_bytes < fp.bytes || (fp.bytes && !ws)) return hipErrorInvalidValue;
    SplitPlan sp;
    sp.G = fp.G;
    sp.S = fp.S;
    sp.ks = a.hidden / fp.S;
    sp.partials = fp.bytes ? static_cast<float *>(ws) : nullptr;
    const int nch = sp.ks / kSplitKC;
    const dim3 grid(fp.G * fp.S), block(kSplitWaves * 64);
    switch (nch) {
      case 4:
        hipLaunchKernelGGL((qkv_splitk_kernel<kSplitNTW, kSplitNGW, kSplitNST, 4, kSplitWaves, kSplitKC>), grid, block, 0,
                           s, a, sp);
        break;
      case 8:
        hipLaunchKernelGGL((qkv_splitk_kernel<kSplitNTW, kSplitNGW, kSplitNST, 8, kSplitWaves, kSplitKC>), grid, block, 0,
                           s, a, sp);
        break;
      case 16:
        hipLaunchKernelGGL((qkv_splitk_kernel<kSplitNTW, kSplitNGW, kSplitNST, 16, kSplitWaves, kSplitKC>), grid, block,
                           0, s, a, sp);
        break;
      case 32:
        hipLaunchKernelGGL((qkv_splitk_kernel<kSplitNTW, kSplitNGW, kSplitNST, 32, kSplitWaves, kSplitKC>), grid, block,
                           0, s, a, sp);
        break;
      default:
        hipLaunchKernelGGL((qkv_splitk_kernel<kSplitNTW, kSplitNGW, kSplitNST, 0, kSplitWaves, kSplitKC>), grid, block, 0,
                           s, a, sp);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fp.S == 1) return e;
    const int items = fp.G * a.rows * (kSplitCW / 2);
    hipLaunchKernelGGL((qkv_reduce_kernel<kSplitCW>), dim3((items + 255) / 256), dim3(256), 0, s,
                       a, sp);
    return hipGetLastError();
  }
  // More than 64 rows (or a hidden size the chunking does not divide): the
  // tiled MFMA kernel.  When a grid of 128 rows x 96 rotary pairs (six waves)
  // fits one workgroup per CU, that form runs with K in steps of 64 and one
  // register stage (each workgroup owns its CU; half the barriers per MFMA);
  // failing that, 256-row tiles of the same width if their grid fits (twice
  // the reuse of each weight tile); larger grids take 128 rows x 128 pairs
  // (eight waves) in steps of 32 with two register stages, two workgroups per
  // CU, whose loads in flight hide more of the weight stream's latency.
  // Measured on the bench: 76.9 against 94.5 us at 512 rows, 137.4 against
  // 157.3 us at 1024, 237.5 against 254.3 us at 2048 (the other forms).  Every
  // form accumulates in the same order, so the results are the same.
  const int total_pairs = 3 * a.c.H * (a.c.D / 2);
  constexpr int BM = 128;
  const int cus = device_cus();
  const int ncol6 = (total_pairs + 95) / 96;
  const int nrow = (a.rows + BM - 1) / BM, nrow2 = (a.rows + 2 * BM - 1) / (2 * BM);
  if (nrow * ncol6 <= cus) {
    hipLaunchKernelGGL((qkv_gemm_kernel<BM, 3, 1, 64>), dim3(nrow * ncol6), dim3(128 * 3), 0, s,
                       a, nrow, ncol6);
  } else if (nrow2 * ncol6 <= cus) {
    hipLaunchKernelGGL((qkv_gemm_kernel<2 * BM, 3, 1, 64>), dim3(nrow2 * ncol6), dim3(128 * 3), 0,
                       s, a, nrow2, ncol6);
  } else {
    const int ncol8 = (total_pairs + 127) / 128;
    hipLaunchKernelGGL((qkv_gemm_kernel<BM, 4, 2, 32>), dim3(nrow * ncol8), dim3(128 * 4), 0, s,
                       a, nrow, ncol8);
  }
  return hipGetLastError();
}

size_t flash_cache_unfused_workspace_bytes(int rows, int hidden, int H, int D) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(flash_cache_workspace_bytes(rows, hidden, H, D)) +
         al((size_t)rows * 3 * H * D * sizeof(float)) + 2 * al((size_t)rows * H * D * 2);
}

// The same step as three launches with the intermediates in HBM: projection
// (fp32 Y out), rotary + rounding (bf16 staging out), cache scatter.  The
// projection kernels and the rounding helper are the fused path's own, so the
// results are bitwise identical; only the memory traffic differs.
hipError_t launch_flash_cache_unfused(const FlashCacheArgs &a, void *ws, size_t ws_bytes,
                                      hipStream_t s) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int H = a.c.H, D = a.c.D;
  const size_t part = al(flash_cache_workspace_bytes(a.rows, a.hidden, H, D));
  const size_t ybytes = al((size_t)a.rows * 3 * H * D * sizeof(float));
  const size_t sbytes = al((size_t)a.rows * H * D * 2);
  if (ws_bytes < part + ybytes + 2 * sbytes || !ws) return hipErrorInvalidValue;
  char *base = static_cast<char *>(ws);
  FlashCacheArgs g = a;
  g.y_out = reinterpret_cast<float *>(base + part);
  g.slot_mapping = nullptr;
  hipError_t e = launch_flash_cache(g, part ? base : nullptr, part, s);
  if (e != hipSuccess) return e;
  uint16_t *ks = reinterpret_cast<uint16_t *>(base + part + ybytes);
  uint16_t *vs = reinterpret_cast<uint16_t *>(base + part + ybytes + sbytes);
  const size_t n1 = (size_t)a.rows * 3 * H * (D / 2);
  hipLaunchKernelGGL(rope_round_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s, a,
                     g.y_out, ks, vs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t n2 = (size_t)a.rows * H * (D / 8);
  hipLaunchKernelGGL(scatter_kv_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, a,
                     ks, vs);
  return hipGetLastError();
}

#endif  // FDL_DEVICE_ONLY

}  // namespace fdl

