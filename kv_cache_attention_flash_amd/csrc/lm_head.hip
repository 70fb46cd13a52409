// Mask-view confidence producer for gfx950: LM-head logits z = h . W^T over the
// vocabulary, and per row the argmax token and its softmax probability.
//
// Source: [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for
// Fast, Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary),
// para 3 (a position is accepted when the two views agree and the mask-view
// confidence exceeds the threshold).  Reading: token = argmax of the logits
// (ties to the lower id), confidence = its softmax probability.
//
// The logits never reach HBM: a tile kernel computes 128 rows x 256 vocabulary
// columns with MFMA and reduces each row of its tile to (max, the lowest id
// holding it, sum of exp(z - max)); a merge kernel combines the tiles of a
// row in a fixed order.
#include "device_common.h"
#include "internal.h"

namespace fdl {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInfL = -__builtin_huge_valf();

// (max, id) pairs: the larger value wins, equal values go to the lower id.
__device__ __forceinline__ void arg_take(float &m, int &id, float om, int oid) {
  if (om > m || (om == m && oid < id)) {
    m = om;
    id = oid;
  }
}

// BM rows x BN = 64 * NWN vocabulary columns per workgroup, 2 x NWN waves;
// wave (wm, wn) owns BM/2 rows and columns 32 wn + l32 of each 32 * NWN
// column half.  K advances 32 elements at a time through double-buffered LDS
// (16-byte slots swizzled by (row / 4) % 4) with NREG register stages of
// global loads ahead; every iteration issues the same loads (clamped past the
// end).  Workgroups of one column tile are dealt to one XCD so the weight
// tile is shared through its L2.
template <int BM, int NWN, int NREG>
__global__ __launch_bounds__(128 * NWN) void lmhead_tile_kernel(LmHeadArgs a, int nrow_tiles,
                                                                 int ncol_tiles) {
  constexpr int NT = 128 * NWN;
  constexpr int BH = 32 * NWN;                         // columns per half
  constexpr int BN = 2 * BH;                           // columns per tile
  constexpr int BK = 32, PIECES = BK / 8;
  constexpr int MTW = BM / 64;
  constexpr int TR = BM + BN;
  constexpr int LD = TR * PIECES / NT;
  static_assert(TR * PIECES % NT == 0, "step must split evenly over the threads");
  __shared__ u32x4 lds[2][TR * PIECES];
  __shared__ float s_m[NWN][BM], s_l[NWN][BM];
  __shared__ int s_i[NWN][BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = nrow_tiles * ncol_tiles;
  int idx = blockIdx.x;
  if (nb % 8 == 0) idx = (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8;
  const int ct = idx / nrow_tiles, rtile = idx % nrow_tiles;
  const int row0 = rtile * BM, col0 = ct * BN;
  const int hidden = a.hidden;

  const int piece = tid % PIECES;
  const uint16_t *src[LD];
  int slot[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int tr = tid / PIECES + (NT / PIECES) * i;
    if (tr < BM) {
      src[i] = a.h + (size_t)min(row0 + tr, a.rows - 1) * hidden + piece * 8;
    } else {
      src[i] = a.w + (size_t)min(col0 + tr - BM, a.vocab - 1) * hidden + piece * 8;
    }
    slot[i] = tr * PIECES + (piece ^ ((tr >> 2) & 3));
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
            af[mt] = buf[row * PIECES + (pc ^ ((row >> 2) & 3))];
          }
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int row = BM + BH * c + 32 * wn + l32;
            bfr[c] = buf[row * PIECES + (pc ^ ((row >> 2) & 3))];
          }
#pragma unroll
          for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int c = 0; c < 2; ++c) acc[mt][c] = mfma32(af[mt], bfr[c], acc[mt][c]);
        }
      }
      store(lds[(kt + 1) & 1], rg[s]);
      load(rg[s], kt + 1 + NREG);
    }
  }

  // Epilogue.  Lane (l32, hi) holds columns cA = col0 + 32 wn + l32 and
  // cB = cA + BH for rows 32 mt + 8 (e / 4) + 4 hi + e % 4 of its wave's half.
  const int cA = col0 + 32 * wn + l32, cB = cA + BH;
  const bool okA = cA < a.vocab, okB = cB < a.vocab;
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float v0 = okA ? acc[mt][0][e] : kNegInfL;
      const float v1 = okB ? acc[mt][1][e] : kNegInfL;
      float m = v0;
      int id = cA;
      arg_take(m, id, v1, cB);
      // Butterfly over the 32 column lanes of this half (fixed order).
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        const float om = __shfl_xor(m, o, 64);
        const int oid = __shfl_xor(id, o, 64);
        arg_take(m, id, om, oid);
      }
      // a wave whose columns all lie past the vocabulary (last tile) has no maximum
      float s = m == kNegInfL ? 0.f : exp2f((v0 - m) * kLog2e) + exp2f((v1 - m) * kLog2e);
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) s += __shfl_xor(s, o, 64);
      const int rl = wm * (BM / 2) + 32 * mt + 8 * (e / 4) + 4 * hi + (e % 4);
      if (l32 == 0) {
        s_m[wn][rl] = m;
        s_i[wn][rl] = id;
        s_l[wn][rl] = s;
      }
    }
  __syncthreads();
  for (int rl = tid; rl < BM; rl += NT) {
    float m = s_m[0][rl];
    int id = s_i[0][rl];
#pragma unroll
    for (int w2 = 1; w2 < NWN; ++w2) arg_take(m, id, s_m[w2][rl], s_i[w2][rl]);
    float l = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NWN; ++w2)
      if (s_m[w2][rl] != kNegInfL) l += s_l[w2][rl] * exp2f((s_m[w2][rl] - m) * kLog2e);
    const int r = row0 + rl;
    if (r < a.rows) {
      const size_t o = (size_t)r * ncol_tiles + ct;
      a.part_ml[2 * o] = m;
      a.part_ml[2 * o + 1] = l;
      a.part_idx[o] = id;
    }
  }
}

// One wave per row: lane t merges column tiles t, t + 64, ... in order, then
// a butterfly over the 64 lanes (fixed order) gives the row's maximum, its
// lowest id and the sum of exp(z - max); confidence = 1 / that sum.
__global__ __launch_bounds__(256) void lmhead_merge_kernel(LmHeadArgs a, int ncol_tiles) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.rows) return;
  const float *pm = a.part_ml + (size_t)r * ncol_tiles * 2;
  const int32_t *pi = a.part_idx + (size_t)r * ncol_tiles;
  float m = kNegInfL, l = 0.f;
  int id = 0x7fffffff;
  for (int t = lane; t < ncol_tiles; t += 64) {
    const float tm = pm[2 * t], tl = pm[2 * t + 1];
    const int ti = pi[t];
    const float mx = fmaxf(m, tm);
    l = (m == kNegInfL ? 0.f : l * exp2f((m - mx) * kLog2e)) + tl * exp2f((tm - mx) * kLog2e);
    arg_take(m, id, tm, ti);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float om = __shfl_xor(m, o, 64), ol = __shfl_xor(l, o, 64);
    const int oid = __shfl_xor(id, o, 64);
    const float mx = fmaxf(m, om);
    const float la = m == kNegInfL ? 0.f : l * exp2f((m - mx) * kLog2e);
    const float lb = om == kNegInfL ? 0.f : ol * exp2f((om - mx) * kLog2e);
    l = (lane & o) ? lb + la : la + lb;  // the pair adds the same two terms in one order
    arg_take(m, id, om, oid);
  }
  if (lane == 0) {
    a.token[r] = id;
    a.conf[r] = 1.f / l;
  }
}

}  // namespace

int lm_head_col_tiles(int vocab) { return (vocab + 255) / 256; }

size_t lm_head_workspace_bytes(int rows, int vocab) {
  const size_t n = (size_t)rows * lm_head_col_tiles(vocab);
  return ((n * 2 * sizeof(float) + 255) & ~(size_t)255) + n * sizeof(int32_t);
}

hipError_t launch_lm_head(LmHeadArgs a, void *ws, hipStream_t s) {
  const int ncol = lm_head_col_tiles(a.vocab);
  const size_t n = (size_t)a.rows * ncol;
  char *base = static_cast<char *>(ws);
  a.part_ml = reinterpret_cast<float *>(base);
  a.part_idx = reinterpret_cast<int32_t *>(base + ((n * 2 * sizeof(float) + 255) & ~(size_t)255));
  constexpr int BM = 128, NWN = 4;
  const int nrow = (a.rows + BM - 1) / BM;
  hipLaunchKernelGGL((lmhead_tile_kernel<BM, NWN, 2>), dim3(nrow * ncol), dim3(128 * NWN), 0, s,
                     a, nrow, ncol);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lmhead_merge_kernel, dim3((a.rows + 3) / 4), dim3(256), 0, s, a, ncol);
  return hipGetLastError();
}

}  // namespace fdl
