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
// same workgroup and the rotation needs no extra memory traffic.  A workgroup
// owns NT x 8 consecutive pairs (16 x NT output features) for a strip of
// 16 x MT rows and the WHOLE reduction dimension, split across its NW waves:
// every weight byte is read from HBM exactly once per row strip.  The waves'
// partial sums meet in LDS; the epilogue adds them in wave order (deterministic),
// rotates in fp32 with an fp64-reduced angle, rounds to bf16 (RNE) and scatters
// K/V through the block table.  MFMA: v_mfma_f32_16x16x32_bf16, both operands
// loaded 16 bytes per lane straight from global memory (the weight is stored
// feature-major, so each lane's 8 reduction elements are contiguous).
#include "device_common.h"
#include "internal.h"

namespace fdl {

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

// Largest b with cu_rows[b] <= r (empty sequences are skipped over).
__device__ __forceinline__ int row_to_seq(const int32_t *cu_rows, int batch, int r) {
  int lo = 0, hi = batch;  // invariant: cu_rows[lo] <= r < cu_rows[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu_rows[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// cos/sin of position * base^(-2i/D): angle and its reduction to [-pi, pi] in
// fp64, the trigonometric functions in fp32 on the reduced angle.
__device__ __forceinline__ void rope_cs(int pos, int i, int D, double log2_base, float &c,
                                        float &s) {
  double theta = exp2(-(2.0 * (double)i / (double)D) * log2_base);
  double ang = (double)pos * theta;
  double k = rint(ang * (1.0 / kTwoPi));
  double red = fma(-k, kTwoPi, ang);
  sincosf((float)red, &s, &c);
}

template <int MT, int NT, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void qkv_rope_write_kernel(FlashCacheArgs a) {
  constexpr int ROWS = 16 * MT;
  constexpr int COLS = 16 * NT;
  constexpr int PAIRS = 8 * NT;
  __shared__ float red[NW][ROWS][COLS + 1];
  __shared__ int s_blk[ROWS], s_off[ROWS], s_pos[ROWS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int H = a.c.H, D = a.c.D, half = D >> 1;
  const int total_pairs = 3 * H * half;
  const int pair0 = blockIdx.x * PAIRS;
  const int row0 = blockIdx.y * ROWS;
  const int hidden = a.hidden;

  // Row metadata: sequence, physical slot, rotary position.
  if (tid < ROWS) {
    int r = row0 + tid;
    if (r < a.rows) {
      int b = row_to_seq(a.cu_rows, a.batch, r);
      int s = a.slots[r];
      int blk = a.c.block_table[(size_t)b * a.c.max_blocks + s / a.c.bs];
      int off = s % a.c.bs;
      s_blk[tid] = blk;
      s_off[tid] = off;
      s_pos[tid] = a.positions[r];
      if (blockIdx.x == 0 && a.slot_mapping)
        a.slot_mapping[r] = (int64_t)blk * a.c.bs + off;
    }
  }

  // Operand rows of this lane.
  const int g = lane >> 4;  // reduction slot group
  const int j = lane & 15;  // A row / B column inside a 16-tile
  const uint16_t *xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = row0 + mt * 16 + j;
    r = r < a.rows ? r : a.rows - 1;
    xrow[mt] = a.x + (size_t)r * hidden + 8 * g;
  }
  const uint16_t *wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int p = pair0 + 8 * t + (j & 7);
    p = p < total_pairs ? p : total_pairs - 1;
    int feat = (p / half) * D + (p % half) + ((j & 8) ? half : 0);
    wrow[t] = a.w + (size_t)feat * hidden + 8 * g;
  }

  // Reduction steps of 32 split evenly over the waves.
  const int steps = hidden / 32;
  const int per = (steps + NW - 1) / NW;
  const int s_begin = wave * per;
  const int s_end = min(steps, s_begin + per);

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Register ring of DEPTH reduction steps in flight per wave: the loads of
  // step st + DEPTH are issued as soon as step st's operands are consumed, so
  // every wave keeps DEPTH * (MT + NT) KiB of loads outstanding.
  // Loads are unconditional (addresses clamped to the last valid step) so the
  // compiler can count outstanding loads exactly across the unrolled ring.
  u32x4 abuf[DEPTH][MT], bbuf[DEPTH][NT];
  const int nsteps = max(0, s_end - s_begin);
  const int nfull = nsteps / DEPTH * DEPTH;
  // Workgroups start their step loop at different offsets (rotation by the
  // workgroup's index within its XCD) so that the many workgroups sharing an
  // L2 do not all read the same activation lines at the same moment.
#ifndef FDL_FC_ROTATE
#define FDL_FC_ROTATE 1
#endif
  const int rot = FDL_FC_ROTATE ? (int)(blockIdx.x >> 3) : 0;
  auto issue = [&](int d, int st) {
    const int rel = min(st, s_end - 1) - s_begin;
    const int k = (nsteps > 0 ? s_begin + (rel + rot) % nsteps : 0) * 32;
#pragma unroll
    for (int t = 0; t < NT; ++t) bbuf[d][t] = ld16(wrow[t] + k);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) abuf[d][mt] = ld16(xrow[mt] + k);
  };
  auto consume = [&](int d) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[mt][t] = mfma16(abuf[d][mt], bbuf[d][t], acc[mt][t]);
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue(d, s_begin + d);
  for (int st0 = 0; st0 < nfull; st0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      consume(d);
      issue(d, s_begin + st0 + d + DEPTH);
    }
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < nsteps - nfull) consume(d);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][mt * 16 + 4 * g + e][t * 16 + j] = acc[mt][t][e];
  __syncthreads();

  // Epilogue: one (row, pair) per thread and iteration.
  for (int item = tid; item < ROWS * PAIRS; item += NW * 64) {
    const int rl = item / PAIRS;
    const int pl = item % PAIRS;
    const int r = row0 + rl;
    const int p = pair0 + pl;
    if (r >= a.rows || p >= total_pairs) continue;
    const int clo = (pl >> 3) * 16 + (pl & 7);
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lo += red[w][rl][clo];
      hi += red[w][rl][clo + 8];
    }
    const int sh = p / half;  // section * H + head
    const int i = p % half;
    const int sec = sh / H;
    const int h = sh % H;
    if (sec < 2) {
      float c, s;
      rope_cs(s_pos[rl], i, D, a.log2_base, c, s);
      const float rlo = lo * c - hi * s;
      const float rhi = hi * c + lo * s;
      lo = rlo;
      hi = rhi;
    }
    const uint16_t blo = f32_to_bf16_rne(lo), bhi = f32_to_bf16_rne(hi);
    uint16_t *dst;
    if (sec == 0) {
      dst = a.q_out + ((size_t)r * H + h) * D;
    } else {
      uint16_t *pool = sec == 1 ? a.c.k : a.c.v;
      dst = pool + (((size_t)s_blk[rl] * H + h) * a.c.bs + s_off[rl]) * D;
    }
    dst[i] = blo;
    dst[i + half] = bhi;
  }
}

}  // namespace

// Tile shape of the skinny (few active rows) projection: 16*MT rows, 8*NT
// rotary pairs and NW waves per workgroup, DEPTH reduction steps in flight.
#ifndef FDL_FC_NT
#define FDL_FC_NT 3
#endif
#ifndef FDL_FC_NW
#define FDL_FC_NW 8
#endif
#ifndef FDL_FC_DEPTH
#define FDL_FC_DEPTH 4
#endif

hipError_t launch_flash_cache(const FlashCacheArgs &a, hipStream_t s) {
  constexpr int MT = 4, NT = FDL_FC_NT, NW = FDL_FC_NW, DEPTH = FDL_FC_DEPTH;
  const int total_pairs = 3 * a.c.H * (a.c.D / 2);
  dim3 grid((total_pairs + 8 * NT - 1) / (8 * NT), (a.rows + 16 * MT - 1) / (16 * MT));
  hipLaunchKernelGGL((qkv_rope_write_kernel<MT, NT, NW, DEPTH>), grid, dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace fdl
