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
// K (row-major) and V (transposed) are staged in LDS and shared by the 4 waves.
// Per wave S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys along M) so that each
// lane holds one query row: row maxima and sums are in-lane plus two shuffles,
// and the fp32 probabilities convert in-register into the B operand of
// O^T += V^T P^T.  The K rows feeding the two 16-key M tiles are permuted so
// that lane group g ends up holding the 8 consecutive keys 8g..8g+7, which
// makes each V^T operand one 16-byte LDS read.  Online softmax in base 2.
// With several KV splits the unnormalised partials meet in attn_merge (fixed
// split order).
//
// Mass: m[b][j] = sum_h sum_r exp(s_rj - LSE_r) needs every row's final
// log-sum-exp, known only after all keys, so the mass is a second pass over K
// (attn_mass) using the LSE of pass 1; per-(sequence, head) partial sums are
// added over heads in head order by mass_head_reduce.  Nothing uses floating
// atomics: results are bitwise reproducible.
#include "device_common.h"
#include "internal.h"

namespace fdl {

namespace {

constexpr int KT = 32;  // keys per tile
constexpr float kNegInf = -__builtin_huge_valf();

struct SeqInfo {
  int r0, nrows, L, w0, wl, d0;
};

__device__ __forceinline__ SeqInfo seq_info(const AttnArgs &a, int b) {
  SeqInfo si;
  si.r0 = a.cu_rows[b];
  si.nrows = a.cu_rows[b + 1] - si.r0;
  si.L = a.kv_len[b];
  if (a.views) {
    si.w0 = a.views[3 * b];
    si.wl = a.views[3 * b + 1];
    si.d0 = a.views[3 * b + 2];
  } else {
    si.w0 = si.wl = si.d0 = 0;
  }
  return si;
}

// May local row t of a sequence see slot j?
__device__ __forceinline__ bool visible(const SeqInfo &si, int t, int j) {
  if (j >= si.L) return false;
  if (si.wl == 0) return true;
  if (t < si.wl) {
    bool ctx = j < si.d0 && (j < si.w0 || j >= si.w0 + si.wl);
    return ctx || (j >= si.d0 && j <= si.d0 + t);
  }
  return j < si.d0;
}

// Stage one 32-key tile of head h: K as [key][D + 8], V transposed as [D][KT + 8].
template <int D>
__device__ __forceinline__ void stage_tile(const AttnArgs &a, int b, int h, int key0,
                                           uint16_t (*klds)[D + 8], uint16_t (*vt)[KT + 8],
                                           bool want_v) {
  const int bs = a.c.bs;
  const int page = a.c.block_table[(size_t)b * a.c.max_blocks + key0 / bs];
  const size_t base = (((size_t)page * a.c.H + h) * bs + (key0 % bs)) * D;
  constexpr int CH = D / 8;            // 16-byte chunks per key
  constexpr int N = KT * CH;           // chunks per tile
  for (int c = threadIdx.x; c < N; c += blockDim.x) {
    const int key = c / CH, dc = c % CH;
    u32x4 kv = ld16(a.c.k + base + (size_t)c * 8);
    st16(&klds[key][dc * 8], kv);
    if (want_v) {
      u32x4 vv = ld16(a.c.v + base + (size_t)c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[dc * 8 + 2 * e][key] = (uint16_t)(vv[e] & 0xffffu);
        vt[dc * 8 + 2 * e + 1][key] = (uint16_t)(vv[e] >> 16);
      }
    }
  }
}

// S^T tile (32 keys x 16 rows) for one wave: s[mt][e] is key 8g + 4mt + e for
// query row (lane & 15).
template <int D>
__device__ __forceinline__ void scores(const uint16_t (*klds)[D + 8], const u32x4 *qf,
                                       int lane, f32x4 s[2]) {
  const int g = lane >> 4, j = lane & 15;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int key = 8 * (j >> 2) + 4 * mt + (j & 3);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      u32x4 kf = ld16(&klds[key][32 * ks + 8 * g]);
      acc = mfma16(kf, qf[ks], acc);
    }
    s[mt] = acc;
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnArgs a, AttnPlan p) {
  __shared__ uint16_t klds[KT][D + 8];
  __shared__ uint16_t vt[D][KT + 8];

  int u = blockIdx.x;
  const int split = u % p.splits; u /= p.splits;
  const int h = u % a.c.H; u /= a.c.H;
  const int rt = u % p.row_tiles;
  const int b = u / p.row_tiles;
  const SeqInfo si = seq_info(a, b);
  const int t0 = rt * 64;
  if (t0 >= si.nrows) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int t = t0 + wave * 16 + j;  // local row of this lane
  const bool row_ok = t < si.nrows;
  const int r = si.r0 + (row_ok ? t : 0);

  u32x4 qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = row_ok ? ld16(a.q + ((size_t)r * a.c.H + h) * D + 32 * ks + 8 * g)
                    : u32x4{0u, 0u, 0u, 0u};

  const int tiles = (si.L + KT - 1) / KT;
  const int tps = (tiles + p.splits - 1) / p.splits;
  const int tb = split * tps, te = min(tiles, tb + tps);

  f32x4 o[D / 16];
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) o[dm] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;

  for (int tile = tb; tile < te; ++tile) {
    const int key0 = tile * KT;
    stage_tile<D>(a, b, h, key0, klds, vt, true);
    __syncthreads();
    f32x4 s[2];
    scores<D>(klds, qf, lane, s);
    float v[8];
    float tmax = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = key0 + 8 * g + 4 * mt + e;
        const bool vis = row_ok && visible(si, t, jj);
        const float x = vis ? s[mt][e] * a.scale_log2 : kNegInf;
        v[mt * 4 + e] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    float pv[8];
    float alpha = 1.f, rs = 0.f;
    if (mnew == kNegInf) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = 0.f;
    } else {
      alpha = exp2f(m - mnew);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = v[e] == kNegInf ? 0.f : exp2f(v[e] - mnew);
        rs += pv[e];
      }
    }
    rs += shfl_xor(rs, 16);
    rs += shfl_xor(rs, 32);
    l = l * alpha + rs;
    m = mnew;
    u32x4 pb;
    pb[0] = pack_bf16x2(pv[0], pv[1]);
    pb[1] = pack_bf16x2(pv[2], pv[3]);
    pb[2] = pack_bf16x2(pv[4], pv[5]);
    pb[3] = pack_bf16x2(pv[6], pv[7]);
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) {
      o[dm] *= alpha;
      u32x4 vf = ld16(&vt[16 * dm + j][8 * g]);
      o[dm] = mfma16(vf, pb, o[dm]);
    }
    __syncthreads();
  }

  if (!row_ok) return;
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

// Merge KV-split partials: one thread per (row, head, 4 features).
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, AttnPlan p) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t rh = idx / (D / 4);
  const int d4 = (int)(idx % (D / 4)) * 4;
  if (rh >= (size_t)a.rows * a.c.H) return;
  const float *po = reinterpret_cast<const float *>(a.ws + p.off_part_o);
  const float *pml = reinterpret_cast<const float *>(a.ws + p.off_part_ml);
  const size_t stride = (size_t)a.rows * a.c.H;
  float mx = kNegInf;
  for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, pml[2 * (s * stride + rh)]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (mx != kNegInf) {
    for (int s = 0; s < p.splits; ++s) {
      const size_t k = s * stride + rh;
      const float ms = pml[2 * k];
      if (ms == kNegInf) continue;
      const float f = exp2f(ms - mx);
      l += pml[2 * k + 1] * f;
      acc += *reinterpret_cast<const f32x4 *>(po + k * D + d4) * f;
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  *reinterpret_cast<f32x4 *>(a.out + rh * D + d4) = acc * inv;
  if (p.mass_splits && d4 == 0) {
    float *lse = reinterpret_cast<float *>(a.ws + p.off_lse);
    lse[rh] = l > 0.f ? mx + log2f(l) : kNegInf;
  }
}

// Attention mass pass: one workgroup per (sequence, head, key chunk).
template <int D>
__global__ __launch_bounds__(256) void attn_mass_kernel(AttnArgs a, AttnPlan p) {
  constexpr int MAXK = 32 * KT;  // keys per chunk (bounded by the host plan)
  __shared__ uint16_t klds[KT][D + 8];
  __shared__ float wsum[4][KT];
  __shared__ float macc[MAXK];

  int u = blockIdx.x;
  const int chunk = u % p.mass_splits; u /= p.mass_splits;
  const int h = u % a.c.H;
  const int b = u / a.c.H;
  const SeqInfo si = seq_info(a, b);
  const int tiles = (si.L + KT - 1) / KT;
  const int tpc = (tiles + p.mass_splits - 1) / p.mass_splits;
  const int tb = chunk * tpc, te = min(tiles, tb + tpc);
  if (tb >= te) return;
  const int nkeys = (te - tb) * KT;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const float *lse = reinterpret_cast<const float *>(a.ws + p.off_lse);

  for (int k = threadIdx.x; k < nkeys; k += blockDim.x) macc[k] = 0.f;

  const int nrt = (si.nrows + 63) / 64;
  for (int rt = 0; rt < nrt; ++rt) {
    const int t = rt * 64 + wave * 16 + j;
    const bool row_ok = t < si.nrows;
    const int r = si.r0 + (row_ok ? t : 0);
    u32x4 qf[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[ks] = row_ok ? ld16(a.q + ((size_t)r * a.c.H + h) * D + 32 * ks + 8 * g)
                      : u32x4{0u, 0u, 0u, 0u};
    const float lr = row_ok ? lse[(size_t)r * a.c.H + h] : kNegInf;

    for (int tile = tb; tile < te; ++tile) {
      const int key0 = tile * KT;
      stage_tile<D>(a, b, h, key0, klds, nullptr, false);
      __syncthreads();
      f32x4 s[2];
      scores<D>(klds, qf, lane, s);
      float pv[8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = key0 + 8 * g + 4 * mt + e;
          const bool vis = row_ok && lr != kNegInf && visible(si, t, jj);
          pv[mt * 4 + e] = vis ? exp2f(s[mt][e] * a.scale_log2 - lr) : 0.f;
        }
      // Reduce over the 16 rows of the wave (lanes sharing g): reduce-scatter.
      const int b3 = (j >> 3) & 1, b2 = (j >> 2) & 1, b1 = (j >> 1) & 1;
      float q4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float give = b3 ? pv[i] : pv[i + 4];
        const float keep = b3 ? pv[i + 4] : pv[i];
        q4[i] = keep + shfl_xor(give, 8);
      }
      float q2[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float give = b2 ? q4[i] : q4[i + 2];
        const float keep = b2 ? q4[i + 2] : q4[i];
        q2[i] = keep + shfl_xor(give, 4);
      }
      float q1;
      {
        const float give = b1 ? q2[0] : q2[1];
        const float keep = b1 ? q2[1] : q2[0];
        q1 = keep + shfl_xor(give, 2);
      }
      // Lanes l and l^1 now hold the same key; add them in a fixed order.
      const float other = shfl_xor(q1, 1);
      const float tot = (j & 1) ? other + q1 : q1 + other;
      if ((j & 1) == 0) wsum[wave][8 * g + 4 * b3 + 2 * b2 + b1] = tot;
      __syncthreads();
      if (threadIdx.x < KT) {
        const int k = threadIdx.x;
        const float sum = ((wsum[0][k] + wsum[1][k]) + wsum[2][k]) + wsum[3][k];
        macc[(tile - tb) * KT + k] += sum;
      }
      __syncthreads();
    }
  }
  float *mp = reinterpret_cast<float *>(a.ws + p.off_mass_part) +
              ((size_t)b * a.c.H + h) * a.mass_stride;
  for (int k = threadIdx.x; k < nkeys; k += blockDim.x) {
    const int jj = tb * KT + k;
    if (jj < si.L) mp[jj] = macc[k];
  }
}

// mass[b][j] = sum over heads (in head order) of the per-head partials.
__global__ __launch_bounds__(256) void mass_head_reduce_kernel(AttnArgs a, AttnPlan p) {
  const int b = blockIdx.y;
  const int jj = blockIdx.x * blockDim.x + threadIdx.x;
  if (jj >= a.mass_stride) return;
  const int L = a.kv_len[b];
  float sum = 0.f;
  if (jj < L) {
    const float *mp = reinterpret_cast<const float *>(a.ws + p.off_mass_part) +
                      (size_t)b * a.c.H * a.mass_stride + jj;
    for (int h = 0; h < a.c.H; ++h) sum += mp[(size_t)h * a.mass_stride];
  }
  a.mass[(size_t)b * a.mass_stride + jj] = sum;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

AttnPlan plan_attention(int batch, int rows, int H, int D, int max_kv_len,
                        int max_rows_per_seq, int mass_stride) {
  AttnPlan p{};
  p.row_tiles = max(1, (max_rows_per_seq + 63) / 64);
  const int max_tiles = max(1, (max_kv_len + KT - 1) / KT);
  const long base = (long)batch * p.row_tiles * H;
  int splits = (int)((512 + base - 1) / max(base, 1L));
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

hipError_t launch_attention(const AttnArgs &a, const AttnPlan &p, hipStream_t s) {
  const int units = a.batch * p.row_tiles * a.c.H * p.splits;
  if (a.c.D == 128) {
    hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(units), dim3(256), 0, s, a, p);
  } else {
    hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(units), dim3(256), 0, s, a, p);
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
  if (p.mass_splits) {
    const int mu = a.batch * a.c.H * p.mass_splits;
    if (a.c.D == 128)
      hipLaunchKernelGGL(attn_mass_kernel<128>, dim3(mu), dim3(256), 0, s, a, p);
    else
      hipLaunchKernelGGL(attn_mass_kernel<64>, dim3(mu), dim3(256), 0, s, a, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dim3 grid((a.mass_stride + 255) / 256, a.batch);
    hipLaunchKernelGGL(mass_head_reduce_kernel, grid, dim3(256), 0, s, a, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fdl
