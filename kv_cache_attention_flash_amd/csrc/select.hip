// Tracking-set selection (top-B most-attended keys) and the Flash-Verify accept
// scan, for gfx950.
//
// Sources: [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for
// Fast, Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary),
// para 2 (a fixed budget of the most-attended tokens is kept and updated),
// para 3 (accept while both views agree and the mask-view confidence exceeds
// the threshold, in causal order, stopping at the first mismatch).
#include "device_common.h"
#include "internal.h"

namespace fdl {

namespace {

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (ALU
// latency, no LDS round trips): shifts by 1, 2, 4, 8 inside each row of 16
// lanes, then row 0's total into row 1 and row 2's into row 3 (broadcast of
// lane 15), then lane 31's running total into rows 2 and 3.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned v) {
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// One workgroup of NT threads per sequence (1024 for long rows, so a few
// sequences still keep many waves busy; 512 otherwise).  Masses are non-negative, so their
// fp32 bit patterns order like the values: a 4-pass radix select over 8-bit
// digits finds the bit pattern T of the B-th largest mass; every key above T
// is taken, and keys equal to T are taken in index order until B are chosen.
// Each pass costs one barrier: the four LDS histograms are zeroed up front,
// and after a pass every wave reads the whole histogram (four bins a lane,
// from the top digit down) and finds the digit with a DPP wave scan of its
// own.  The chosen indices are written in ascending order: each wave counts
// its segment's keys, one barrier shares the counts, and each wave places its
// segment's keys 64 at a time with ballots.  Rows of up to kCached keys (by
// stride) are held in LDS across the passes.
constexpr int kCached = 8192;

template <int NT>
__global__ __launch_bounds__(NT) void topb_kernel(const float *mass, int stride,
                                                  const int32_t *kv_len, int topb,
                                                  int32_t *out) {
  constexpr int NW = NT / 64;
  static_assert(NT >= 256 && NT % 64 == 0, "whole waves, 256+ threads");
  __shared__ unsigned hist[4][256];
  __shared__ unsigned seg_eq[NW], seg_gt[NW];
  __shared__ uint32_t cache[kCached];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t *mb = reinterpret_cast<const uint32_t *>(mass + (size_t)b * stride);
  // The row's loads go out with the length's (the stride bounds them).
  const bool cached = stride <= kCached;
  if (cached)
    for (int k = tid; k < stride; k += NT) cache[k] = mb[k];
  for (int i = tid; i < 4 * 256; i += NT) (&hist[0][0])[i] = 0u;
  const int L = min(kv_len[b], stride);  // a length past the row stride is clamped
  int32_t *ob = out + (size_t)b * topb;

  if (L <= topb) {
    for (int k = tid; k < topb; k += NT) ob[k] = k < L ? k : -1;
    return;
  }
  auto key = [&](int k) -> uint32_t { return cached ? cache[k] : mb[k]; };
  __syncthreads();

  uint32_t prefix = 0, pmask = 0;
  unsigned remaining = (unsigned)topb;  // keys still to take below the digits fixed so far
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int k = tid; k < L; k += NT) {
      const uint32_t u = key(k);
      if ((u & pmask) == prefix) atomicAdd(&hist[pass][(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    // Lane l holds digits 255-4l .. 252-4l; `incl` counts candidates with a
    // digit at or above its lowest one.  The digit holding the remaining-th
    // largest candidate lies in the one lane where the count crosses.
    unsigned c[4], lsum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = hist[pass][255 - 4 * lane - i];
      lsum += c[i];
    }
    const unsigned incl = wave_incl_scan(lsum);
    const unsigned excl = incl - lsum;
    // Exactly one lane crosses (the candidates number at least `remaining`);
    // the clamp keeps the lane index valid whatever the counts.
    const int src =
        max(0, __ffsll((long long)__ballot(excl < remaining && incl >= remaining)) - 1);
    unsigned digit = 0, rem = 0, cum = excl;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!found && cum + c[i] >= remaining) {
        digit = 255u - 4u * lane - i;
        rem = remaining - cum;
        found = true;
      }
      cum += c[i];
    }
    digit = (unsigned)__builtin_amdgcn_readlane((int)digit, src);
    rem = (unsigned)__builtin_amdgcn_readlane((int)rem, src);
    prefix |= digit << shift;
    pmask |= 255u << shift;
    remaining = rem;
  }
  const uint32_t T = prefix;

  // `remaining` keys equal to T are taken (lowest indices first) after every
  // key above T.  Wave w owns a contiguous segment of keys: it counts its
  // keys above and equal to T, the counts of the waves before it give its
  // first output position, and it places its chosen keys 64 at a time.
  const int w = tid >> 6;
  const int seg = (L + NW * 64 - 1) / (NW * 64) * 64;
  const int s0 = min(w * seg, L), s1 = min(s0 + seg, L);
  unsigned weq = 0, wgt = 0;
  for (int c0 = s0; c0 < s1; c0 += 64) {
    const int k = c0 + lane;
    const uint32_t u = k < s1 ? key(k) : 0u;
    weq += __popcll(__ballot(k < s1 && u == T));
    wgt += __popcll(__ballot(k < s1 && u > T));
  }
  if (lane == 0) {
    seg_eq[w] = weq;
    seg_gt[w] = wgt;
  }
  __syncthreads();
  unsigned eq_seen = 0, gt_before = 0;
  for (int ww = 0; ww < w; ++ww) {
    eq_seen += seg_eq[ww];
    gt_before += seg_gt[ww];
  }
  int sel_seen = (int)(gt_before + min(eq_seen, remaining));
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int c0 = s0; c0 < s1 && sel_seen < topb; c0 += 64) {
    const int k = c0 + lane;
    const uint32_t u = k < s1 ? key(k) : 0u;
    const bool eq = k < s1 && u == T;
    const unsigned long long beq = __ballot(eq);
    const bool sel = (k < s1 && u > T) || (eq && eq_seen + __popcll(beq & below) < remaining);
    const unsigned long long bsel = __ballot(sel);
    const int pos = sel_seen + __popcll(bsel & below);
    if (sel && pos < topb) ob[pos] = k;
    eq_seen += __popcll(beq);
    sel_seen += __popcll(bsel);
  }
}

// One wave per sequence: ballot the pass/fail flags 64 positions at a time and
// stop at the first failure.
__global__ __launch_bounds__(256) void verify_kernel(const int32_t *draft, const int32_t *mask,
                                                     const float *conf, int batch, int window,
                                                     float thr, int32_t *out) {
  const int lane = threadIdx.x & 63;
  const int seq = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seq >= batch) return;
  const size_t row = (size_t)seq * window;
  int len = window;
  for (int base = 0; base < window; base += 64) {
    const int k = base + lane;
    bool ok = true;
    if (k < window) ok = draft[row + k] == mask[row + k] && conf[row + k] > thr;
    const unsigned long long fails = ~__ballot(ok);
    if (fails) {
      len = base + __ffsll((long long)fails) - 1;
      break;
    }
  }
  if (lane == 0) out[seq] = len;
}

}  // namespace

hipError_t launch_topb(const float *mass, int stride, const int32_t *kv_len, int batch,
                       int topb, int32_t *out, hipStream_t s) {
  // Widths measured under rocprofv3 on the masses of the layer shapes: rows
  // of 4096 keys 9.98 / 11.32 / 16.31 us with 1024 / 512 / 256 threads; rows
  // of 512-1024 keys (batch 32) 6.18 / 6.00 / 7.01 us, of 768 keys (batch 1)
  // 4.63 / 4.58 / 5.25 us.
  if (stride > 2048)
    hipLaunchKernelGGL(topb_kernel<1024>, dim3(batch), dim3(1024), 0, s, mass, stride, kv_len,
                       topb, out);
  else
    hipLaunchKernelGGL(topb_kernel<512>, dim3(batch), dim3(512), 0, s, mass, stride, kv_len, topb,
                       out);
  return hipGetLastError();
}

hipError_t launch_verify(const int32_t *draft, const int32_t *mask, const float *conf,
                         int batch, int window, float thr, int32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(verify_kernel, dim3((batch + 3) / 4), dim3(256), 0, s, draft, mask, conf,
                     batch, window, thr, out);
  return hipGetLastError();
}

}  // namespace fdl
