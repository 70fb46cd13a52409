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

// Exclusive prefix count of `flag` over the block (in thread order) and the
// block total; NW waves.
template <int NW>
__device__ __forceinline__ int block_excl_count(bool flag, int &total, int *sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) sh[wave] = __popcll(bal);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = sh[w];
    before += w < wave ? c : 0;
    total += c;
  }
  __syncthreads();
  return before + in_wave;
}

// Inclusive prefix sum over the block's threads (thread order); NW waves.
template <int NW>
__device__ __forceinline__ unsigned block_incl_sum(unsigned v, unsigned *sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  unsigned before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) before += w < wave ? sh[w] : 0u;
  __syncthreads();
  return v + before;
}

// One workgroup of NT threads per sequence (1024 for long rows, so a few
// sequences still keep many waves busy).  Masses are non-negative, so their
// fp32 bit patterns order like the values: a 4-pass radix select over 8-bit
// digits (LDS histogram, then a parallel scan from the top digit down over
// the first 256 threads) finds the bit pattern T of the B-th largest mass;
// every key above T is taken, and keys equal to T are taken in index order
// until B are chosen.  A final in-order scan writes the chosen indices
// ascending.  Rows of up to kCached keys (by stride) are held in LDS across
// the passes.
constexpr int kCached = 8192;

template <int NT>
__global__ __launch_bounds__(NT) void topb_kernel(const float *mass, int stride,
                                                  const int32_t *kv_len, int topb,
                                                  int32_t *out) {
  constexpr int NW = NT / 64;
  static_assert(NT >= 256, "the digit scan needs one thread per bin");
  __shared__ unsigned hist[256];
  __shared__ unsigned s_digit, s_remaining;
  __shared__ unsigned shs[NW];
  __shared__ int sh[NW];
  __shared__ uint32_t cache[kCached];
  const int b = blockIdx.x;
  const uint32_t *mb = reinterpret_cast<const uint32_t *>(mass + (size_t)b * stride);
  // The row's loads go out with the length's (the stride bounds them).
  const bool cached = stride <= kCached;
  if (cached)
    for (int k = threadIdx.x; k < stride; k += NT) cache[k] = mb[k];
  const int L = min(kv_len[b], stride);  // a length past the row stride is clamped
  int32_t *ob = out + (size_t)b * topb;

  if (L <= topb) {
    for (int k = threadIdx.x; k < topb; k += NT) ob[k] = k < L ? k : -1;
    return;
  }
  auto key = [&](int k) -> uint32_t { return cached ? cache[k] : mb[k]; };

  uint32_t prefix = 0, pmask = 0;
  unsigned remaining = (unsigned)topb;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    __syncthreads();
    for (int k = threadIdx.x; k < L; k += NT) {
      const uint32_t u = key(k);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    // Thread t < 256 looks at digit 255 - t; cum = candidates with digit >= it.
    const unsigned c = threadIdx.x < 256 ? hist[255 - threadIdx.x] : 0u;
    const unsigned cum = block_incl_sum<NW>(c, shs);
    if (c > 0 && cum >= remaining && cum - c < remaining) {
      s_digit = 255u - threadIdx.x;
      s_remaining = remaining - (cum - c);
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    remaining = s_remaining;
    __syncthreads();
  }
  const uint32_t T = prefix;
  // `remaining` keys equal to T are needed (after all keys above T).
  int base_sel = 0, base_eq = 0;
  for (int c0 = 0; c0 < L; c0 += NT) {
    const int k = c0 + threadIdx.x;
    const uint32_t u = k < L ? key(k) : 0u;
    const bool gt = k < L && u > T;
    const bool eq = k < L && u == T;
    int eq_total, sel_total;
    const int eq_rank = base_eq + block_excl_count<NW>(eq, eq_total, sh);
    const bool sel = gt || (eq && eq_rank < (int)remaining);
    const int pos = base_sel + block_excl_count<NW>(sel, sel_total, sh);
    if (sel && pos < topb) ob[pos] = k;
    base_eq += eq_total;
    base_sel += sel_total;
    if (base_sel >= topb) break;
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
  if (stride > 2048)
    hipLaunchKernelGGL(topb_kernel<1024>, dim3(batch), dim3(1024), 0, s, mass, stride, kv_len,
                       topb, out);
  else
    hipLaunchKernelGGL(topb_kernel<256>, dim3(batch), dim3(256), 0, s, mass, stride, kv_len, topb,
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
