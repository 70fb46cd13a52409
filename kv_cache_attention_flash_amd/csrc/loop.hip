// Device-side planning of a multi-step decoding loop, for gfx950: the next
// step's active rows (sliding window plus tracked rows) and their hidden
// states, computed on the GPU from the previous step's top-B set and accept
// lengths, so the loop needs no host round trip between steps.
//
// Sources: [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for
// Fast, Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary),
// para 1 (caching and update stages alternate within a batch, so lengths
// diverge and a block table schedules them), para 2 (each step's queries are
// a sliding unmasking window plus a fixed budget of the most-attended tokens),
// para 3 (accepted tokens are committed in causal order).  The planning rules
// below are a reading of these passages (the pages give no loop in detail).
#include "device_common.h"
#include "internal.h"

namespace fdl {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// Per-sequence quantities every phase needs, recomputed from the inputs.
struct SeqPlan {
  int L, f, stage, w0, nwin;
};

// The commit and window rules for sequence b (uniform across the wave).
__device__ __forceinline__ SeqPlan seq_plan(const PlanArgs &a, int b) {
  SeqPlan s;
  s.L = max(0, a.kv_len[b]);
  int f = min(max(a.frontier[b], 0), s.L);
  if (a.step > 0 && f < s.L) {
    // At least one token per step (progress), at most the window's W.
    const int acc = min(max(a.accept_len[b], 0), a.window);
    f = min(s.L, f + max(1, acc));
  }
  s.f = f;
  if (f >= s.L) {
    s.stage = kStageDone;
    s.w0 = s.nwin = 0;
    return s;
  }
  const bool refresh = a.refresh_period > 0 && (a.step + b) % a.refresh_period == 0;
  s.stage = refresh ? kStageRefresh : kStageUpdate;
  // Refresh: the window starts at the block boundary at or below f.
  s.w0 = refresh ? f - f % a.block_size : f;
  s.nwin = min(s.w0 + a.window, s.L) - s.w0;
  return s;
}

// Walks sequence b's tracked entries 64 at a time.  An entry is kept when it
// lies in [0, L), outside the window and above every valid entry before it
// (a valid entry above all earlier ones is exactly one above every entry kept
// before it, so a running maximum over the valid entries decides).  Calls
// emit(lane_keeps, value, rank among kept entries) for each chunk; returns
// the number kept.
template <class Emit>
__device__ __forceinline__ int filter_tracked(const PlanArgs &a, int b, const SeqPlan &s,
                                              Emit emit) {
  const int lane = threadIdx.x & 63;
  const int32_t *tr = a.tracked + (size_t)b * a.topb;
  int run_max = -1, kept = 0;
  for (int c0 = 0; c0 < a.topb; c0 += 64) {
    const int i = c0 + lane;
    const int t = i < a.topb ? tr[i] : -1;
    const bool valid = t >= 0 && t < s.L && !(t >= s.w0 && t < s.w0 + s.nwin);
    // Exclusive running maximum of the valid entries, lane order.
    int m = valid ? t : -1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(m, o, 64);
      if (lane >= o) m = max(m, u);
    }
    int before = __shfl_up(m, 1, 64);
    before = lane == 0 ? run_max : max(before, run_max);
    const bool keep = valid && t > before;
    const unsigned long long bal = __ballot(keep);
    emit(keep, t, kept + __popcll(bal & ((1ull << lane) - 1ull)));
    kept += __popcll(bal);
    run_max = max(run_max, __shfl(m, 63, 64));
  }
  return kept;
}

// One workgroup plans the whole batch: (1) a wave per sequence counts its
// rows, (2) an exclusive scan over the batch gives cu_rows, (3) a wave per
// sequence writes its rows (window positions, then the kept tracked
// positions; slot = position), its stage and its new frontier.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int s_off[kPlanMaxBatch + 1];
  __shared__ int s_wsum[kPlanWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  for (int b = wave; b < a.batch; b += kPlanWaves) {
    const SeqPlan s = seq_plan(a, b);
    int n = s.nwin;
    if (s.stage != kStageDone) n += filter_tracked(a, b, s, [](bool, int, int) {});
    if (lane == 0) s_off[b] = n;
  }
  __syncthreads();

  // Exclusive scan of the counts: thread t sums a contiguous chunk.
  const int per = (a.batch + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(a.batch, (int)threadIdx.x * per), hi = min(a.batch, lo + per);
  int local = 0;
  for (int b = lo; b < hi; ++b) local += s_off[b];
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int base = incl - local;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
  __syncthreads();  // every count is read before it is overwritten
  for (int b = lo; b < hi; ++b) {
    const int n = s_off[b];
    s_off[b] = base;
    base += n;
  }
  if (threadIdx.x == kPlanThreads - 1) s_off[a.batch] = base;
  __syncthreads();
  if (threadIdx.x == 0) a.cu_rows[0] = 0;

  for (int b = wave; b < a.batch; b += kPlanWaves) {
    const SeqPlan s = seq_plan(a, b);
    const int r0 = s_off[b];
    for (int i = lane; i < s.nwin; i += 64) {
      a.positions[r0 + i] = s.w0 + i;
      a.slots[r0 + i] = s.w0 + i;
    }
    if (s.stage != kStageDone) {
      const int rt = r0 + s.nwin;
      filter_tracked(a, b, s, [&](bool keep, int t, int rank) {
        if (keep) {
          a.positions[rt + rank] = t;
          a.slots[rt + rank] = t;
        }
      });
    }
    if (lane == 0) {
      a.cu_rows[b + 1] = s_off[b + 1];
      if (a.stage) a.stage[b] = s.stage;
    }
  }
  // The frontier is read by every phase above; it is updated last.
  __syncthreads();
  for (int b = threadIdx.x; b < a.batch; b += kPlanThreads) {
    const SeqPlan s = seq_plan(a, b);
    a.frontier_out[b] = s.f;
  }
}

// Largest b with cu_rows[b] <= r.
__device__ __forceinline__ int seq_of_row(const int32_t *cu_rows, int batch, int r) {
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_rows[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// One wave per active row copies its hidden-state row (hidden bf16 values,
// 16 bytes per lane per load) from the committed-token table when the
// position lies below the sequence's frontier, else from the masked-token
// table.  Positions are clamped into the tables.
__global__ __launch_bounds__(256) void gather_hidden_kernel(GatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int act = max(0, min(a.rows, a.cu_rows[a.batch]));
  if (r >= act) return;
  const int b = seq_of_row(a.cu_rows, a.batch, r);
  const int p = min(max(a.positions[r], 0), a.max_len - 1);
  const uint16_t *tab = p < a.frontier[b] ? a.committed : a.masked;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(tab + ((size_t)b * a.max_len + p) * a.hidden);
  u32x4 *dst = reinterpret_cast<u32x4 *>(a.x_out + (size_t)r * a.hidden);
  const int chunks = a.hidden / 8;
  for (int c0 = 0; c0 < chunks; c0 += 64 * 4) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + 64 * i + lane;
      if (c < chunks) v[i] = src[c];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + 64 * i + lane;
      if (c < chunks) dst[c] = v[i];
    }
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather_hidden(const GatherArgs &a, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.rows + 3) / 4);
  if (blocks) hipLaunchKernelGGL(gather_hidden_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fdl
