// Single-launch decode step for gfx950: Flash-Cache (QKV projection, rotary
// embedding, cache write) then scheduled attention with the attention mass,
// in one persistent launch.
//
// Source: [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for
// Fast, Memory-Efficient Diffusion LLMs" (ai4snews.wisdomeyes.cn summary),
// para 1 (the fused cache kernel is combined with scheduled attention) and
// para 3 (the verify mask sits inside the fused kernel).
//
// The unit compiles the projection and attention files for their workgroup
// bodies (FDL_DEVICE_ONLY leaves their own launchers out), so each item runs
// the code of the separate calls.  The projection's column groups are formed
// per XCD here, so a split-K group adds its K chunks in another order than the
// separate kernel's group holding the same pairs: Q, K and V agree with the
// separate calls up to that fp32 reassociation (bitwise for the tiled
// projection, whose order does not depend on the tile), and every call gives
// bitwise the same results as the last.
//
// Items are dealt to the XCDs by head: XCD x owns heads x, x + 8, x + 16, ...
// Its queue holds the projection items that compute those heads' Q, K and V
// features (XcdPairMap gives each XCD a contiguous local pair space, head by
// head), then the row-group attention items of those heads.  A
// workgroup reads the XCD it runs on from the hardware (XCC_ID) and takes
// items from that XCD's ticket counter, so producer and consumer of every
// hand-off share one L2: a projection item completes its stores (they are
// in that L2 once the memory counter drains) and counts itself into each head
// it covers; an attention item polls its head's count, invalidates its CU's
// L1 and reads Q and the written K/V from the shared L2.  No L2 is written
// back or invalidated on the way, and an attention item starts as soon as its
// own head is projected.  The mass items sum over every head, so they cross
// XCDs: the last attention item of each XCD writes its L2 back once (a
// device-scope release), and a mass item starts after every XCD has done so
// (a device-scope acquire).
// Every item only waits for items with lower tickets in its own queue (or,
// for the mass, for queues whose items are all claimed by running
// workgroups), so the ordinary launch needs no co-residency guarantee.
// Every wait is bounded: past the bound it sets the error word and goes on.
// The last workgroup to leave resets the counters for the next call.
#include <algorithm>

#define FDL_DEVICE_ONLY 1
#include "flash_cache.hip"
#include "attention.hip"
#undef FDL_DEVICE_ONLY

namespace fdl {

namespace {

constexpr int kFusedThreads = 512;
constexpr int kSpinLimit = 1 << 20;  // ~1 s of polling: far beyond any item
constexpr int kXcds = 8;             // XCDs of the part (XCC_ID 0..7)
// Counter words at the start of the workspace.
constexpr int kMassTicket = 0, kXcdsDone = 1, kExitCount = 2, kErrorWord = 3;
constexpr int kTicket0 = 4;     // one ticket per XCD
constexpr int kAttDone0 = 12;   // attention items finished, per XCD
constexpr int kHeadReady0 = 20; // projection items finished, per head
// The counters live in the workspace's first kFusedSyncBytes bytes.
constexpr int kFusedMaxHeads = (int)(kFusedSyncBytes / 4) - kHeadReady0;
static_assert(kErrorWord * 4 == 12, "the error word sits at byte 12");

// The XCD the workgroup runs on (the hardware register XCC_ID, bits 0..3).
__device__ __forceinline__ int this_xcd() {
  return (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (kXcds - 1));
}

// Local pair space of the XCDs: XCD x owns the pairs [x span, (x + 1) span),
// head by head (its j-th head is x + 8 j), each head's Q, K and V pairs in
// section order; indices past the XCD's heads map past the last pair.
struct XcdPairMap {
  static constexpr bool kIdentity = false;
  int H, half, span, total;
  __device__ int operator()(int p) const {
    const int x = p / span, lp = p - x * span;
    const int per = 3 * half;
    const int j = lp / per, rem = lp - j * per;
    const int h = x + kXcds * j;
    if (h >= H) return total;
    const int sec = rem / half;
    return (sec * H + h) * half + (rem - sec * half);
  }
};
// Column units of cpw pairs per XCD (enough for XCD 0, which owns the most heads).
inline int xcd_units(int H, int D, int cpw) {
  return ((H + kXcds - 1) / kXcds * 3 * (D / 2) + cpw - 1) / cpw;
}

// Shape of the XCD queues: column units of CPW pairs (split-K column groups
// or tiled-projection column tiles), NRU row units each.
struct XcdQueues {
  int H, half, cpw, nru, cpx, batch, rgroups;
  __device__ int heads(int x) const { return H > x ? (H - 1 - x) / kXcds + 1 : 0; }
  __device__ int nproj(int x) const { return (heads(x) * 3 * half + cpw - 1) / cpw * nru; }
  __device__ int natt(int x) const { return heads(x) * batch * rgroups; }
  // projection items (of any queue) that cover local head j
  __device__ int head_items(int j) const {
    const int per = 3 * half;
    return ((j + 1) * per - 1) / cpw - j * per / cpw + 1;
  }
};

// Producer side of an XCD-local hand-off: every wave's stores have reached
// the L2 (the vector memory counter covers stores) before the count.
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
}

// Consumer side: the invalidate completes (it counts as a vector memory
// operation) before the barrier that lets the workgroup's loads go.
__device__ __forceinline__ void invalidate_l1() {
  asm volatile("buffer_inv sc0\n\ts_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ bool poll_until(int *counter, int target, int *error) {
  int spins = 0;
  while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (++spins > kSpinLimit) {
      __hip_atomic_store(error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  return true;
}

// KIND: 0 split-K projection with 16 chunks (hidden 4096), 1 split-K with a
// run-time chunk count, 2 tiled projection (more than 64 rows).  One kind per
// instantiation keeps the register peak at that of the separate kernels.
template <int D, int MAXT, int KIND>
__global__ __launch_bounds__(kFusedThreads) void fused_step_kernel(FlashCacheArgs fa, SplitPlan sp,
                                                                   int nrow_tiles, XcdQueues xq,
                                                                   AttnArgs aa, AttnPlan ap,
                                                                   int *sync) {
  static_assert(kSplitWaves * 64 == kFusedThreads, "split-K workgroup size");
  union Lds {
    SplitLds<kSplitNTW, kSplitNGW, kSplitKC> split;
    GemmLds<128, 4> gemm;
    RowsLds<D> rows;
    float mass[2][8][32];
  };
  __shared__ Lds lds;
  __shared__ int s_ticket;
  int *error = sync + kErrorWord;
  const int x = this_xcd();
  const int nproj = xq.nproj(x), natt = xq.natt(x), nown = nproj + natt;
  const int per = 3 * xq.half;
  const XcdPairMap pmap{xq.H, xq.half, xq.cpx * xq.cpw, 3 * xq.H * xq.half};
  const int unit_rows = xq.batch * xq.rgroups;  // attention items per head

  // This XCD's items: projection units (local column unit, row unit), then
  // the attention items of its heads, head by head.
  for (;;) {
    __syncthreads();  // the previous item is done with s_ticket and the LDS
    if (threadIdx.x == 0)
      s_ticket = __hip_atomic_fetch_add(sync + kTicket0 + x, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int it = s_ticket;
    if (it >= nown) break;
    if (it < nproj) {
      const int lct = it / xq.nru, rt = it % xq.nru;
      const int ct = x * xq.cpx + lct;  // global column unit
      if constexpr (KIND == 0)
        qkv_splitk_body<kSplitNTW, kSplitNGW, kSplitNST, 16, kSplitWaves, kSplitKC>(
            fa, sp, ct, lds.split, pmap);
      else if constexpr (KIND == 1)
        qkv_splitk_body<kSplitNTW, kSplitNGW, kSplitNST, 0, kSplitWaves, kSplitKC>(
            fa, sp, ct, lds.split, pmap);
      else
        qkv_gemm_body<128, 4, 2>(fa, nrow_tiles, 0, ct * nrow_tiles + rt, lds.gemm, pmap);
      stores_done();
      if (threadIdx.x == 0) {
        const int lo = lct * xq.cpw, hi = min(lo + xq.cpw, xq.heads(x) * per) - 1;
        for (int j = lo / per; j <= hi / per; ++j)
          __hip_atomic_fetch_add(sync + kHeadReady0 + x + kXcds * j, 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      const int ai = it - nproj;
      const int j = ai / unit_rows, rem = ai % unit_rows;
      const int h = x + kXcds * j, b = rem / xq.rgroups, rg = rem % xq.rgroups;
      if (threadIdx.x == 0) {
        poll_until(sync + kHeadReady0 + h, xq.head_items(j) * xq.nru, error);
        // Q and the written K/V are in this XCD's L2; drop any copy in the
        // CU's L1 before reading them.
        invalidate_l1();
      }
      __syncthreads();
      attn_rows_body<D, MAXT, true>(aa, ap, (b * xq.H + h) * xq.rgroups + rg, 1, lds.rows);
      stores_done();
      if (threadIdx.x == 0) {
        const int n = __hip_atomic_fetch_add(sync + kAttDone0 + x, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        if (n == natt - 1) {
          // The XCD's last attention item: write its L2 back once for the
          // mass items on the other XCDs.
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          __hip_atomic_fetch_add(sync + kXcdsDone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  // Mass items (two per workgroup, one per 256-thread half), from one shared
  // ticket, once every XCD with attention items has released them.
  const int nmass = aa.batch * ((aa.mass_stride + 31) / 32);
  const int npair = (nmass + 1) / 2;
  const int xcds_att = unit_rows > 0 ? min(kXcds, xq.H) : 0;
  bool waited = false;
  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0)
      s_ticket = __hip_atomic_fetch_add(sync + kMassTicket, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int it = s_ticket;
    if (it >= npair) break;
    if (!waited) {
      if (threadIdx.x == 0) {
        poll_until(sync + kXcdsDone, xcds_att, error);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // the invalidate done before the barrier
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
      }
      __syncthreads();
      waited = true;
    }
    const int half = threadIdx.x >> 8;
    const int item = 2 * it + half;
    attn_rows_mass_body(aa, ap, item, threadIdx.x & 255, item < nmass, lds.mass[half]);
  }

  // The last workgroup out (every other one has claimed its final tickets and
  // is past all of its waits) resets the counters for the next call.  The
  // counters are only ever touched by device-scope atomics, and a workgroup's
  // count follows its last ticket (whose value it used), so the count needs
  // no fence: a fence per workgroup would write its XCD's L2 back each time.
  // The kernel's end publishes the results and the reset.
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const int n = __hip_atomic_fetch_add(sync + kExitCount, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    s_last = n == (int)gridDim.x - 1;
  }
  __syncthreads();
  if (s_last) {
    for (int i = threadIdx.x; i < kHeadReady0 + xq.H; i += kFusedThreads)
      if (i != kErrorWord && i != kExitCount)
        __hip_atomic_store(sync + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(sync + kExitCount, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Resident workgroups of one instantiation on the current device (cached):
// more would only claim the final ticket and leave.
template <int D, int MAXT, int KIND>
int fused_capacity() {
  static int cap[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cap[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(&fused_step_kernel<D, MAXT, KIND>),
            kFusedThreads,
            0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cap[dev] = per_cu * cus;
  }
  return cap[dev];
}

template <int D, int MAXT, int KIND>
hipError_t launch_fused_inst(FlashCacheArgs fa, SplitPlan sp, int nrow, const XcdQueues &xq,
                             AttnArgs aa, AttnPlan ap, int *sync, hipStream_t s) {
  const int cap = fused_capacity<D, MAXT, KIND>();
  if (cap <= 0) return hipErrorInvalidConfiguration;
  // Every CU gets a workgroup (the XCDs' queues are served by the workgroups
  // dispatched to them).
  hipLaunchKernelGGL((fused_step_kernel<D, MAXT, KIND>), dim3(std::max(cap, kXcds)),
                     dim3(kFusedThreads), 0, s, fa, sp, nrow, xq, aa, ap, sync);
  return hipGetLastError();
}

template <int D, int KIND>
hipError_t launch_fused_d(FlashCacheArgs fa, SplitPlan sp, int nrow, const XcdQueues &xq,
                          AttnArgs aa, AttnPlan ap, int *sync, hipStream_t s) {
  if (ap.maxt == 1) return launch_fused_inst<D, 1, KIND>(fa, sp, nrow, xq, aa, ap, sync, s);
  if (ap.maxt == 2) return launch_fused_inst<D, 2, KIND>(fa, sp, nrow, xq, aa, ap, sync, s);
  return launch_fused_inst<D, 4, KIND>(fa, sp, nrow, xq, aa, ap, sync, s);
}

}  // namespace

bool fused_step_supported(const FlashCacheArgs &fa, const AttnPlan &ap, bool mass) {
  if (!mass || !ap.rows_path) return false;
  if (fa.c.H > kFusedMaxHeads) return false;  // one readiness counter per head
  const FcPlan fp = plan_fc(fa.rows, fa.hidden, fa.c.H, fa.c.D);
  if (!fp.splitk) return true;
  if (fp.S != 1) return false;
  const int nch = fa.hidden / kSplitKC;
  return nch == 16 || (nch != 4 && nch != 8 && nch != 32);
}

hipError_t launch_fused_step(const FlashCacheArgs &fa, const AttnArgs &aa, const AttnPlan &ap,
                             int *sync, hipStream_t s) {
  const FcPlan fp = plan_fc(fa.rows, fa.hidden, fa.c.H, fa.c.D);
  SplitPlan sp{};
  int kind = 2, nrow = 0;
  XcdQueues xq{};
  xq.H = fa.c.H;
  xq.half = fa.c.D / 2;
  xq.batch = aa.batch;
  xq.rgroups = ap.rgroups;
  if (fp.splitk) {
    sp.G = fp.G;
    sp.S = 1;
    sp.ks = fa.hidden;
    sp.partials = nullptr;
    kind = fa.hidden / kSplitKC == 16 ? 0 : 1;
    xq.cpw = kSplitCW / 2;  // pairs per split-K column group
    xq.nru = 1;
  } else {
    nrow = (fa.rows + 127) / 128;
    xq.cpw = 128;  // pairs per column tile of qkv_gemm_body<128, 4, ...>
    xq.nru = nrow;
  }
  xq.cpx = xcd_units(xq.H, fa.c.D, xq.cpw);
  const bool d128 = aa.c.D == 128;
  if (kind == 0)
    return d128 ? launch_fused_d<128, 0>(fa, sp, nrow, xq, aa, ap, sync, s)
                : launch_fused_d<64, 0>(fa, sp, nrow, xq, aa, ap, sync, s);
  if (kind == 1)
    return d128 ? launch_fused_d<128, 1>(fa, sp, nrow, xq, aa, ap, sync, s)
                : launch_fused_d<64, 1>(fa, sp, nrow, xq, aa, ap, sync, s);
  return d128 ? launch_fused_d<128, 2>(fa, sp, nrow, xq, aa, ap, sync, s)
              : launch_fused_d<64, 2>(fa, sp, nrow, xq, aa, ap, sync, s);
}

}  // namespace fdl
