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
// bodies (FDL_DEVICE_ONLY leaves their own launchers out), so each phase runs
// exactly the code of the separate calls: the results are bitwise theirs.
// Items: every projection item, then the row-group attention items (each
// waits until all projection items are done), then the mass items (each waits
// until all attention items are done).  A workgroup takes its next item from
// a ticket counter, so the items are claimed in that order: an item only ever
// waits for items with lower tickets, which are held by running workgroups
// that do not wait for it, and the launch needs no co-residency guarantee
// (an ordinary launch, not a cooperative one).  Hand-offs cross XCDs (each
// has its own L2): a workgroup's items end with a device-scope release (the
// writes leave its L2) and a count; a waiting workgroup polls the count, then
// acquires at device scope (its caches are invalidated before it reads).
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
constexpr int kSpinLimit = 1 << 20;  // ~1 s of polling: far beyond any phase

__device__ __forceinline__ void phase_signal(int *counter) {
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls with relaxed device-scope loads (an acquiring poll would invalidate
// the XCD's L2 on every try, under the workgroups still streaming through
// it), then one acquire fence once the count is reached.
__device__ __forceinline__ void phase_wait(int *counter, int target, int *error) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++spins > kSpinLimit) {
        __hip_atomic_store(error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// KIND: 0 split-K projection with 16 chunks (hidden 4096), 1 split-K with a
// run-time chunk count, 2 tiled projection (more than 64 rows).  One kind per
// instantiation keeps the register peak at that of the separate kernels.
template <int D, int MAXT, int KIND>
__global__ __launch_bounds__(kFusedThreads) void fused_step_kernel(FlashCacheArgs fa, SplitPlan sp,
                                                                   int nrow_tiles, int ncol_tiles,
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
  int *proj_done = sync, *attn_done = sync + 1, *exit_count = sync + 2, *error = sync + 3;
  int *ticket = sync + 4;

  const int nproj = KIND == 2 ? nrow_tiles * ncol_tiles : sp.G * sp.S;
  const int natt = aa.batch * aa.c.H * ap.rgroups;
  const int nmass = aa.batch * ((aa.mass_stride + 31) / 32);
  const int npair = (nmass + 1) / 2;  // mass items two at a time, one per 256-thread half
  const int total = nproj + natt + npair;
  bool waited_proj = false, waited_attn = false;
  for (;;) {
    __syncthreads();  // the previous item is done with s_ticket and the LDS
    if (threadIdx.x == 0)
      s_ticket = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int it = s_ticket;
    if (it >= total) break;
    if (it < nproj) {
      if constexpr (KIND == 0)
        qkv_splitk_body<kSplitNTW, kSplitNGW, kSplitNST, 16, kSplitWaves, kSplitKC>(fa, sp, it,
                                                                                   lds.split);
      else if constexpr (KIND == 1)
        qkv_splitk_body<kSplitNTW, kSplitNGW, kSplitNST, 0, kSplitWaves, kSplitKC>(fa, sp, it,
                                                                                  lds.split);
      else
        qkv_gemm_body<128, 4, 2>(fa, nrow_tiles, ncol_tiles, it, lds.gemm);
      phase_signal(proj_done);
    } else if (it < nproj + natt) {
      if (!waited_proj) phase_wait(proj_done, nproj, error);
      waited_proj = true;
      attn_rows_body<D, MAXT, true>(aa, ap, it - nproj, natt, lds.rows);
      phase_signal(attn_done);
    } else {
      if (!waited_attn) phase_wait(attn_done, natt, error);
      waited_attn = true;
      const int half = threadIdx.x >> 8;
      const int item = 2 * (it - nproj - natt) + half;
      attn_rows_mass_body(aa, ap, item, threadIdx.x & 255, item < nmass, lds.mass[half]);
    }
  }

  // The last workgroup out (every other one has claimed its final ticket and
  // is past all of its waits) resets the counters for the next call.
  if (threadIdx.x == 0) {
    const int n = __hip_atomic_fetch_add(exit_count, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (n == (int)gridDim.x - 1) {
      __hip_atomic_store(proj_done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(attn_done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(exit_count, 0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
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
hipError_t launch_fused_inst(FlashCacheArgs fa, SplitPlan sp, int nrow, int ncol, AttnArgs aa,
                             AttnPlan ap, int *sync, hipStream_t s) {
  const int nproj = KIND == 2 ? nrow * ncol : sp.G * sp.S;
  const int natt = aa.batch * aa.c.H * ap.rgroups;
  const int npair = (aa.batch * ((aa.mass_stride + 31) / 32) + 1) / 2;
  const int cap = fused_capacity<D, MAXT, KIND>();
  if (cap <= 0) return hipErrorInvalidConfiguration;
  const int grid = std::max(1, std::min(std::max(nproj, std::max(natt, npair)), cap));
  hipLaunchKernelGGL((fused_step_kernel<D, MAXT, KIND>), dim3(grid), dim3(kFusedThreads), 0, s,
                     fa, sp, nrow, ncol, aa, ap, sync);
  return hipGetLastError();
}

template <int D, int KIND>
hipError_t launch_fused_d(FlashCacheArgs fa, SplitPlan sp, int nrow, int ncol, AttnArgs aa,
                          AttnPlan ap, int *sync, hipStream_t s) {
  if (ap.maxt == 1) return launch_fused_inst<D, 1, KIND>(fa, sp, nrow, ncol, aa, ap, sync, s);
  if (ap.maxt == 2) return launch_fused_inst<D, 2, KIND>(fa, sp, nrow, ncol, aa, ap, sync, s);
  return launch_fused_inst<D, 4, KIND>(fa, sp, nrow, ncol, aa, ap, sync, s);
}

}  // namespace

bool fused_step_supported(const FlashCacheArgs &fa, const AttnPlan &ap, bool mass) {
  if (!mass || !ap.rows_path) return false;
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
  int kind = 2, nrow = 0, ncol = 0;
  if (fp.splitk) {
    sp.G = fp.G;
    sp.S = 1;
    sp.ks = fa.hidden;
    sp.partials = nullptr;
    kind = fa.hidden / kSplitKC == 16 ? 0 : 1;
  } else {
    const int total_pairs = 3 * fa.c.H * (fa.c.D / 2);
    nrow = (fa.rows + 127) / 128;
    ncol = (total_pairs + 127) / 128;
  }
  const bool d128 = aa.c.D == 128;
  if (kind == 0)
    return d128 ? launch_fused_d<128, 0>(fa, sp, nrow, ncol, aa, ap, sync, s)
                : launch_fused_d<64, 0>(fa, sp, nrow, ncol, aa, ap, sync, s);
  if (kind == 1)
    return d128 ? launch_fused_d<128, 1>(fa, sp, nrow, ncol, aa, ap, sync, s)
                : launch_fused_d<64, 1>(fa, sp, nrow, ncol, aa, ap, sync, s);
  return d128 ? launch_fused_d<128, 2>(fa, sp, nrow, ncol, aa, ap, sync, s)
              : launch_fused_d<64, 2>(fa, sp, nrow, ncol, aa, ap, sync, s);
}

}  // namespace fdl
