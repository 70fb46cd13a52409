// C ABI of libfdllm: host-side argument validation and kernel dispatch.  The
// declarations, with the page passages each call implements, are in
// include/fdllm.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "../../include/fdllm.h"
#include "internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FDL_OK;
  g_last_hip_error = (int)e;
  return FDL_EHIP;
}

bool block_size_ok(int bs) { return bs == 32 || bs == 64 || bs == 128 || bs == 256; }

int check_cache(const fdl_kv_cache *c, bool need_pools) {
  if (!c) return FDL_EINVAL;
  if (c->num_heads <= 0 || c->head_dim <= 0 || c->block_size <= 0 || c->num_blocks <= 0 ||
      c->max_blocks_per_seq <= 0)
    return FDL_EINVAL;
  if (!c->block_table) return FDL_EINVAL;
  if (need_pools && (!c->k_cache || !c->v_cache)) return FDL_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return FDL_EUNSUPPORTED;
  if (!block_size_ok(c->block_size)) return FDL_EUNSUPPORTED;
  if ((long)c->num_heads * c->head_dim > 16384) return FDL_EUNSUPPORTED;
  return FDL_OK;
}

fdl::CacheView view_of(const fdl_kv_cache *c) {
  fdl::CacheView v;
  v.H = c->num_heads;
  v.D = c->head_dim;
  v.bs = c->block_size;
  v.bs_shift = 0;
  while ((1 << v.bs_shift) < v.bs) ++v.bs_shift;  // block sizes are powers of two
  v.num_blocks = c->num_blocks;
  v.max_blocks = c->max_blocks_per_seq;
  v.k = static_cast<uint16_t *>(c->k_cache);
  v.v = static_cast<uint16_t *>(c->v_cache);
  v.block_table = c->block_table;
  return v;
}

// FDL_DEBUG=1 in the environment (read at every call): the calls that index
// the cache synchronise their stream, copy the index arrays to the host and
// refuse out-of-range or duplicate entries with FDL_EINVAL before launching.
bool debug_mode() {
  const char *e = std::getenv("FDL_DEBUG");
  return e && e[0] == '1' && e[1] == '\0';
}

// n int32 values of device memory into h (the stream already synchronised).
bool fetch_i32(std::vector<int32_t> &h, const int32_t *d, size_t n) {
  h.assign(n, 0);
  return n == 0 || hipMemcpy(h.data(), d, n * sizeof(int32_t), hipMemcpyDeviceToHost) == hipSuccess;
}

// Row offsets: cu[0] = 0, non-decreasing, cu[batch] <= num_rows.
int debug_check_cu(const std::vector<int32_t> &cu, int batch, int num_rows) {
  if (cu[0] != 0 || cu[batch] > num_rows) return FDL_EINVAL;
  for (int b = 0; b < batch; ++b)
    if (cu[b + 1] < cu[b]) return FDL_EINVAL;
  return FDL_OK;
}

// flash_cache_step's index arrays: non-negative positions; logical slots within
// the block table's row; block ids within the pool; no physical slot written
// twice.
int debug_check_rows(const fdl_kv_cache *c, int batch, int num_rows, const int32_t *cu_rows,
                     const int32_t *positions, const int32_t *slots, hipStream_t s) {
  if (hipStreamSynchronize(s) != hipSuccess) return FDL_EHIP;
  std::vector<int32_t> cu, pos, sl, bt;
  if (!fetch_i32(cu, cu_rows, (size_t)batch + 1)) return FDL_EHIP;
  int st = debug_check_cu(cu, batch, num_rows);
  if (st) return st;
  const int act = cu[batch];
  if (!fetch_i32(pos, positions, act) || !fetch_i32(sl, slots, act) ||
      !fetch_i32(bt, c->block_table, (size_t)batch * c->max_blocks_per_seq))
    return FDL_EHIP;
  const long span = (long)c->max_blocks_per_seq * c->block_size;
  std::vector<char> used((size_t)c->num_blocks * c->block_size, 0);
  for (int b = 0; b < batch; ++b)
    for (int r = cu[b]; r < cu[b + 1]; ++r) {
      if (pos[r] < 0 || sl[r] < 0 || sl[r] >= span) return FDL_EINVAL;
      const int blk = bt[(size_t)b * c->max_blocks_per_seq + sl[r] / c->block_size];
      if (blk < 0 || blk >= c->num_blocks) return FDL_EINVAL;
      char &u = used[(size_t)blk * c->block_size + sl[r] % c->block_size];
      if (u) return FDL_EINVAL;
      u = 1;
    }
  return FDL_OK;
}

// scheduled_attention's index arrays: row offsets, each sequence's row count
// within max_rows_per_seq, non-negative lengths, the block ids of every page a
// visible slot lies in, and the two-view descriptors' stated inequalities
// (window_start + window_len <= draft_slot_start, draft_slot_start +
// window_len <= kv_len, all non-negative).
int debug_check_attention(const fdl_kv_cache *c, int batch, int num_rows,
                          const int32_t *cu_rows, const int32_t *kv_len, int max_kv_len,
                          int max_rows_per_seq, const fdl_two_view *views, hipStream_t s) {
  if (hipStreamSynchronize(s) != hipSuccess) return FDL_EHIP;
  std::vector<int32_t> cu, kl, bt, vw;
  if (!fetch_i32(cu, cu_rows, (size_t)batch + 1) || !fetch_i32(kl, kv_len, batch) ||
      !fetch_i32(bt, c->block_table, (size_t)batch * c->max_blocks_per_seq))
    return FDL_EHIP;
  if (views && !fetch_i32(vw, reinterpret_cast<const int32_t *>(views), (size_t)batch * 3))
    return FDL_EHIP;
  int st = debug_check_cu(cu, batch, num_rows);
  if (st) return st;
  for (int b = 0; b < batch; ++b) {
    if (cu[b + 1] - cu[b] > max_rows_per_seq) return FDL_EINVAL;
    if (kl[b] < 0) return FDL_EINVAL;
    if (views) {
      const int w0 = vw[3 * b], wl = vw[3 * b + 1], d0 = vw[3 * b + 2];
      if (w0 < 0 || wl < 0 || d0 < 0) return FDL_EINVAL;
      if (wl > 0 && ((long)w0 + wl > d0 || (long)d0 + wl > kl[b])) return FDL_EINVAL;
    }
    const int L = kl[b] < max_kv_len ? kl[b] : max_kv_len;
    for (int p = 0; p < (L + c->block_size - 1) / c->block_size; ++p) {
      const int blk = bt[(size_t)b * c->max_blocks_per_seq + p];
      if (blk < 0 || blk >= c->num_blocks) return FDL_EINVAL;
    }
  }
  return FDL_OK;
}

}  // namespace

extern "C" {

const char *fdl_status_string(int status) {
  switch (status) {
    case FDL_OK: return "ok";
    case FDL_EINVAL: return "invalid argument (null pointer or inconsistent size)";
    case FDL_EUNSUPPORTED: return "unsupported shape (head_dim, block_size or hidden)";
    case FDL_EWORKSPACE: return "workspace too small";
    case FDL_EHIP: return "HIP launch failed";
    case FDL_ESCRATCH:
      return "sizes need more scratch than the static buffer holds (fdl_static_scratch_bytes)";
    default: return "unknown status";
  }
}

int fdl_last_hip_error(void) { return g_last_hip_error; }

const char *fdl_version(void) { return "fdllm 0.1 gfx950"; }

}  // extern "C"

namespace {

// Host validation of flash_cache_step's arguments into launch arguments.
// Returns a status; empty is set when the call has nothing to do.
int fc_args(const fdl_kv_cache *cache, const void *x, int32_t hidden, const void *w_qkv,
            int32_t batch, int32_t num_rows, const int32_t *cu_rows, const int32_t *positions,
            const int32_t *slots, float rope_base, void *q_out, int64_t *slot_mapping_out,
            fdl::FlashCacheArgs &a, bool &empty) {
  empty = false;
  int st = check_cache(cache, true);
  if (st) return st;
  if (batch < 0 || num_rows < 0 || hidden <= 0) return FDL_EINVAL;
  if (!(rope_base > 0.f) || !std::isfinite(rope_base)) return FDL_EINVAL;
  if (hidden % 128 != 0 || hidden > 32768) return FDL_EUNSUPPORTED;
  if (batch == 0 || num_rows == 0) {
    empty = true;
    return FDL_OK;
  }
  if (!x || !w_qkv || !cu_rows || !positions || !slots || !q_out) return FDL_EINVAL;
  // the projection reads X and W and writes Q and the pools in 16-byte pieces
  auto misaligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  if (misaligned(x) || misaligned(w_qkv) || misaligned(q_out) || misaligned(cache->k_cache) ||
      misaligned(cache->v_cache))
    return FDL_EINVAL;
  a.c = view_of(cache);
  a.x = static_cast<const uint16_t *>(x);
  a.w = static_cast<const uint16_t *>(w_qkv);
  a.hidden = hidden;
  a.batch = batch;
  a.rows = num_rows;
  a.cu_rows = cu_rows;
  a.positions = positions;
  a.slots = slots;
  a.log2_base = std::log2((double)rope_base);
  a.q_out = static_cast<uint16_t *>(q_out);
  a.slot_mapping = slot_mapping_out;
  a.y_out = nullptr;
  return FDL_OK;
}

// Validation and launch shared by the fused step and its unfused ablation.
int flash_cache_common(bool unfused, const fdl_kv_cache *cache, const void *x, int32_t hidden,
                       const void *w_qkv, int32_t batch, int32_t num_rows,
                       const int32_t *cu_rows, const int32_t *positions, const int32_t *slots,
                       float rope_base, void *q_out, int64_t *slot_mapping_out,
                       void *workspace, size_t workspace_bytes, void *stream) {
  fdl::FlashCacheArgs a;
  bool empty;
  int st = fc_args(cache, x, hidden, w_qkv, batch, num_rows, cu_rows, positions, slots, rope_base,
                   q_out, slot_mapping_out, a, empty);
  if (st || empty) return st;
  const size_t need =
      unfused ? fdl::flash_cache_unfused_workspace_bytes(num_rows, hidden, cache->num_heads,
                                                         cache->head_dim)
              : fdl::flash_cache_workspace_bytes(num_rows, hidden, cache->num_heads,
                                                 cache->head_dim);
  if (workspace_bytes < need || (need && !workspace)) return FDL_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_mode() &&
      (st = debug_check_rows(cache, batch, num_rows, cu_rows, positions, slots, s)))
    return st;
  return hip_status(unfused ? fdl::launch_flash_cache_unfused(a, workspace, workspace_bytes, s)
                            : fdl::launch_flash_cache(a, workspace, workspace_bytes, s));
}

// Host validation of scheduled_attention's arguments (workspace aside) into
// launch arguments and the plan.  empty: 1 = no sequences (nothing to check
// further), 2 = no rows and no mass (nothing to launch once the workspace
// is checked), 0 = launch.
int attn_args(const fdl_kv_cache *cache, const void *q, int32_t batch, int32_t num_rows,
              const int32_t *cu_rows, const int32_t *kv_len, int32_t max_kv_len,
              int32_t max_rows_per_seq, const fdl_two_view *views, float softmax_scale,
              float *out, float *mass, int32_t mass_stride, fdl::AttnArgs &a, fdl::AttnPlan &plan,
              int &empty) {
  empty = 0;
  int st = check_cache(cache, true);
  if (st) return st;
  if (batch < 0 || num_rows < 0 || max_kv_len < 0 || max_rows_per_seq < 0) return FDL_EINVAL;
  if (!(softmax_scale >= 0.f) || !std::isfinite(softmax_scale)) return FDL_EINVAL;
  if ((long)max_kv_len > (long)cache->max_blocks_per_seq * cache->block_size) return FDL_EINVAL;
  if ((max_kv_len + cache->block_size - 1) / cache->block_size > 1024) return FDL_EUNSUPPORTED;
  if (mass && mass_stride < max_kv_len) return FDL_EINVAL;
  if (mass && mass_stride <= 0) return FDL_EINVAL;
  const int ms = mass ? mass_stride : 0;
  plan = fdl::plan_attention(batch, num_rows, cache->num_heads, cache->head_dim, max_kv_len,
                             max_rows_per_seq, ms);
  if (batch == 0) {
    empty = 1;
    return FDL_OK;
  }
  if (!cu_rows || !kv_len) return FDL_EINVAL;
  if (num_rows > 0 && (!q || !out)) return FDL_EINVAL;
  if (num_rows > 0 && max_rows_per_seq == 0) return FDL_EINVAL;
  if (num_rows == 0 && !mass) empty = 2;
  a.c = view_of(cache);
  a.q = static_cast<const uint16_t *>(q);
  a.batch = batch;
  a.rows = num_rows;
  a.cu_rows = cu_rows;
  a.kv_len = kv_len;
  a.max_kv_len = max_kv_len;
  a.views = reinterpret_cast<const int32_t *>(views);
  const double scale = softmax_scale > 0.f ? (double)softmax_scale
                                            : 1.0 / std::sqrt((double)cache->head_dim);
  a.scale_log2 = (float)(scale * 1.4426950408889634073599246810019);
  a.out = out;
  a.mass = mass;
  a.mass_stride = ms;
  a.ws = nullptr;
  return FDL_OK;
}

using fdl::kFusedSyncBytes;

}  // namespace

extern "C" {

int flash_cache_step(const fdl_kv_cache *cache, const void *x, int32_t hidden, const void *w_qkv,
                     int32_t batch, int32_t num_rows, const int32_t *cu_rows,
                     const int32_t *positions, const int32_t *slots, float rope_base,
                     void *q_out, int64_t *slot_mapping_out, void *workspace,
                     size_t workspace_bytes, void *stream) {
  return flash_cache_common(false, cache, x, hidden, w_qkv, batch, num_rows, cu_rows, positions,
                            slots, rope_base, q_out, slot_mapping_out, workspace,
                            workspace_bytes, stream);
}

int flash_cache_step_unfused(const fdl_kv_cache *cache, const void *x, int32_t hidden,
                             const void *w_qkv, int32_t batch, int32_t num_rows,
                             const int32_t *cu_rows, const int32_t *positions,
                             const int32_t *slots, float rope_base, void *q_out,
                             int64_t *slot_mapping_out, void *workspace,
                             size_t workspace_bytes, void *stream) {
  return flash_cache_common(true, cache, x, hidden, w_qkv, batch, num_rows, cu_rows, positions,
                            slots, rope_base, q_out, slot_mapping_out, workspace,
                            workspace_bytes, stream);
}

size_t fdl_flash_cache_unfused_workspace_bytes(int32_t num_rows, int32_t hidden,
                                               int32_t num_heads, int32_t head_dim) {
  if (num_rows < 0 || hidden <= 0 || num_heads <= 0 || head_dim <= 0) return 0;
  return fdl::flash_cache_unfused_workspace_bytes(num_rows, hidden, num_heads, head_dim);
}

size_t fdl_flash_cache_workspace_bytes(int32_t num_rows, int32_t hidden, int32_t num_heads,
                                       int32_t head_dim) {
  if (num_rows < 0 || hidden <= 0 || num_heads <= 0 || head_dim <= 0) return 0;
  return fdl::flash_cache_workspace_bytes(num_rows, hidden, num_heads, head_dim);
}

size_t fdl_attention_workspace_bytes(int32_t batch, int32_t num_rows, int32_t num_heads,
                                     int32_t head_dim, int32_t max_kv_len,
                                     int32_t max_rows_per_seq, int32_t mass_stride) {
  if (batch < 0 || num_rows < 0 || num_heads <= 0 || head_dim <= 0 || max_kv_len < 0 ||
      max_rows_per_seq < 0 || mass_stride < 0)
    return 0;
  return fdl::plan_attention(batch, num_rows, num_heads, head_dim, max_kv_len, max_rows_per_seq,
                             mass_stride)
      .bytes;
}

}  // extern "C"

namespace {

// scheduled_attention_static's scratch: one static device buffer per GPU
// (each device holds its own copy of the array, at its own address).  In host
// code `scratch` names a host-side stand-in, never device memory: kernels and
// copies get the per-device address from hipGetSymbolAddress.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the device's first
// call, with the device current); nullptr and a HIP status on failure.
void *device_scratch(hipError_t &err) {
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p) {
      if (err == hipSuccess) err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t fdl_static_scratch_bytes(void) { return kStaticScratchBytes; }

int scheduled_attention_static(const fdl_kv_cache *cache, const void *q, int32_t batch,
                               int32_t num_rows, const int32_t *cu_rows, const int32_t *kv_len,
                               int32_t max_kv_len, int32_t max_rows_per_seq,
                               const fdl_two_view *views, float softmax_scale, float *out,
                               float *mass, int32_t mass_stride, void *stream) {
  fdl::AttnArgs a;
  fdl::AttnPlan plan;
  int empty;
  int st = attn_args(cache, q, batch, num_rows, cu_rows, kv_len, max_kv_len, max_rows_per_seq,
                     views, softmax_scale, out, mass, mass_stride, a, plan, empty);
  if (st || empty == 1) return st;
  if (plan.bytes > kStaticScratchBytes) return FDL_ESCRATCH;
  if (empty) return FDL_OK;
  if (debug_mode() &&
      (st = debug_check_attention(cache, batch, num_rows, cu_rows, kv_len, max_kv_len,
                                  max_rows_per_seq, views, static_cast<hipStream_t>(stream))))
    return st;
  hipError_t err;
  void *ws = device_scratch(err);
  if (!ws) return hip_status(err);
  a.ws = static_cast<char *>(ws);
  return hip_status(fdl::launch_attention(a, plan, static_cast<hipStream_t>(stream)));
}

int fdl_attention_path(int32_t batch, int32_t num_rows, int32_t num_heads, int32_t head_dim,
                       int32_t max_kv_len, int32_t max_rows_per_seq, int32_t mass_stride) {
  if (batch < 0 || num_rows < 0 || num_heads <= 0 || head_dim <= 0 || max_kv_len < 0 ||
      max_rows_per_seq < 0 || mass_stride < 0)
    return 0;
  const fdl::AttnPlan p = fdl::plan_attention(batch, num_rows, num_heads, head_dim, max_kv_len,
                                              max_rows_per_seq, mass_stride);
  if (p.rows_path) return FDL_PATH_ROW_GROUPS;
  if (p.fwd_mass) return FDL_PATH_SPLIT_MASS_REREAD;
  if (p.xmass) return FDL_PATH_SPLIT_MASS_EXCHANGE;
  return FDL_PATH_SPLIT;
}

int scheduled_attention(const fdl_kv_cache *cache, const void *q, int32_t batch,
                        int32_t num_rows, const int32_t *cu_rows, const int32_t *kv_len,
                        int32_t max_kv_len, int32_t max_rows_per_seq, const fdl_two_view *views,
                        float softmax_scale, float *out, float *mass, int32_t mass_stride,
                        void *workspace, size_t workspace_bytes, void *stream) {
  fdl::AttnArgs a;
  fdl::AttnPlan plan;
  int empty;
  int st = attn_args(cache, q, batch, num_rows, cu_rows, kv_len, max_kv_len, max_rows_per_seq,
                     views, softmax_scale, out, mass, mass_stride, a, plan, empty);
  if (st || empty == 1) return st;
  if (plan.bytes > workspace_bytes || (plan.bytes && !workspace)) return FDL_EWORKSPACE;
  if (empty) return FDL_OK;
  if (debug_mode() &&
      (st = debug_check_attention(cache, batch, num_rows, cu_rows, kv_len, max_kv_len,
                                  max_rows_per_seq, views, static_cast<hipStream_t>(stream))))
    return st;
  a.ws = static_cast<char *>(workspace);
  return hip_status(fdl::launch_attention(a, plan, static_cast<hipStream_t>(stream)));
}

size_t fdl_fused_step_workspace_bytes(int32_t batch, int32_t num_rows, int32_t num_heads,
                                      int32_t head_dim, int32_t max_kv_len,
                                      int32_t max_rows_per_seq, int32_t mass_stride) {
  if (batch < 0 || num_rows < 0 || num_heads <= 0 || head_dim <= 0 || max_kv_len < 0 ||
      max_rows_per_seq < 0 || mass_stride <= 0)
    return 0;
  // [counters of the single launch][attention workspace][projection partials]
  return kFusedSyncBytes +
         fdl::plan_attention(batch, num_rows, num_heads, head_dim, max_kv_len, max_rows_per_seq,
                             mass_stride)
             .bytes +
         fdl::flash_cache_workspace_max();
}

int flash_cache_attention_step(const fdl_kv_cache *cache, const void *x, int32_t hidden,
                               const void *w_qkv, int32_t batch, int32_t num_rows,
                               const int32_t *cu_rows, const int32_t *positions,
                               const int32_t *slots, float rope_base, void *q_out,
                               int64_t *slot_mapping_out, const int32_t *kv_len,
                               int32_t max_kv_len, int32_t max_rows_per_seq,
                               const fdl_two_view *views, float softmax_scale, float *out,
                               float *mass, int32_t mass_stride, void *workspace,
                               size_t workspace_bytes, void *stream) {
  fdl::FlashCacheArgs fa;
  fdl::AttnArgs aa;
  fdl::AttnPlan plan;
  bool empty_fc;
  int empty_at;
  int st = fc_args(cache, x, hidden, w_qkv, batch, num_rows, cu_rows, positions, slots,
                   rope_base, q_out, slot_mapping_out, fa, empty_fc);
  if (st) return st;
  st = attn_args(cache, q_out, batch, num_rows, cu_rows, kv_len, max_kv_len, max_rows_per_seq,
                 views, softmax_scale, out, mass, mass_stride, aa, plan, empty_at);
  if (st || empty_at == 1) return st;
  if (!mass) return FDL_EINVAL;
  const size_t fc_need =
      fdl::flash_cache_workspace_bytes(num_rows, hidden, cache->num_heads, cache->head_dim);
  // the documented size (any hidden size), not only this projection's share
  if (workspace_bytes < kFusedSyncBytes + plan.bytes + fdl::flash_cache_workspace_max() ||
      !workspace)
    return FDL_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_mode()) {
    if (!empty_fc && (st = debug_check_rows(cache, batch, num_rows, cu_rows, positions, slots, s)))
      return st;
    if ((st = debug_check_attention(cache, batch, num_rows, cu_rows, kv_len, max_kv_len,
                                    max_rows_per_seq, views, s)))
      return st;
  }
  char *ws = static_cast<char *>(workspace);
  if (!empty_fc) {
    st = hip_status(fdl::launch_flash_cache(fa, fc_need ? ws + kFusedSyncBytes + plan.bytes : nullptr,
                                            fc_need, s));
    if (st) return st;
  }
  aa.ws = ws + kFusedSyncBytes;
  return hip_status(fdl::launch_attention(aa, plan, s));
}

int flash_cache_attention_step_single_launch(const fdl_kv_cache *cache, const void *x, int32_t hidden,
                               const void *w_qkv, int32_t batch, int32_t num_rows,
                               const int32_t *cu_rows, const int32_t *positions,
                               const int32_t *slots, float rope_base, void *q_out,
                               int64_t *slot_mapping_out, const int32_t *kv_len,
                               int32_t max_kv_len, int32_t max_rows_per_seq,
                               const fdl_two_view *views, float softmax_scale, float *out,
                               float *mass, int32_t mass_stride, void *workspace,
                               size_t workspace_bytes, void *stream) {
  fdl::FlashCacheArgs fa;
  fdl::AttnArgs aa;
  fdl::AttnPlan plan;
  bool empty_fc;
  int empty_at;
  int st = fc_args(cache, x, hidden, w_qkv, batch, num_rows, cu_rows, positions, slots,
                   rope_base, q_out, slot_mapping_out, fa, empty_fc);
  if (st) return st;
  st = attn_args(cache, q_out, batch, num_rows, cu_rows, kv_len, max_kv_len, max_rows_per_seq,
                 views, softmax_scale, out, mass, mass_stride, aa, plan, empty_at);
  if (st || empty_at == 1) return st;
  if (!mass) return FDL_EINVAL;
  if (workspace_bytes < kFusedSyncBytes + plan.bytes || !workspace) return FDL_EWORKSPACE;
  if (debug_mode()) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!empty_fc && (st = debug_check_rows(cache, batch, num_rows, cu_rows, positions, slots, s)))
      return st;
    if ((st = debug_check_attention(cache, batch, num_rows, cu_rows, kv_len, max_kv_len,
                                    max_rows_per_seq, views, s)))
      return st;
  }
  if (empty_fc) {
    // No rows to project: what remains is the attention call's (with the
    // mass asked for, it writes zeros).
    aa.ws = static_cast<char *>(workspace) + kFusedSyncBytes;
    return hip_status(fdl::launch_attention(aa, plan, static_cast<hipStream_t>(stream)));
  }
  if (!fdl::fused_step_supported(fa, plan, true)) return FDL_EUNSUPPORTED;
  aa.ws = static_cast<char *>(workspace) + kFusedSyncBytes;
  return hip_status(fdl::launch_fused_step(fa, aa, plan, static_cast<int *>(workspace),
                                           static_cast<hipStream_t>(stream)));
}

int track_topb(const float *mass, int32_t mass_stride, const int32_t *kv_len, int32_t batch,
               int32_t topb, int32_t *idx_out, void *stream) {
  if (batch < 0 || topb <= 0 || mass_stride <= 0) return FDL_EINVAL;
  if (batch == 0) return FDL_OK;
  if (!mass || !kv_len || !idx_out) return FDL_EINVAL;
  return hip_status(
      fdl::launch_topb(mass, mass_stride, kv_len, batch, topb, idx_out, static_cast<hipStream_t>(stream)));
}

int verify_accept(const int32_t *draft_tok, const int32_t *mask_tok, const float *conf,
                  int32_t batch, int32_t window, float threshold, int32_t *accept_len_out,
                  void *stream) {
  if (batch < 0 || window < 0) return FDL_EINVAL;
  if (batch == 0) return FDL_OK;
  if (!accept_len_out) return FDL_EINVAL;
  if (window > 0 && (!draft_tok || !mask_tok || !conf)) return FDL_EINVAL;
  return hip_status(fdl::launch_verify(draft_tok, mask_tok, conf, batch, window, threshold,
                                       accept_len_out, static_cast<hipStream_t>(stream)));
}

int decode_plan(int32_t batch, const int32_t *kv_len, int32_t window_len, int32_t block_size,
                int32_t refresh_period, int32_t step, const int32_t *tracked, int32_t topb,
                const int32_t *accept_len, int32_t *frontier, int32_t *cu_rows_out,
                int32_t *positions_out, int32_t *slots_out, int32_t *stage_out,
                int32_t row_capacity, void *stream) {
  if (batch < 0 || window_len < 1 || block_size < 1 || refresh_period < 0 || step < 0 ||
      topb < 0 || row_capacity < 0)
    return FDL_EINVAL;
  if (batch > fdl::kPlanMaxBatch) return FDL_EUNSUPPORTED;
  if ((int64_t)row_capacity < (int64_t)batch * ((int64_t)window_len + topb)) return FDL_EINVAL;
  if (batch == 0) return FDL_OK;
  if (!kv_len || !frontier || !cu_rows_out || !positions_out || !slots_out) return FDL_EINVAL;
  if (topb > 0 && !tracked) return FDL_EINVAL;
  if (step > 0 && !accept_len) return FDL_EINVAL;
  fdl::PlanArgs a;
  a.batch = batch;
  a.window = window_len;
  a.block_size = block_size;
  a.refresh_period = refresh_period;
  a.step = step;
  a.topb = topb;
  a.kv_len = kv_len;
  a.tracked = tracked;
  a.accept_len = accept_len;
  a.frontier = frontier;
  a.frontier_out = frontier;
  a.cu_rows = cu_rows_out;
  a.positions = positions_out;
  a.slots = slots_out;
  a.stage = stage_out;
  return hip_status(fdl::launch_plan(a, static_cast<hipStream_t>(stream)));
}

int gather_hidden(int32_t batch, int32_t row_capacity, const int32_t *cu_rows,
                  const int32_t *positions, const int32_t *frontier,
                  const void *hidden_committed, const void *hidden_masked, int32_t max_len,
                  int32_t hidden, void *x_out, void *stream) {
  if (batch < 0 || row_capacity < 0 || max_len < 1 || hidden <= 0 || hidden % 8 != 0)
    return FDL_EINVAL;
  if (batch == 0 || row_capacity == 0) return FDL_OK;
  if (!cu_rows || !positions || !frontier || !hidden_committed || !hidden_masked || !x_out)
    return FDL_EINVAL;
  auto misaligned = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  if (misaligned(hidden_committed) || misaligned(hidden_masked) || misaligned(x_out))
    return FDL_EINVAL;
  fdl::GatherArgs a;
  a.batch = batch;
  a.rows = row_capacity;
  a.max_len = max_len;
  a.hidden = hidden;
  a.cu_rows = cu_rows;
  a.positions = positions;
  a.frontier = frontier;
  a.committed = static_cast<const uint16_t *>(hidden_committed);
  a.masked = static_cast<const uint16_t *>(hidden_masked);
  a.x_out = static_cast<uint16_t *>(x_out);
  return hip_status(fdl::launch_gather_hidden(a, static_cast<hipStream_t>(stream)));
}

size_t fdl_lm_head_workspace_bytes(int32_t rows, int32_t vocab) {
  if (rows < 0 || vocab <= 0) return 0;
  return fdl::lm_head_workspace_bytes(rows, vocab);
}

int lm_head_confidence(const void *hidden_states, const void *w_lm, int32_t rows, int32_t vocab,
                       int32_t hidden, int32_t *token_out, float *conf_out, void *workspace,
                       size_t workspace_bytes, void *stream) {
  if (rows < 0 || vocab <= 0 || hidden <= 0) return FDL_EINVAL;
  if (hidden % 32 != 0 || hidden > 65536) return FDL_EUNSUPPORTED;
  if (rows == 0) return FDL_OK;
  if (!hidden_states || !w_lm || !token_out || !conf_out) return FDL_EINVAL;
  const size_t need = fdl::lm_head_workspace_bytes(rows, vocab);
  if (workspace_bytes < need || !workspace) return FDL_EWORKSPACE;
  fdl::LmHeadArgs a;
  a.h = static_cast<const uint16_t *>(hidden_states);
  a.w = static_cast<const uint16_t *>(w_lm);
  a.rows = rows;
  a.vocab = vocab;
  a.hidden = hidden;
  a.token = token_out;
  a.conf = conf_out;
  a.part_ml = nullptr;
  a.part_idx = nullptr;
  return hip_status(fdl::launch_lm_head(a, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
