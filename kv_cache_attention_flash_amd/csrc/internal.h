// Host-side launch interfaces between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fdl {

struct CacheView {
  int H, D, bs, bs_shift, num_blocks, max_blocks;  // bs = 1 << bs_shift
  uint16_t *k, *v;
  const int32_t *block_table;
};

struct FlashCacheArgs {
  CacheView c;
  const uint16_t *x;
  const uint16_t *w;
  int hidden, batch, rows;
  const int32_t *cu_rows, *positions, *slots;
  double log2_base;
  uint16_t *q_out;
  int64_t *slot_mapping;
  float *y_out;  // non-null: store the raw fp32 projection [rows][3HD] instead (unfused ablation)
};

size_t flash_cache_workspace_bytes(int rows, int hidden, int H, int D);
size_t flash_cache_workspace_max();
hipError_t launch_flash_cache(const FlashCacheArgs &a, void *ws, size_t ws_bytes, hipStream_t s);
size_t flash_cache_unfused_workspace_bytes(int rows, int hidden, int H, int D);
hipError_t launch_flash_cache_unfused(const FlashCacheArgs &a, void *ws, size_t ws_bytes,
                                      hipStream_t s);

struct AttnPlan {
  int rows_path;      // 1: row-group kernel (whole cache per workgroup)
  int rgroups;        // ceil(max_rows_per_seq / 16), row-group path
  int maxt;           // tiles per wave kept for the mass, row-group path
  int row_tiles;      // ceil(max_rows_per_seq / 64), split path
  int splits;         // KV splits per (sequence, row tile, head), split path
  int xmass;          // 1: split path with the mass
  int fwd_mass;       // xmass by one workgroup per unit with a second pass over K (long caches)
  int sync_ints;      // xmass with splits > 1: ticket, error word, one count per group
  size_t off_part_o, off_part_ml, off_mass_part, off_sync, bytes;
};

AttnPlan plan_attention(int batch, int rows, int H, int D, int max_kv_len,
                        int max_rows_per_seq, int mass_stride);

struct AttnArgs {
  CacheView c;
  const uint16_t *q;
  int batch, rows;
  const int32_t *cu_rows, *kv_len, *views;
  int max_kv_len;
  float scale_log2;
  float *out, *mass;
  int mass_stride;
  char *ws;
};

hipError_t launch_attention(const AttnArgs &a, const AttnPlan &p, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cus();

// Single-launch step (fused.hip): the projection then row-group attention with
// the mass, for shapes whose separate calls take a one-launch projection (no
// split reduction) and the row-group attention path.  sync: 5 ints of device
// memory, zero before the first call (each call leaves them zero).
// Leading bytes of the one-call steps' workspace: the single launch's
// counters (tickets, per-XCD and per-head counts) and its error word (byte 12).
constexpr size_t kFusedSyncBytes = 4096;
bool fused_step_supported(const FlashCacheArgs &fa, const AttnPlan &ap, bool mass);
hipError_t launch_fused_step(const FlashCacheArgs &fa, const AttnArgs &aa, const AttnPlan &ap,
                             int *sync, hipStream_t s);

hipError_t launch_topb(const float *mass, int stride, const int32_t *kv_len, int batch,
                       int topb, int32_t *out, hipStream_t s);

hipError_t launch_verify(const int32_t *draft, const int32_t *mask, const float *conf,
                         int batch, int window, float thr, int32_t *out, hipStream_t s);

// Multi-step loop planning (loop.hip).
constexpr int kStageUpdate = 0, kStageRefresh = 1, kStageDone = 2;
constexpr int kPlanMaxBatch = 4096;

struct PlanArgs {
  int batch, window, block_size, refresh_period, step, topb;
  const int32_t *kv_len, *tracked, *accept_len, *frontier;
  int32_t *frontier_out, *cu_rows, *positions, *slots, *stage;
};

hipError_t launch_plan(const PlanArgs &a, hipStream_t s);

struct GatherArgs {
  int batch, rows, max_len, hidden;  // rows = capacity of x_out
  const int32_t *cu_rows, *positions, *frontier;
  const uint16_t *committed, *masked;
  uint16_t *x_out;
};

hipError_t launch_gather_hidden(const GatherArgs &a, hipStream_t s);

// Mask-view confidence producer (lm_head.hip).
struct LmHeadArgs {
  const uint16_t *h, *w;  // bf16 [rows][hidden], [vocab][hidden]
  int rows, vocab, hidden;
  int32_t *token;
  float *conf;
  float *part_ml;     // workspace: [rows][col tiles][2] (max, sum of exp)
  int32_t *part_idx;  // workspace: [rows][col tiles]
};

int lm_head_col_tiles(int vocab);
size_t lm_head_workspace_bytes(int rows, int vocab);
hipError_t launch_lm_head(LmHeadArgs a, void *ws, hipStream_t s);

}  // namespace fdl
