// Internal types of libpagedattn: the schedule a plan holds and the launch
// interface between the C ABI (api.cpp) and the kernels (kernels.hip).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/pagedattn.h"

namespace pa {

// One unit of attention work for one KV head (the KV head is the grid's y index).
// Columns are (query position, query head) pairs: position n in [0, nrows) is
// token row row0 + n.  Keys [kv_begin, kv_end) of block-table row `seq` are read;
// with `causal` set, position n sees only keys t <= lim0 + n.
struct WorkItem {
  int32_t seq;
  int32_t row0;
  int32_t nrows;
  int32_t lim0;
  int32_t kv_begin;
  int32_t kv_end;
  int32_t slot;    // partial record = row_pbase[row] + slot when row_pbase[row] >= 0
  int32_t causal;
};
static_assert(sizeof(WorkItem) == 32, "WorkItem layout");

// A token row whose result is the LSE-merge of `count` partial records
// starting at `pbase`.
struct MergeRow {
  int32_t row;
  int32_t pbase;
  int32_t count;
  int32_t pad;
};
static_assert(sizeof(MergeRow) == 16, "MergeRow layout");

// Prefill tiling: a workgroup owns `tiles` column tiles of 16 (two per wave).
// Tile j holds head (j / tiles_per_head) of the workgroup's head group and
// positions 16 * (j % tiles_per_head) .. +15.
struct PrefillShape {
  int tiles;           // column tiles per workgroup (8, or 16 for the 8-wave wide prefill)
  int heads_per_wg;    // 1, 2, 4 or 8, divides g, at most max_heads
  int tiles_per_head;  // tiles / heads_per_wg
  int rows_per_item;   // 16 * tiles_per_head
  int head_groups;     // g / heads_per_wg
};
PrefillShape prefill_shape(int group, int tiles, int max_heads);
// The wide prefill kernel serves bf16 queries with head size 128 (bf16 or
// e4m3 pool): 4 waves, 8 column tiles per workgroup (8 waves and 16 tiles
// beside decodes, see wide_prefill_tiles), both tiles of a wave on one head.
inline bool use_wide_prefill(int dtype, int head_size, int kv_dtype) {
  return dtype == PA_BF16 && head_size == 128 && (kv_dtype == PA_KV_SAME || kv_dtype == PA_KV_FP8_E4M3);
}
// Column tiles per wide-prefill workgroup.  Beside decodes a bf16 pool's
// prefill runs 8-wave workgroups, each filling the register file of its CU: a
// 4-wave prefill workgroup leaves a CU half empty yet too full for an 8-wave
// decode workgroup, so the decode would get fewer CUs.  Otherwise 4-wave
// workgroups, two per CU, whose independent barriers let one's softmax
// overlap the other's MFMAs.
inline int wide_prefill_tiles(bool beside_decodes, int kv_dtype) {
  return beside_decodes && kv_dtype == PA_KV_SAME ? 16 : 8;
}

// Everything the kernels need besides the caller's tensors.
struct LaunchGeom {
  int H, Hkv, g, D, bs, max_blocks, dtype, kv_dtype;
  int slot_stride, head_stride;  // pool elements between slots / KV heads (see pool_strides)
  float scale_log2;  // scale * log2(e)
  PrefillShape ps;
};

struct DeviceSchedule {
  const WorkItem* decode;
  int n_decode;
  const int32_t* decode_lists;  // [n_decode_lists + 1] first item of each list
  int n_decode_lists;
  const WorkItem* prefill;
  int n_prefill;
  const WorkItem* prefix;
  int n_prefix;
  const MergeRow* merge;
  int n_merge;
  const int32_t* row_pbase;
  int num_partials;
  bool prefix_beside;  // see HostPlan::prefix_beside
};

struct Tensors {
  const void* q;
  const void* kv;
  const int32_t* block_table;
  void* out;
  float* lse;
  float* ws_o;    // [num_partials, H, D]
  float* ws_lse;  // [num_partials, H]
  const float* k_scale;  // e4m3 pool: [n_scales] K and V scales (1 or Hkv); else null
  const float* v_scale;
  int n_scales;
};

// The caller's stream, plus an optional side stream with fork/join events: when
// present, prefill and shared-prefix launches go to the side stream after it
// waits for the caller's stream, and the caller's stream waits for them before
// the merge.
struct Streams {
  void* main;
  void* aux;      // may be null: everything runs on `main`
  void* ev_fork;
  void* ev_join;
};

// Launchers (kernels.hip).  Each returns a HIP error code (0 = success).
int launch_forward(const LaunchGeom& g, const DeviceSchedule& s, const Tensors& t, const Streams& st);
int launch_merge_states(const void* oa, const float* la, const void* ob, const float* lb, void* o,
                        float* l, int n_tok, int n_heads, int head_size, int dtype, void* stream);
int launch_gather(const void* kv, const int32_t* bt_row, int seq_len, int bs, int Hkv, int D,
                  int elem_bytes, int64_t slot_stride, int64_t head_stride, void* k_out, void* v_out,
                  void* stream);
// One workgroup comparing the caller's device metadata with the plan's copies
// (NULL caller arrays and a NULL p_bt are skipped or replaced by the pool range
// check); writes the mismatch count to *bad.
int launch_check_metadata(const int32_t* bt, const int32_t* qsl, const int32_t* sl, const int32_t* p_bt,
                          const int32_t* p_qsl, const int32_t* p_sl, int B, int mb, int bs, int num_blocks,
                          int32_t* bad, void* stream);
int launch_write_kv(const void* k, const void* v, const int64_t* slots, int n_tok, int Hkv, int head_bytes, int bs,
                    int64_t n_slots, int64_t slot_bstride, int64_t head_bstride, void* kv, void* stream);
int launch_write_kv_fp8(const void* k, const void* v, const int64_t* slots, int n_tok, int Hkv, int D, int bs,
                        int64_t n_slots, int64_t slot_stride, int64_t head_stride, const float* k_scale,
                        const float* v_scale, int n_scales, void* kv, void* stream);

// Pool element strides of the memory order `layout` (pa_kv_layout): between
// consecutive slots of one KV head, and between KV heads of one slot.  NHD
// (blocks, 2, slot, head, d): Hkv * D and D; HND (blocks, 2, head, slot, d):
// D and bs * D.  The K/V halves and blocks are bs * Hkv * D apart either way.
inline void pool_strides(int layout, int bs, int Hkv, int D, int& slot_stride, int& head_stride) {
  if (layout == PA_KV_HND) {
    slot_stride = D;
    head_stride = bs * D;
  } else {
    slot_stride = Hkv * D;
    head_stride = D;
  }
}

// The calling thread's error message for pa_last_error (api.cpp); returns `s`.
pa_status set_last_error(pa_status s, const std::string& msg);
// The device a plan runs on (< 0: host-only plan).
int plan_device(const pa_plan* plan);

// Launch bookkeeping for pa_profile_* (api.cpp).
void profile_before(const char* name, void* stream);
void profile_after(void* stream);

// Host planner (planner.cpp): validates and builds the schedule.
struct HostPlan {
  pa_params p{};
  int32_t T = 0;
  std::vector<int32_t> order, is_decode, prefix_blocks, row_partials, row_pbase;
  // the metadata the plan was built from (block_table empty when none was given)
  std::vector<int32_t> qsl, seq_lens, block_table;
  std::vector<WorkItem> decode_items, prefill_items, prefix_items;
  std::vector<int32_t> decode_lists;  // [lists + 1]
  std::vector<MergeRow> merges;
  pa_plan_info info{};
  PrefillShape ps{};
  int num_partials = 0;
  // the shared-prefix pass runs beside the decode on CUs of its own, in the
  // decode's launch (8-wave prefix workgroups, decode lists sized for the
  // other CUs)
  bool prefix_beside = false;
};

// Decode launch shape: the Hkv x ceil(g / 16) units of an item are run by
// workgroups of this many waves (the largest divisor of the unit count up to 8).
inline int decode_waves_per_wg(int units) {
  int nw = 8;
  while (units % nw != 0) --nw;
  return nw;
}
// Decode workgroups of `waves` waves that fit on one CU at once, for the
// variant that balanced lists run (two steps in flight for bf16 queries; kernels.hip;
// the device must be current), or 0 if the query fails.
int decode_workgroups_per_cu(int dtype, int kv_dtype, int head_size, int waves);

// Returns PA_OK or an error with `err` filled in.  decode_wgs_per_cu: resident
// decode workgroups per CU (0 = unknown: no balanced decode lists).
pa_status build_host_plan(const pa_params& p, const int32_t* qsl, const int32_t* seq_lens,
                          const int32_t* block_table, int num_cus, int decode_wgs_per_cu, HostPlan& out,
                          std::string& err);

}  // namespace pa
