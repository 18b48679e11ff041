// C ABI of libpagedattn: argument checks, plan ownership, device copies of the
// schedule, error reporting and the optional per-launch timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

struct pa_plan {
  pa::HostPlan hp;
  int device = -1;
  void* dev_buf = nullptr;
  pa::DeviceSchedule ds{};
  size_t ws_bytes = 0;
  // side stream and fork/join events, created with the plan when it holds both
  // decode work and prefill work, so that the MFMA-bound launches overlap the
  // HBM-bound decode (a shared-prefix pass with decodes alone runs in the
  // decode's own launch, or before it)
  hipStream_t aux = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // Held by a forward from its event record on the caller's stream to the
  // caller's wait on the join event, so that two host threads sharing the plan
  // cannot interleave their records of the two events (one side-stream pass
  // would then wait on the other caller's stream).
  std::mutex fork_mu;
  // Held by a metadata check from its launch to the read of its result: the
  // plan has one 4-byte result buffer for every caller.
  std::mutex check_mu;
  // Device copies of the metadata the plan was built from, for
  // pa_plan_check_metadata: query_start_loc [B+1], seq_lens [B], the host block
  // table [B * max_blocks_per_seq] when one was given, and a 4-byte result.
  const int32_t* dev_qsl = nullptr;
  const int32_t* dev_seq_lens = nullptr;
  const int32_t* dev_bt = nullptr;
  int32_t* dev_check = nullptr;
};

namespace {

thread_local std::string g_err;

pa_status set_err(pa_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

pa_status hip_err(hipError_t e, const char* what) {
  return set_err(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Makes `dev` current for the scope of a call and restores the caller's device.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (dev >= 0 && dev != prev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ProfRec {
  std::string name;
  hipEvent_t begin, end;
};

struct ProfState {
  bool active = false;
  int max = 0;
  int pending = -1;
  std::vector<hipEvent_t> pool;
  std::vector<ProfRec> recs;
};

thread_local ProfState g_prof;

void prof_release() {
  for (hipEvent_t e : g_prof.pool) (void)hipEventDestroy(e);
  g_prof = ProfState{};
}

}  // namespace

namespace pa {

pa_status set_last_error(pa_status s, const std::string& msg) { return set_err(s, msg); }

int plan_device(const pa_plan* plan) { return plan ? plan->device : -1; }

void profile_before(const char* name, void* stream) {
  if (!g_prof.active || (int)g_prof.recs.size() >= g_prof.max) return;
  const size_t i = g_prof.recs.size();
  ProfRec r{name, g_prof.pool[2 * i], g_prof.pool[2 * i + 1]};
  if (hipEventRecord(r.begin, static_cast<hipStream_t>(stream)) != hipSuccess) return;
  g_prof.recs.push_back(r);
  g_prof.pending = (int)i;
}

void profile_after(void* stream) {
  if (g_prof.pending < 0) return;
  (void)hipEventRecord(g_prof.recs[g_prof.pending].end, static_cast<hipStream_t>(stream));
  g_prof.pending = -1;
}

}  // namespace pa

extern "C" {

pa_status pa_kv_cache_shape(int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                            int64_t shape_out[5]) {
  g_err.clear();
  if (!shape_out) return set_err(PA_ERR_INVALID_ARG, "shape_out is NULL");
  if (block_size < 16 || block_size % 16 != 0)
    return set_err(PA_ERR_INVALID_ARG, "block size must be a positive multiple of 16");
  if (num_blocks < 1 || num_kv_heads < 1 || head_size < 1)
    return set_err(PA_ERR_INVALID_ARG, "num_blocks, num_kv_heads and head_size must be >= 1");
  shape_out[0] = num_blocks;
  shape_out[1] = 2;
  shape_out[2] = block_size;
  shape_out[3] = num_kv_heads;
  shape_out[4] = head_size;
  return PA_OK;
}

pa_status pa_kv_cache_stride_order(int32_t layout, int32_t order_out[5]) {
  g_err.clear();
  if (!order_out) return set_err(PA_ERR_INVALID_ARG, "order_out is NULL");
  if (layout != PA_KV_NHD && layout != PA_KV_HND) return set_err(PA_ERR_INVALID_ARG, "unknown layout");
  const int32_t nhd[5] = {0, 1, 2, 3, 4}, hnd[5] = {0, 1, 3, 2, 4};
  for (int i = 0; i < 5; ++i) order_out[i] = layout == PA_KV_HND ? hnd[i] : nhd[i];
  return PA_OK;
}

pa_status pa_plan_create(const pa_params* params, const int32_t* query_start_loc, const int32_t* seq_lens,
                         const int32_t* block_table, int device, pa_plan** plan_out) {
  g_err.clear();
  if (!plan_out) return set_err(PA_ERR_INVALID_ARG, "plan_out is NULL");
  *plan_out = nullptr;
  if (!params) return set_err(PA_ERR_INVALID_ARG, "params is NULL");

  int num_cus = 256;
  if (device >= 0) {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return hip_err(e, "hipGetDeviceCount");
    if (device >= n) return set_err(PA_ERR_INVALID_ARG, "device index out of range");
    e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_err(e, "hipDeviceGetAttribute");
  }

  // resident decode workgroups per CU (for the balanced decode lists); a
  // host-only plan assumes one
  int dec_wgs = 1;
  if (device >= 0 && params->num_kv_heads >= 1 && params->num_heads >= params->num_kv_heads &&
      params->num_heads % params->num_kv_heads == 0) {
    const int g = params->num_heads / params->num_kv_heads;
    const int nw = pa::decode_waves_per_wg(params->num_kv_heads * ((g + 15) / 16));
    DeviceGuard guard(device);
    dec_wgs = guard.ok ? pa::decode_workgroups_per_cu(params->dtype, params->kv_dtype, params->head_size, nw) : 0;
  }

  pa_plan* plan = new (std::nothrow) pa_plan();
  if (!plan) return set_err(PA_ERR_OOM, "host allocation failed");
  std::string err;
  pa_status st =
      pa::build_host_plan(*params, query_start_loc, seq_lens, block_table, num_cus, dec_wgs, plan->hp, err);
  if (st != PA_OK) {
    delete plan;
    return set_err(st, err);
  }
  pa::HostPlan& hp = plan->hp;
  plan->device = device;
  plan->ws_bytes = hp.num_partials > 0
                       ? align256((size_t)hp.num_partials * params->num_heads * params->head_size * sizeof(float)) +
                             align256((size_t)hp.num_partials * params->num_heads * sizeof(float))
                       : 0;

  if (device >= 0) {
    // one device buffer: the schedule, then the metadata copies; every
    // section starts on a 256-byte boundary
    struct Section {
      const void* src;
      size_t bytes;
      size_t off;
    };
    std::vector<Section> sec = {
        {hp.decode_items.data(), hp.decode_items.size() * sizeof(pa::WorkItem), 0},
        {hp.prefill_items.data(), hp.prefill_items.size() * sizeof(pa::WorkItem), 0},
        {hp.prefix_items.data(), hp.prefix_items.size() * sizeof(pa::WorkItem), 0},
        {hp.merges.data(), hp.merges.size() * sizeof(pa::MergeRow), 0},
        {hp.row_pbase.data(), hp.row_pbase.size() * sizeof(int32_t), 0},
        {hp.decode_lists.data(), hp.decode_lists.size() * sizeof(int32_t), 0},
        {hp.qsl.data(), hp.qsl.size() * sizeof(int32_t), 0},
        {hp.seq_lens.data(), hp.seq_lens.size() * sizeof(int32_t), 0},
        {hp.block_table.data(), hp.block_table.size() * sizeof(int32_t), 0},
        {nullptr, sizeof(int32_t), 0},  // metadata check result
    };
    size_t total = 0;
    for (Section& x : sec) {
      x.off = total;
      total += align256(x.bytes);
    }
    DeviceGuard guard(device);
    if (!guard.ok) {
      delete plan;
      return set_err(PA_ERR_HIP, "hipSetDevice failed");
    }
    std::vector<unsigned char> host(total, 0);
    for (const Section& x : sec)  // an empty vector's data() may be null
      if (x.bytes && x.src) std::memcpy(host.data() + x.off, x.src, x.bytes);
    hipError_t e = hipMalloc(&plan->dev_buf, total);
    if (e != hipSuccess) {
      plan->dev_buf = nullptr;
      delete plan;
      return set_err(PA_ERR_OOM, std::string("hipMalloc: ") + hipGetErrorString(e));
    }
    e = hipMemcpy(plan->dev_buf, host.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      pa_plan_destroy(plan);
      return hip_err(e, "hipMemcpy");
    }
    unsigned char* base = static_cast<unsigned char*>(plan->dev_buf);
    pa::DeviceSchedule& ds = plan->ds;
    ds.decode = reinterpret_cast<const pa::WorkItem*>(base + sec[0].off);
    ds.n_decode = (int)hp.decode_items.size();
    ds.prefill = reinterpret_cast<const pa::WorkItem*>(base + sec[1].off);
    ds.n_prefill = (int)hp.prefill_items.size();
    ds.prefix = reinterpret_cast<const pa::WorkItem*>(base + sec[2].off);
    ds.n_prefix = (int)hp.prefix_items.size();
    ds.merge = reinterpret_cast<const pa::MergeRow*>(base + sec[3].off);
    ds.n_merge = (int)hp.merges.size();
    ds.row_pbase = reinterpret_cast<const int32_t*>(base + sec[4].off);
    ds.decode_lists = reinterpret_cast<const int32_t*>(base + sec[5].off);
    ds.n_decode_lists = hp.decode_lists.empty() ? 0 : (int)hp.decode_lists.size() - 1;
    ds.num_partials = hp.num_partials;
    ds.prefix_beside = hp.prefix_beside;
    plan->dev_qsl = reinterpret_cast<const int32_t*>(base + sec[6].off);
    plan->dev_seq_lens = reinterpret_cast<const int32_t*>(base + sec[7].off);
    plan->dev_bt = hp.block_table.empty() ? nullptr : reinterpret_cast<const int32_t*>(base + sec[8].off);
    plan->dev_check = reinterpret_cast<int32_t*>(base + sec[9].off);
    if (!hp.decode_items.empty() && !hp.prefill_items.empty()) {
      e = hipStreamCreateWithFlags(&plan->aux, hipStreamNonBlocking);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&plan->ev_fork, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&plan->ev_join, hipEventDisableTiming);
      if (e != hipSuccess) {
        pa_plan_destroy(plan);
        return hip_err(e, "stream/event creation");
      }
    }
  }
  *plan_out = plan;
  return PA_OK;
}

pa_status pa_plan_get_info(const pa_plan* plan, pa_plan_info* info) {
  g_err.clear();
  if (!plan || !info) return set_err(PA_ERR_INVALID_ARG, "plan or info is NULL");
  *info = plan->hp.info;
  return PA_OK;
}

pa_status pa_plan_get_array(const pa_plan* plan, int32_t which, int32_t* dst, int64_t capacity, int64_t* count) {
  g_err.clear();
  if (!plan) return set_err(PA_ERR_INVALID_ARG, "plan is NULL");
  const std::vector<int32_t>* v = nullptr;
  std::vector<int32_t> spans;
  switch (which) {
    case PA_ARRAY_ORDER: v = &plan->hp.order; break;
    case PA_ARRAY_IS_DECODE: v = &plan->hp.is_decode; break;
    case PA_ARRAY_PREFIX_BLOCKS: v = &plan->hp.prefix_blocks; break;
    case PA_ARRAY_ROW_PARTIALS: v = &plan->hp.row_partials; break;
    case PA_ARRAY_DECODE_LISTS: v = &plan->hp.decode_lists; break;
    case PA_ARRAY_DECODE_SPANS:
      spans.reserve(3 * plan->hp.decode_items.size());
      for (const pa::WorkItem& it : plan->hp.decode_items) {
        spans.push_back(it.seq);
        spans.push_back(it.kv_begin);
        spans.push_back(it.kv_end);
      }
      v = &spans;
      break;
    default: return set_err(PA_ERR_INVALID_ARG, "unknown plan array");
  }
  if (count) *count = (int64_t)v->size();
  if ((int64_t)v->size() > capacity) return set_err(PA_ERR_INVALID_ARG, "capacity too small");
  if (!v->empty()) {
    if (!dst) return set_err(PA_ERR_INVALID_ARG, "dst is NULL");
    std::memcpy(dst, v->data(), v->size() * sizeof(int32_t));
  }
  return PA_OK;
}

size_t pa_plan_workspace_bytes(const pa_plan* plan) { return plan ? plan->ws_bytes : 0; }

}  // extern "C"

namespace {

bool misaligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; }

// Compare the caller's device metadata with the plan's copies (one small
// kernel, then a wait for its 4-byte result on `stream`).  NULL arrays are not
// compared.  PA_OK, INVALID_ARG on a mismatch, or HIP.
pa_status check_metadata(const pa_plan* plan, const int32_t* block_table, const int32_t* qsl,
                         const int32_t* seq_lens, void* stream) {
  const pa::HostPlan& hp = plan->hp;
  const pa_params& p = hp.p;
  if (misaligned(block_table, 4) || misaligned(qsl, 4) || misaligned(seq_lens, 4))
    return set_err(PA_ERR_INVALID_ARG, "metadata arrays must be 4-byte aligned");
  std::lock_guard<std::mutex> lock(const_cast<pa_plan*>(plan)->check_mu);
  int e = pa::launch_check_metadata(block_table, qsl, seq_lens, plan->dev_bt, plan->dev_qsl, plan->dev_seq_lens,
                                    p.num_seqs, p.max_blocks_per_seq, p.block_size, p.num_blocks, plan->dev_check,
                                    stream);
  if (e != 0) return hip_err((hipError_t)e, "metadata check launch");
  int32_t bad = -1;
  hipError_t h = hipMemcpyAsync(&bad, plan->dev_check, sizeof(bad), hipMemcpyDeviceToHost,
                                static_cast<hipStream_t>(stream));
  if (h == hipSuccess) h = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (h != hipSuccess) return hip_err(h, "metadata check");
  if (bad != 0)
    return set_err(PA_ERR_INVALID_ARG,
                   "device metadata differs from the plan's (query_start_loc, seq_lens or block_table): " +
                       std::to_string(bad) + " threads saw a mismatch");
  return PA_OK;
}

// The forward of pa_forward and pa_forward_fp8 after their own checks.
pa_status forward_common(const pa_plan* plan, const void* q, const void* kv_cache, const int32_t* block_table,
                         const int32_t* qsl, const int32_t* seq_lens, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream, const float* k_scale, const float* v_scale,
                         int n_scales) {
  const pa::HostPlan& hp = plan->hp;
  if (hp.T == 0) return PA_OK;
  if (!q || !kv_cache || !block_table || !out) return set_err(PA_ERR_INVALID_ARG, "q/kv_cache/block_table/out is NULL");
  if (workspace_bytes < plan->ws_bytes) return set_err(PA_ERR_INVALID_ARG, "workspace too small");
  if (plan->ws_bytes > 0 && !workspace) return set_err(PA_ERR_INVALID_ARG, "workspace is NULL");
  // the kernels move q, out, the pool and the workspace in 16-byte pieces
  if (misaligned(q, 16) || misaligned(out, 16) || misaligned(kv_cache, 16) ||
      (plan->ws_bytes > 0 && misaligned(workspace, 16)))
    return set_err(PA_ERR_INVALID_ARG, "q, out, kv_cache and workspace must be 16-byte aligned");
  if (misaligned(block_table, 4) || misaligned(lse, 4))
    return set_err(PA_ERR_INVALID_ARG, "block_table and lse must be 4-byte aligned");

  const pa_params& p = hp.p;
  pa::LaunchGeom g{};
  g.H = p.num_heads;
  g.Hkv = p.num_kv_heads;
  g.g = p.num_heads / p.num_kv_heads;
  g.D = p.head_size;
  g.bs = p.block_size;
  g.max_blocks = p.max_blocks_per_seq;
  g.dtype = p.dtype;
  g.kv_dtype = p.kv_dtype;
  pa::pool_strides(p.kv_layout, p.block_size, p.num_kv_heads, p.head_size, g.slot_stride, g.head_stride);
  g.scale_log2 = (float)((double)p.scale * 1.4426950408889634);
  g.ps = hp.ps;

  pa::Tensors t{};
  t.q = q;
  t.kv = kv_cache;
  t.block_table = block_table;
  t.out = out;
  t.lse = lse;
  t.k_scale = k_scale;
  t.v_scale = v_scale;
  t.n_scales = n_scales;
  if (plan->ws_bytes > 0) {
    unsigned char* w = static_cast<unsigned char*>(workspace);
    t.ws_o = reinterpret_cast<float*>(w);
    t.ws_lse = reinterpret_cast<float*>(w + align256((size_t)hp.num_partials * p.num_heads * p.head_size * sizeof(float)));
  }
  DeviceGuard guard(plan->device);
  if (!guard.ok) return set_err(PA_ERR_HIP, "hipSetDevice failed");
  if (p.check_metadata) {
    const pa_status cs = check_metadata(plan, block_table, qsl, seq_lens, stream);
    if (cs != PA_OK) return cs;
  }
  const pa::Streams st{stream, plan->aux, plan->ev_fork, plan->ev_join};
  int e;
  if (plan->aux) {
    std::lock_guard<std::mutex> lock(const_cast<pa_plan*>(plan)->fork_mu);
    e = pa::launch_forward(g, plan->ds, t, st);
  } else {
    e = pa::launch_forward(g, plan->ds, t, st);
  }
  if (e != 0) return hip_err((hipError_t)e, "kernel launch");
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_plan_check_metadata(const pa_plan* plan, const int32_t* block_table, const int32_t* query_start_loc,
                                 const int32_t* seq_lens, void* stream) {
  g_err.clear();
  if (!plan) return set_err(PA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->device < 0) return set_err(PA_ERR_INVALID_ARG, "host-only plan cannot run");
  DeviceGuard guard(plan->device);
  if (!guard.ok) return set_err(PA_ERR_HIP, "hipSetDevice failed");
  return check_metadata(plan, block_table, query_start_loc, seq_lens, stream);
}

pa_status pa_forward(const pa_plan* plan, const void* q, const void* kv_cache, const int32_t* block_table,
                     const int32_t* query_start_loc, const int32_t* seq_lens, void* out, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!plan) return set_err(PA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->device < 0) return set_err(PA_ERR_INVALID_ARG, "host-only plan cannot run");
  if (plan->hp.p.kv_dtype != PA_KV_SAME)
    return set_err(PA_ERR_INVALID_ARG, "the plan's pool holds e4m3 codes: use pa_forward_fp8 with its scales");
  return forward_common(plan, q, kv_cache, block_table, query_start_loc, seq_lens, out, lse, workspace,
                        workspace_bytes, stream, nullptr, nullptr, 0);
}

pa_status pa_forward_fp8(const pa_plan* plan, const void* q, const void* kv_cache, const int32_t* block_table,
                         const int32_t* query_start_loc, const int32_t* seq_lens, const float* k_scale,
                         const float* v_scale, int32_t num_scales, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!plan) return set_err(PA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->device < 0) return set_err(PA_ERR_INVALID_ARG, "host-only plan cannot run");
  const pa_params& p = plan->hp.p;
  if (p.kv_dtype != PA_KV_FP8_E4M3)
    return set_err(PA_ERR_INVALID_ARG, "pa_forward_fp8 needs a plan made with kv_dtype = PA_KV_FP8_E4M3");
  if (num_scales != 1 && num_scales != p.num_kv_heads)
    return set_err(PA_ERR_INVALID_ARG, "num_scales must be 1 or num_kv_heads");
  if (plan->hp.T == 0) return PA_OK;
  if (!k_scale || !v_scale) return set_err(PA_ERR_INVALID_ARG, "k_scale / v_scale is NULL");
  if (misaligned(k_scale, 4) || misaligned(v_scale, 4))
    return set_err(PA_ERR_INVALID_ARG, "k_scale and v_scale must be 4-byte aligned");
  return forward_common(plan, q, kv_cache, block_table, query_start_loc, seq_lens, out, lse, workspace,
                        workspace_bytes, stream, k_scale, v_scale, num_scales);
}

pa_status pa_merge_states(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o_out,
                          float* lse_out, int32_t num_tokens, int32_t num_heads, int32_t head_size, int32_t dtype,
                          void* stream) {
  g_err.clear();
  if (num_tokens < 0 || num_heads < 1) return set_err(PA_ERR_INVALID_ARG, "num_tokens < 0 or num_heads < 1");
  if (dtype != PA_BF16 && dtype != PA_FP32) return set_err(PA_ERR_UNSUPPORTED, "dtype not built");
  if (head_size != 64 && head_size != 128) return set_err(PA_ERR_UNSUPPORTED, "head_size not built (64, 128)");
  if (num_tokens == 0) return PA_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out) return set_err(PA_ERR_INVALID_ARG, "NULL pointer");
  // each thread moves four elements: 8 bytes of bf16, 16 of float32
  const uintptr_t oal = dtype == PA_BF16 ? 8 : 16;
  if (misaligned(o_a, oal) || misaligned(o_b, oal) || misaligned(o_out, oal))
    return set_err(PA_ERR_INVALID_ARG, "o_a, o_b and o_out must be aligned to 4 elements (8 bytes bf16, 16 float32)");
  if (misaligned(lse_a, 4) || misaligned(lse_b, 4) || misaligned(lse_out, 4))
    return set_err(PA_ERR_INVALID_ARG, "lse_a, lse_b and lse_out must be 4-byte aligned");
  const int e = pa::launch_merge_states(o_a, lse_a, o_b, lse_b, o_out, lse_out, num_tokens, num_heads, head_size,
                                        dtype, stream);
  if (e != 0) return hip_err((hipError_t)e, "kernel launch");
  return PA_OK;
}

pa_status pa_gather_kv(const void* kv_cache, const int32_t* block_table_row, int32_t seq_len, const pa_params* params,
                       void* k_out, void* v_out, void* stream) {
  g_err.clear();
  if (!params) return set_err(PA_ERR_INVALID_ARG, "params is NULL");
  if (seq_len < 0) return set_err(PA_ERR_INVALID_ARG, "seq_len < 0");
  if (params->block_size < 16 || params->block_size % 16 != 0)
    return set_err(PA_ERR_INVALID_ARG, "block size must be a positive multiple of 16");
  if (params->num_kv_heads < 1 || params->head_size < 1 || params->head_size % 8 != 0)
    return set_err(PA_ERR_INVALID_ARG, "num_kv_heads >= 1 and head_size a positive multiple of 8 required");
  if (params->dtype != PA_BF16 && params->dtype != PA_FP32) return set_err(PA_ERR_UNSUPPORTED, "dtype not built");
  if (params->kv_dtype != PA_KV_SAME && params->kv_dtype != PA_KV_FP8_E4M3)
    return set_err(PA_ERR_INVALID_ARG, "kv_dtype must be PA_KV_SAME or PA_KV_FP8_E4M3");
  if (params->kv_layout != PA_KV_NHD && params->kv_layout != PA_KV_HND)
    return set_err(PA_ERR_INVALID_ARG, "kv_layout must be PA_KV_NHD or PA_KV_HND");
  const int elem = params->kv_dtype == PA_KV_FP8_E4M3 ? 1 : params->dtype == PA_BF16 ? 2 : 4;
  if ((int64_t)params->head_size * elem % 16 != 0)
    return set_err(PA_ERR_UNSUPPORTED, "a head row (head_size elements) must be a multiple of 16 bytes");
  if ((int64_t)params->block_size * params->head_size > INT32_MAX / 2)
    return set_err(PA_ERR_INVALID_ARG, "block_size * head_size too large");
  if (seq_len == 0) return PA_OK;
  if (!kv_cache || !block_table_row || !k_out || !v_out) return set_err(PA_ERR_INVALID_ARG, "NULL pointer");
  if (misaligned(kv_cache, 16) || misaligned(k_out, 16) || misaligned(v_out, 16) || misaligned(block_table_row, 4))
    return set_err(PA_ERR_INVALID_ARG, "kv_cache, k_out and v_out must be 16-byte aligned, block_table_row 4-byte");
  int ss = 0, hs = 0;
  pa::pool_strides(params->kv_layout, params->block_size, params->num_kv_heads, params->head_size, ss, hs);
  const int e = pa::launch_gather(kv_cache, block_table_row, seq_len, params->block_size, params->num_kv_heads,
                                  params->head_size, elem, ss, hs, k_out, v_out, stream);
  if (e != 0) return hip_err((hipError_t)e, "kernel launch");
  return PA_OK;
}

pa_status pa_write_kv(const void* key, const void* value, const int64_t* slot_mapping, int32_t num_tokens,
                      const pa_params* params, void* kv_cache, void* stream) {
  g_err.clear();
  if (!params) return set_err(PA_ERR_INVALID_ARG, "params is NULL");
  if (num_tokens < 0) return set_err(PA_ERR_INVALID_ARG, "num_tokens < 0");
  if (params->block_size < 16 || params->block_size % 16 != 0)
    return set_err(PA_ERR_INVALID_ARG, "block size must be a positive multiple of 16");
  if (params->num_kv_heads < 1 || params->head_size < 1 || params->num_blocks < 1)
    return set_err(PA_ERR_INVALID_ARG, "num_kv_heads, head_size and num_blocks must be >= 1");
  if (params->dtype != PA_BF16 && params->dtype != PA_FP32) return set_err(PA_ERR_UNSUPPORTED, "dtype not built");
  if (params->kv_dtype != PA_KV_SAME)
    return set_err(PA_ERR_INVALID_ARG, "an e4m3 pool is written by pa_write_kv_fp8 (with its scales)");
  if (params->kv_layout != PA_KV_NHD && params->kv_layout != PA_KV_HND)
    return set_err(PA_ERR_INVALID_ARG, "kv_layout must be PA_KV_NHD or PA_KV_HND");
  const int elem = params->dtype == PA_BF16 ? 2 : 4;
  const int64_t head_bytes = (int64_t)params->head_size * elem;
  const int64_t row_bytes = (int64_t)params->num_kv_heads * head_bytes;
  if (head_bytes % 16 != 0 || row_bytes > INT32_MAX / 2 || (int64_t)params->block_size * head_bytes > INT32_MAX / 2)
    return set_err(PA_ERR_UNSUPPORTED, "a head row (head_size elements) must be a multiple of 16 bytes");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping || !kv_cache) return set_err(PA_ERR_INVALID_ARG, "NULL pointer");
  if ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) | reinterpret_cast<uintptr_t>(kv_cache)) %
          16 != 0)
    return set_err(PA_ERR_INVALID_ARG, "key, value and kv_cache must be 16-byte aligned");
  int ss = 0, hs = 0;
  pa::pool_strides(params->kv_layout, params->block_size, params->num_kv_heads, params->head_size, ss, hs);
  const int e = pa::launch_write_kv(key, value, slot_mapping, num_tokens, params->num_kv_heads, (int)head_bytes,
                                    params->block_size, (int64_t)params->num_blocks * params->block_size,
                                    (int64_t)ss * elem, (int64_t)hs * elem, kv_cache, stream);
  if (e != 0) return hip_err((hipError_t)e, "kernel launch");
  return PA_OK;
}

pa_status pa_write_kv_fp8(const void* key, const void* value, const int64_t* slot_mapping, int32_t num_tokens,
                          const pa_params* params, const float* k_scale, const float* v_scale, int32_t num_scales,
                          void* kv_cache, void* stream) {
  g_err.clear();
  if (!params) return set_err(PA_ERR_INVALID_ARG, "params is NULL");
  if (num_tokens < 0) return set_err(PA_ERR_INVALID_ARG, "num_tokens < 0");
  if (params->block_size < 16 || params->block_size % 16 != 0)
    return set_err(PA_ERR_INVALID_ARG, "block size must be a positive multiple of 16");
  if (params->num_kv_heads < 1 || params->head_size < 1 || params->num_blocks < 1)
    return set_err(PA_ERR_INVALID_ARG, "num_kv_heads, head_size and num_blocks must be >= 1");
  if (params->kv_dtype != PA_KV_FP8_E4M3) return set_err(PA_ERR_INVALID_ARG, "params->kv_dtype is not PA_KV_FP8_E4M3");
  if (params->dtype != PA_BF16) return set_err(PA_ERR_UNSUPPORTED, "e4m3 writes take bf16 key/value");
  if (params->head_size % 16 != 0) return set_err(PA_ERR_UNSUPPORTED, "head_size must be a multiple of 16");
  if (params->kv_layout != PA_KV_NHD && params->kv_layout != PA_KV_HND)
    return set_err(PA_ERR_INVALID_ARG, "kv_layout must be PA_KV_NHD or PA_KV_HND");
  if ((int64_t)params->block_size * params->head_size > INT32_MAX / 2)
    return set_err(PA_ERR_INVALID_ARG, "block_size * head_size too large");
  if ((int64_t)params->num_kv_heads * params->head_size > INT32_MAX / 4)
    return set_err(PA_ERR_INVALID_ARG, "K row too large");
  if (num_scales != 1 && num_scales != params->num_kv_heads)
    return set_err(PA_ERR_INVALID_ARG, "num_scales must be 1 or num_kv_heads");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping || !kv_cache || !k_scale || !v_scale)
    return set_err(PA_ERR_INVALID_ARG, "NULL pointer");
  if ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) | reinterpret_cast<uintptr_t>(kv_cache)) %
          16 != 0)
    return set_err(PA_ERR_INVALID_ARG, "key, value and kv_cache must be 16-byte aligned");
  int ss = 0, hs = 0;
  pa::pool_strides(params->kv_layout, params->block_size, params->num_kv_heads, params->head_size, ss, hs);
  const int e = pa::launch_write_kv_fp8(key, value, slot_mapping, num_tokens, params->num_kv_heads, params->head_size,
                                        params->block_size, (int64_t)params->num_blocks * params->block_size, ss, hs,
                                        k_scale, v_scale, num_scales, kv_cache, stream);
  if (e != 0) return hip_err((hipError_t)e, "kernel launch");
  return PA_OK;
}

void pa_plan_destroy(pa_plan* plan) {
  if (!plan) return;
  if (plan->dev_buf || plan->aux || plan->ev_fork || plan->ev_join) {
    DeviceGuard guard(plan->device);
    if (plan->ev_join) (void)hipEventDestroy(plan->ev_join);
    if (plan->ev_fork) (void)hipEventDestroy(plan->ev_fork);
    if (plan->aux) (void)hipStreamDestroy(plan->aux);
    if (plan->dev_buf) (void)hipFree(plan->dev_buf);
  }
  delete plan;
}

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported";
    case PA_ERR_HIP: return "HIP error";
    case PA_ERR_OOM: return "out of memory";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return g_err.c_str(); }

pa_status pa_profile_start(int32_t max_launches) {
  g_err.clear();
  if (max_launches < 1) return set_err(PA_ERR_INVALID_ARG, "max_launches < 1");
  prof_release();
  g_prof.pool.resize(2 * (size_t)max_launches);
  for (auto& e : g_prof.pool) {
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      e = nullptr;
      g_prof.pool.erase(std::remove(g_prof.pool.begin(), g_prof.pool.end(), nullptr), g_prof.pool.end());
      prof_release();
      return hip_err(r, "hipEventCreate");
    }
  }
  g_prof.max = max_launches;
  g_prof.active = true;
  return PA_OK;
}

pa_status pa_profile_stop(pa_kernel_time* out, int32_t capacity, int32_t* count) {
  g_err.clear();
  if (!g_prof.active) return set_err(PA_ERR_INVALID_ARG, "no profiling session on this thread");
  std::map<std::string, std::vector<double>> agg;
  std::vector<std::string> names;
  pa_status st = PA_OK;
  for (const ProfRec& r : g_prof.recs) {
    hipError_t e = hipEventSynchronize(r.end);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.begin, r.end);
    if (e != hipSuccess) {
      st = hip_err(e, "hipEventElapsedTime");
      break;
    }
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      names.push_back(r.name);
      agg[r.name] = {(double)ms};
    } else {
      it->second.push_back((double)ms);
    }
  }
  prof_release();
  if (st != PA_OK) return st;
  if (count) *count = (int32_t)names.size();
  if ((int32_t)names.size() > capacity || (!out && !names.empty()))
    return set_err(PA_ERR_INVALID_ARG, "capacity too small");
  for (size_t i = 0; i < names.size(); ++i) {
    std::vector<double>& v = agg[names[i]];
    std::sort(v.begin(), v.end());
    const size_t n = v.size();
    std::memset(&out[i], 0, sizeof(pa_kernel_time));
    std::snprintf(out[i].name, sizeof(out[i].name), "%s", names[i].c_str());
    out[i].launches = (int32_t)n;
    for (double x : v) out[i].total_ms += x;
    out[i].min_ms = v.front();
    out[i].max_ms = v.back();
    out[i].median_ms = n % 2 ? v[n / 2] : 0.5 * (v[n / 2 - 1] + v[n / 2]);
  }
  return PA_OK;
}

}  // extern "C"
