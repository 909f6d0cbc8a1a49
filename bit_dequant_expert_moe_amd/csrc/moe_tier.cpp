// moe_tier.cpp -- off-HBM expert tier: experts live in (pinned) host memory,
// a set of expert slots in device memory caches them with least-recently-used
// replacement across all layers, and each layer call copies in only the
// routed experts that miss.
//
// Method: "Flash-MoE: Running a 397B Parameter Model on a Laptop"
// (hysenlabs.com), section "How the SSD expert streaming pipeline works":
// only the K active experts of a layer are read from the slow tier, after the
// routing of that layer is known, and an LRU page cache (the operating
// system's) absorbs the reuse between tokens.  Here the slow tier is host
// memory behind PCIe and the cache is explicit: device slots plus this host
// side table.
//
// One call (moe_tier_decode):
//   1. route on the compute stream (moe_route), ids to pinned staging;
//      the host waits for them (the copies depend on them);
//   2. plan on the host: hits keep their slot, misses take the least
//      recently used slot not used by this call;
//   3. the copy stream waits for the routing event (every kernel that could
//      still read an evicted slot was enqueued before it), copies the missing
//      blobs, and the compute stream waits for the copies;
//   4. slot ids to the device, expert forward over the slots (the same
//      kernels as the resident path, with slot ids in place of expert ids).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "moe_internal.h"

struct moe_tier {
  moe_dims d;
  int n_layers = 0;
  std::vector<const uint8_t *> host;  // per layer: host base of the E blobs
  int64_t host_stride = 0;
  uint8_t *slots = nullptr;
  int64_t slot_stride = 0;
  int n_slots = 0;
  int t_max = 0;
  hipStream_t copy = nullptr;
  int32_t *stage_ids = nullptr;    // pinned host [t_max K]
  int32_t *stage_slots = nullptr;  // pinned host [t_max K]
  int32_t *dev_ids = nullptr;      // device [t_max K]
  float *dev_w = nullptr;          // device [t_max K]
  int32_t *dev_slots = nullptr;    // device [t_max K]
  // least-recently-used list over the slots: head = most recent
  std::vector<int64_t> key;        // (layer E + expert) held by a slot, -1 = empty
  std::vector<int> prev, next;
  int head = -1, tail = -1;
  std::unordered_map<int64_t, int> where;
  std::vector<uint32_t> mark;      // call number that last used a slot
  uint32_t call = 0;
  std::vector<int32_t> copy_expert;  // per slot id of the current call: expert to copy, or -1
  hipEvent_t ev_ids = nullptr, ev_copy = nullptr;
  int64_t hits = 0, misses = 0, bytes = 0, evictions = 0;
};

namespace {

using namespace moe;

size_t region(const moe_dims &d, int t_max) {
  return align_up((size_t)t_max * d.top_k * 4, kAlign);
}

void unlink(moe_tier *t, int s) {
  if (t->prev[s] >= 0) t->next[t->prev[s]] = t->next[s];
  else t->head = t->next[s];
  if (t->next[s] >= 0) t->prev[t->next[s]] = t->prev[s];
  else t->tail = t->prev[s];
  t->prev[s] = t->next[s] = -1;
}

void push_front(moe_tier *t, int s) {
  t->prev[s] = -1;
  t->next[s] = t->head;
  if (t->head >= 0) t->prev[t->head] = s;
  t->head = s;
  if (t->tail < 0) t->tail = s;
}

// Slot ids for the n expert ids of one call of `layer` (ids outside [0, E)
// map to -1, which the expert forward turns into a zero contribution and the
// sticky error flag).  Misses are listed in copy_expert.
void plan(moe_tier *t, int layer, const int32_t *ids, int n, int32_t *slot_out) {
  ++t->call;
  t->copy_expert.assign((size_t)n, -1);
  for (int i = 0; i < n; ++i) {
    const int e = ids[i];
    if (e < 0 || e >= t->d.n_experts) {
      slot_out[i] = -1;
      continue;
    }
    const int64_t k = (int64_t)layer * t->d.n_experts + e;
    auto it = t->where.find(k);
    int s;
    if (it != t->where.end()) {
      s = it->second;
      if (t->mark[s] != t->call) ++t->hits;  // a repeat inside one call is no new hit
      unlink(t, s);
    } else {
      // least recently used slot that this call does not use
      s = t->tail;
      while (s >= 0 && t->mark[s] == t->call) s = t->prev[s];
      // (n <= t_max K <= n_slots, so a free one exists)
      if (t->key[s] >= 0) {
        t->where.erase(t->key[s]);
        ++t->evictions;
      }
      unlink(t, s);
      t->key[s] = k;
      t->where[k] = s;
      t->copy_expert[i] = e;
      ++t->misses;
      t->bytes += (int64_t)blob_layout(t->d).off[6];
    }
    t->mark[s] = t->call;
    push_front(t, s);
    slot_out[i] = s;
  }
}

}  // namespace

using namespace moe;

extern "C" {

size_t moe_tier_staging_bytes(const moe_dims *dims, int32_t t_max) {
  if (moe_check_dims(dims) != MOE_OK || t_max < 1 || t_max > kMaxT) return 0;
  return 2 * region(*dims, t_max);
}

size_t moe_tier_device_bytes(const moe_dims *dims, int32_t t_max) {
  if (moe_check_dims(dims) != MOE_OK || t_max < 1 || t_max > kMaxT) return 0;
  return 3 * region(*dims, t_max);
}

size_t moe_tier_workspace_bytes(const moe_dims *dims, int32_t n_slots, int32_t T) {
  if (moe_check_dims(dims) != MOE_OK || n_slots < 1 || n_slots > kMaxE) return 0;
  moe_dims ds = *dims;
  ds.n_experts = n_slots;
  const size_t a = moe_workspace_bytes(dims, T), b = moe_workspace_bytes(&ds, T);
  if (a == 0 || b == 0) return 0;
  return a > b ? a : b;
}

moe_status moe_tier_create(const moe_dims *dims, const moe_tier_config *cfg, moe_tier **out) {
  if (!out) return MOE_ERR_NULL;
  *out = nullptr;
  moe_status st = moe_check_dims(dims);
  if (st != MOE_OK) return st;
  if (!cfg || !cfg->host_experts || !cfg->slots || !cfg->staging || !cfg->dev_scratch)
    return MOE_ERR_NULL;
  const size_t blob = blob_layout(*dims).off[6];
  if (cfg->n_layers < 1 || cfg->t_max < 1 || cfg->t_max > kMaxT) return MOE_ERR_SHAPE;
  if (cfg->n_slots < cfg->t_max * dims->top_k || cfg->n_slots > kMaxE) return MOE_ERR_SHAPE;
  if (cfg->host_stride < (int64_t)blob || cfg->slot_stride < (int64_t)blob) return MOE_ERR_SHAPE;
  if (cfg->slot_stride % (int64_t)kAlign || (reinterpret_cast<uintptr_t>(cfg->slots) % kAlign) ||
      (reinterpret_cast<uintptr_t>(cfg->dev_scratch) % kAlign) ||
      (reinterpret_cast<uintptr_t>(cfg->staging) % 16))
    return MOE_ERR_ALIGN;
  for (int l = 0; l < cfg->n_layers; ++l)
    if (!cfg->host_experts[l]) return MOE_ERR_NULL;
  moe_tier *t = new (std::nothrow) moe_tier;
  if (!t) return MOE_ERR_SHAPE;
  t->d = *dims;
  t->n_layers = cfg->n_layers;
  t->host.assign(cfg->host_experts, cfg->host_experts + cfg->n_layers);
  t->host_stride = cfg->host_stride;
  t->slots = static_cast<uint8_t *>(cfg->slots);
  t->slot_stride = cfg->slot_stride;
  t->n_slots = cfg->n_slots;
  t->t_max = cfg->t_max;
  t->copy = static_cast<hipStream_t>(cfg->copy_stream);
  const size_t r = region(*dims, cfg->t_max);
  uint8_t *sg = static_cast<uint8_t *>(cfg->staging);
  t->stage_ids = reinterpret_cast<int32_t *>(sg);
  t->stage_slots = reinterpret_cast<int32_t *>(sg + r);
  uint8_t *dv = static_cast<uint8_t *>(cfg->dev_scratch);
  t->dev_ids = reinterpret_cast<int32_t *>(dv);
  t->dev_w = reinterpret_cast<float *>(dv + r);
  t->dev_slots = reinterpret_cast<int32_t *>(dv + 2 * r);
  t->key.assign((size_t)t->n_slots, -1);
  t->prev.assign((size_t)t->n_slots, -1);
  t->next.assign((size_t)t->n_slots, -1);
  t->mark.assign((size_t)t->n_slots, 0u);
  for (int s = t->n_slots - 1; s >= 0; --s) push_front(t, s);  // slot 0 most recent
  *out = t;
  return MOE_OK;
}

moe_status moe_tier_plan(moe_tier *t, int32_t layer, const int32_t *ids, int32_t T,
                         int32_t *slot_ids, int32_t *copy_expert) {
  if (!t || !ids || !slot_ids) return MOE_ERR_NULL;
  if (layer < 0 || layer >= t->n_layers || T < 1 || T > t->t_max) return MOE_ERR_SHAPE;
  const int n = T * t->d.top_k;
  plan(t, layer, ids, n, slot_ids);
  if (copy_expert) memcpy(copy_expert, t->copy_expert.data(), (size_t)n * 4);
  return MOE_OK;
}

moe_status moe_tier_decode(moe_tier *t, int32_t layer, const uint16_t *router,
                           const uint8_t *shared, const uint16_t *x, int32_t T, float *y,
                           int32_t *ids, float *w, void *ws, size_t ws_bytes, void *stream) {
  if (!t || !router || !x || !y || !ws) return MOE_ERR_NULL;
  if (layer < 0 || layer >= t->n_layers || T < 1 || T > t->t_max) return MOE_ERR_SHAPE;
  if (t->d.has_shared && !shared) return MOE_ERR_NULL;
  if (!t->d.has_shared && shared) return MOE_ERR_SHAPE;
  if (ws_bytes < moe_tier_workspace_bytes(&t->d, t->n_slots, T)) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!t->ev_ids) {
    if (hipEventCreateWithFlags(&t->ev_ids, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&t->ev_copy, hipEventDisableTiming) != hipSuccess)
      return MOE_ERR_HIP;
  }
  const int n = T * t->d.top_k;
  int32_t *ids_d = ids ? ids : t->dev_ids;
  float *w_d = w ? w : t->dev_w;
  moe_status s = moe_route(&t->d, router, x, T, ids_d, w_d, nullptr, ws, ws_bytes, stream);
  if (s != MOE_OK) return s;
  if (hipMemcpyAsync(t->stage_ids, ids_d, (size_t)n * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipEventRecord(t->ev_ids, st) != hipSuccess || hipEventSynchronize(t->ev_ids) != hipSuccess)
    return MOE_ERR_HIP;
  plan(t, layer, t->stage_ids, n, t->stage_slots);
  const size_t blob = blob_layout(t->d).off[6];
  bool copied = false;
  for (int i = 0; i < n; ++i) {
    const int e = t->copy_expert[(size_t)i];
    if (e < 0) continue;
    if (!copied && hipStreamWaitEvent(t->copy, t->ev_ids, 0) != hipSuccess) return MOE_ERR_HIP;
    copied = true;
    const uint8_t *src = t->host[(size_t)layer] + (size_t)e * t->host_stride;
    uint8_t *dst = t->slots + (size_t)t->stage_slots[i] * t->slot_stride;
    if (hipMemcpyAsync(dst, src, blob, hipMemcpyHostToDevice, t->copy) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (copied && (hipEventRecord(t->ev_copy, t->copy) != hipSuccess ||
                 hipStreamWaitEvent(st, t->ev_copy, 0) != hipSuccess))
    return MOE_ERR_HIP;
  if (hipMemcpyAsync(t->dev_slots, t->stage_slots, (size_t)n * 4, hipMemcpyHostToDevice, st) !=
      hipSuccess)
    return MOE_ERR_HIP;
  moe_dims ds = t->d;
  ds.n_experts = t->n_slots;
  moe_layer Ls;
  Ls.router = router;
  Ls.experts = t->slots;
  Ls.expert_stride = t->slot_stride;
  Ls.shared = shared;
  return moe_expert_forward(&ds, &Ls, x, T, t->dev_slots, w_d, y, ws, ws_bytes, stream);
}

moe_status moe_tier_stats(const moe_tier *t, int64_t out[4]) {
  if (!t || !out) return MOE_ERR_NULL;
  out[0] = t->hits;
  out[1] = t->misses;
  out[2] = t->bytes;
  out[3] = t->evictions;
  return MOE_OK;
}

void moe_tier_destroy(moe_tier *t) {
  if (!t) return;
  if (t->ev_ids) (void)hipEventDestroy(t->ev_ids);
  if (t->ev_copy) (void)hipEventDestroy(t->ev_copy);
  delete t;
}

}  // extern "C"
