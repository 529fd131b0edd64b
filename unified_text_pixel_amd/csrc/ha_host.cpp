// C-ABI entry points: host-side validation (before any HIP call), workspace layout and
// kernel dispatch. The declarations and the contract are in include/ha_attn.h.
//
// Validation follows the convention of the hidream-o1-p100a model card ("Serving (HTTP)":
// contract errors are rejected without touching the card): every check runs on the host
// and a failed check returns before the device or the stream is used.
#include "ha_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <string>
#include <vector>

#include "ha_internal.h"

namespace {

thread_local std::string g_last_error;

ha_status fail(ha_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ha_status ok() {
  g_last_error.clear();
  return HA_OK;
}

// HA_DEBUG=1, read at each call: synchronise after every launch and check positions
bool debug_sync() {
  const char* e = std::getenv("HA_DEBUG");
  return e && e[0] == '1';
}

ha_status check_launch(hipError_t e, hipStream_t stream, const char* what) {
  if (e != hipSuccess) return fail(HA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(HA_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
  }
  return HA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- descriptor checks
ha_status check_desc(const ha_attn_desc* d) {
  if (!d) return fail(HA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0 || d->seq_len < 0)
    return fail(HA_ERR_INVALID_ARG, "batch (%d) and seq_len (%d) must be >= 0", d->batch, d->seq_len);
  if (d->seq_len > HA_MAX_SEQ_LEN)
    return fail(HA_ERR_UNSUPPORTED, "seq_len %d exceeds %d", d->seq_len, HA_MAX_SEQ_LEN);
  if (d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(HA_ERR_INVALID_ARG, "head counts must be >= 1 (got %d, %d)", d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(HA_ERR_INVALID_ARG, "n_q_heads %d is not a multiple of n_kv_heads %d", d->n_q_heads,
                d->n_kv_heads);
  const int group = d->n_q_heads / d->n_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(HA_ERR_UNSUPPORTED, "n_q_heads / n_kv_heads = %d; supported: 1, 2, 4, 8", group);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(HA_ERR_UNSUPPORTED, "head_dim %d; supported: 64, 128", d->head_dim);
  if (d->dtype != HA_DTYPE_BF16 && d->dtype != HA_DTYPE_F32)
    return fail(HA_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (!std::isfinite(d->scale) || d->scale < 0.f)
    return fail(HA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (d->q_prescaled != 0 && d->q_prescaled != 1)
    return fail(HA_ERR_INVALID_ARG, "q_prescaled must be 0 or 1");
  if (d->split_parts < 0 || d->split_parts > 64)
    return fail(HA_ERR_INVALID_ARG, "split_parts %d outside [0, 64]", d->split_parts);
  if (d->plan_cus < 0) return fail(HA_ERR_INVALID_ARG, "plan_cus %d must be >= 0", d->plan_cus);
  if ((int64_t)d->n_q_heads * d->head_dim * (int64_t)d->seq_len * (d->batch ? d->batch : 1) >
      (int64_t(1) << 40))
    return fail(HA_ERR_UNSUPPORTED, "tensor too large");
  if (d->batch == 0 || d->seq_len == 0) return HA_OK;  // empty: segments not consulted
  if (!d->segments) return fail(HA_ERR_INVALID_ARG, "segments is NULL");
  if (d->n_segments < 1 || d->n_segments > HA_MAX_SEGMENTS)
    return fail(HA_ERR_SEGMENTS, "n_segments %d outside [1, %d]", d->n_segments, HA_MAX_SEGMENTS);
  for (int b = 0; b < d->batch; ++b) {
    int64_t at = 0;
    for (int s = 0; s < d->n_segments; ++s) {
      const ha_segment& g = d->segments[(int64_t)b * d->n_segments + s];
      if (g.kind != HA_SEG_CAUSAL && g.kind != HA_SEG_FULL && g.kind != HA_SEG_GCA && g.kind != HA_SEG_GEN)
        return fail(HA_ERR_SEGMENTS, "batch %d segment %d: unknown kind %d", b, s, g.kind);
      if (g.length <= 0)
        return fail(HA_ERR_SEGMENTS, "batch %d segment %d: length %d must be > 0", b, s, g.length);
      if (g.start != at)
        return fail(HA_ERR_SEGMENTS, "batch %d segment %d: starts at %d, expected %lld", b, s, g.start,
                    (long long)at);
      at += g.length;
    }
    if (at != d->seq_len)
      return fail(HA_ERR_SEGMENTS, "batch %d: segments cover %lld tokens, seq_len is %d", b, (long long)at,
                  d->seq_len);
  }
  return HA_OK;
}

bool empty(const ha_attn_desc* d) { return d->batch == 0 || d->seq_len == 0; }

// Some segment is a Gen Image (its keys are hidden from the tokens after it).
bool has_gen(const ha_attn_desc* d) {
  if (empty(d)) return false;
  for (int64_t t = 0; t < (int64_t)d->batch * d->n_segments; ++t)
    if (d->segments[t].kind == HA_SEG_GEN) return true;
  return false;
}

// Plan arrays of a layout with Gen Images (null otherwise): key visibility and per query
// block tile lists, written by the classifier and read by the attention kernels.
struct HolePlan {
  int32_t* key_vis = nullptr;
  int32_t* tiles = nullptr;
  int32_t* tile_count = nullptr;
};

ha_status check_tensor(const void* p, const char* name) {
  if (!p) return fail(HA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(HA_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  return HA_OK;
}

int n_axes_of(int rope_kind) { return rope_kind == HA_ROPE_2D ? 2 : (rope_kind == HA_ROPE_MROPE ? 3 : 1); }

ha_status check_prologue(const ha_attn_desc* d, const ha_prologue_desc* p) {
  if (!p) return fail(HA_ERR_INVALID_ARG, "prologue desc is NULL");
  if (p->rope_kind < HA_ROPE_NONE || p->rope_kind > HA_ROPE_MROPE)
    return fail(HA_ERR_INVALID_ARG, "unknown rope_kind %d", p->rope_kind);
  if (p->rope_kind == HA_ROPE_MROPE) {
    const int* s = p->mrope_sections;
    if (s[0] < 0 || s[1] < 0 || s[2] < 0 || s[0] + s[1] + s[2] != d->head_dim / 2)
      return fail(HA_ERR_INVALID_ARG, "mrope_sections (%d, %d, %d) must be >= 0 and sum to %d", s[0], s[1],
                  s[2], d->head_dim / 2);
  }
  if (p->rope_kind != HA_ROPE_NONE) {
    if (!p->positions || !p->cos_sin) return fail(HA_ERR_INVALID_ARG, "positions and cos_sin are required");
    if (!aligned(p->positions, 4) || !aligned(p->cos_sin, 8))
      return fail(HA_ERR_ALIGNMENT, "positions (4) or cos_sin (8) misaligned");
    if (p->n_pos < 1) return fail(HA_ERR_INVALID_ARG, "n_pos must be >= 1");
  }
  if ((p->q_norm_weight == nullptr) != (p->k_norm_weight == nullptr))
    return fail(HA_ERR_INVALID_ARG, "q_norm_weight and k_norm_weight must both be set or both NULL");
  if (p->q_norm_weight) {
    if (!aligned(p->q_norm_weight, 4) || !aligned(p->k_norm_weight, 4))
      return fail(HA_ERR_ALIGNMENT, "norm weights must be 4-byte aligned");
    if (!std::isfinite(p->eps) || p->eps < 0.f) return fail(HA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  }
  if (!std::isfinite(p->q_out_scale) || p->q_out_scale < 0.f)
    return fail(HA_ERR_INVALID_ARG, "q_out_scale must be finite and >= 0");
  if ((d->n_q_heads + d->n_kv_heads) * (d->head_dim / 16) > 1024)
    return fail(HA_ERR_UNSUPPORTED, "prologue: (n_q_heads + n_kv_heads) * head_dim / 16 must be <= 1024");
  return HA_OK;
}

void tile_shape(const ha_attn_desc* d, int* bq, int* bk, int* nq, int* nk) {
  *bq = ha::attn_block_q(d->head_dim, d->n_q_heads / d->n_kv_heads, d->dtype == HA_DTYPE_F32);
  *bk = ha::kBlockK;
  *nq = (int)cdiv(d->seq_len, *bq);
  *nk = (int)cdiv(d->seq_len, *bk);
}

// Launch the classifier over batch chunks whose segment tables fit the kernel arguments.
ha_status run_classify(const ha_attn_desc* d, uint8_t* labels, int32_t* ranges, int32_t* row_limit,
                       hipStream_t stream, const HolePlan& hole = HolePlan{}) {
  ha::ClassifyArgs a{};
  int bq, bk, nq, nk;
  tile_shape(d, &bq, &bk, &nq, &nk);
  a.S = d->seq_len;
  a.nq = nq;
  a.nk = nk;
  a.bq = bq;
  a.bk = bk;
  a.labels = labels;
  a.ranges = ranges;
  a.row_limit = row_limit;
  a.has_gen = has_gen(d);
  a.key_vis = hole.key_vis;
  a.tiles = hole.tiles;
  a.tile_count = hole.tile_count;
  a.kv_stride = ha::key_vis_stride(d->seq_len);
  const int per_launch = ha::kArgSegs / d->n_segments;
  for (int b0 = 0; b0 < d->batch; b0 += per_launch) {
    const int n = std::min(per_launch, d->batch - b0);
    a.seg.n_items = n;
    a.seg.b0 = b0;
    a.seg.n_seg = d->n_segments;
    for (int t = 0; t < n * d->n_segments; ++t) {
      const ha_segment& g = d->segments[(int64_t)b0 * d->n_segments + t];
      a.seg.start[t] = g.start;
      a.seg.end[t] = g.start + g.length;
      a.seg.kind[t] = g.kind;
    }
    ha_status st = check_launch(ha::launch_classify(a, stream), stream, "classifier");
    if (st != HA_OK) return st;
  }
  return HA_OK;
}

void axis_table(const ha_prologue_desc* p, int head_dim, uint8_t* axis) {
  const int half = head_dim / 2;
  if (p->rope_kind == HA_ROPE_2D) {
    for (int i = 0; i < half; ++i) axis[i] = (uint8_t)(i & 1);
  } else if (p->rope_kind == HA_ROPE_MROPE) {
    // deal pairs to T, H, W in turn; an axis leaves the rotation once it holds its count
    int left[3] = {p->mrope_sections[0], p->mrope_sections[1], p->mrope_sections[2]};
    int ax = 0;
    for (int i = 0; i < half;) {
      if (left[ax] > 0) {
        axis[i++] = (uint8_t)ax;
        --left[ax];
      }
      ax = (ax + 1) % 3;
    }
  } else {
    for (int i = 0; i < half; ++i) axis[i] = 0;
  }
}

double softmax_scale(const ha_attn_desc* d) {
  return d->scale > 0.f ? (double)d->scale : 1.0 / std::sqrt((double)d->head_dim);
}

float q_prescale(const ha_attn_desc* d) { return (float)(softmax_scale(d) * 1.4426950408889634074); }

ha_status run_prologue(const ha_attn_desc* d, const ha_prologue_desc* p, const void* q_in, const void* k_in,
                       void* q_out, void* k_out, float q_scale, hipStream_t stream, int token_begin = 0) {
  ha::PrologueArgs a{};
  a.q_in = q_in;
  a.k_in = k_in;
  a.q_out = q_out;
  a.k_out = k_out;
  a.rotate = p->rope_kind != HA_ROPE_NONE;
  a.positions = a.rotate ? p->positions : nullptr;
  a.cos_sin = a.rotate ? p->cos_sin : nullptr;
  a.wq = p->q_norm_weight;
  a.wk = p->k_norm_weight;
  a.B = d->batch;
  a.S = d->seq_len;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.D = d->head_dim;
  a.n_axes = n_axes_of(p->rope_kind);
  a.n_pos = p->n_pos;
  a.eps = p->eps;
  a.q_scale = q_scale;
  a.f32 = d->dtype == HA_DTYPE_F32;
  a.token_begin = token_begin;
  axis_table(p, d->head_dim, a.axis);
  return check_launch(ha::launch_prologue(a, stream), stream, "prologue");
}

// HA_DEBUG: every rotary position of the call in [0, n_pos), checked on the device before
// any kernel reads it (the positions of all batch items and tokens; a caller reusing a
// prefix passes the same table). Without HA_DEBUG nothing is launched here.
ha_status check_positions_debug(const ha_attn_desc* d, const ha_prologue_desc* p, hipStream_t stream) {
  if (!p || p->rope_kind == HA_ROPE_NONE || !debug_sync() || empty(d)) return HA_OK;
  const int64_t count = (int64_t)d->batch * d->seq_len * n_axes_of(p->rope_kind);
  int64_t bad = -1;
  int32_t value = 0;
  const hipError_t e = ha::check_positions(p->positions, count, p->n_pos, stream, &bad, &value);
  if (e != hipSuccess) return fail(HA_ERR_HIP, "position check failed: %s", hipGetErrorString(e));
  if (bad >= 0) {
    const int A = n_axes_of(p->rope_kind);
    const int64_t tok = bad / A;
    return fail(HA_ERR_INVALID_ARG, "positions[%lld][%lld][%d] = %d outside [0, n_pos %d)",
                (long long)(tok / d->seq_len), (long long)(tok % d->seq_len), (int)(bad % A), value, p->n_pos);
  }
  return HA_OK;
}

int plan_cus(const ha_attn_desc* d);

// split query blocks on the device (null items: one work item per query block)
struct SplitRun {
  int32_t* items = nullptr;
  int n_items = 0;
  float* part_o = nullptr;
  float* part_l = nullptr;
  float* part_m = nullptr;
};

ha_status run_attn(const ha_attn_desc* d, const void* q, const void* k, const void* v, const int32_t* row_limit,
                   const int32_t* ranges, void* out, bool prescaled, hipStream_t stream, float* lse = nullptr,
                   int row_begin = 0, const HolePlan& hole = HolePlan{}, const SplitRun& split = SplitRun{}) {
  ha::AttnArgs a{};
  int bq, bk, nq, nk;
  tile_shape(d, &bq, &bk, &nq, &nk);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.row_limit = row_limit;
  a.ranges = ranges;
  a.B = d->batch;
  a.S = d->seq_len;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.D = d->head_dim;
  a.nq = nq;
  a.scale_log2e = q_prescale(d);
  a.q_prescaled = prescaled;
  a.f32 = d->dtype == HA_DTYPE_F32;
  a.lse = lse;
  // the query blocks holding rows >= row_begin: blocks end at S, so that is the last
  // ceil((S - row_begin) / bq) of them
  a.nq_run = (int)cdiv(d->seq_len - row_begin, bq);
  a.row_begin = row_begin;
  a.key_vis = hole.key_vis;
  a.tiles = hole.tiles;
  a.tile_count = hole.tile_count;
  a.kv_stride = ha::key_vis_stride(d->seq_len);
  a.nk = nk;
  a.items = split.items;
  a.n_items = split.n_items;
  a.part_o = split.part_o;
  a.part_l = split.part_l;
  a.part_m = split.part_m;
  // fewer work items than CUs (plain tile ranges): one workgroup per 32-row slice
  a.slices = 1;
  if (!hole.key_vis && !split.items &&
      (int64_t)d->batch * d->n_kv_heads * a.nq_run < plan_cus(d))
    a.slices = ha::attn_slices(d->head_dim, d->n_q_heads / d->n_kv_heads, a.f32 != 0);
  return check_launch(ha::launch_attn(a, stream), stream, "attention");
}

// ---------------------------------------------------------------- split query blocks
// Load balance of the bf16 forward (the workspace entry points). One work item per (batch,
// KV head, query block) can leave the CUs idle: with the HunyuanImage interleave each XCD
// serves one (batch, KV head) pair, 66 blocks of ~92 tiles on 32 CUs, so two of them run
// alone in a third round. The planner sorts each XCD's items by their tile count and splits
// the heavy items past the last whole round into parts that walk shares of their key tiles;
// it picks the part count by simulating list scheduling (the hardware dispatches in table
// order to the CU that frees up first). A merge kernel combines the parts.

// CUs the planner balances over: desc->plan_cus, else the current device's count
int plan_cus(const ha_attn_desc* d) {
  if (d->plan_cus > 0) return d->plan_cus;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

// The host's part of a split plan: per XCD group, how many items it has, which positions of
// its cost-sorted list are split and into how many parts, and where its slots and split
// table rows start. The device builds the table itself (ha::launch_plan).
struct SplitPlan {
  bool active = false;
  int groups = 0, affine = 0, longest = 0;
  int n_items = 0, n_slots = 0, n_splits = 0;
  int n[ha::kPlanGroups] = {}, best[ha::kPlanGroups] = {}, k[ha::kPlanGroups] = {};
  int heavy[ha::kPlanGroups] = {}, slot_base[ha::kPlanGroups] = {}, split_base[ha::kPlanGroups] = {};
  int len[ha::kPlanGroups] = {};
};

// Key tiles each query block of batch item b executes, from the segment table: the tiles
// before its rows' largest key limit, less, with Gen Images, the tiles whose every key is
// hidden from the block's first row (the tile classifier's SKIP rule, so these are the
// counts the classifier writes and the device plan sorts by).
std::vector<int> block_costs(const ha_attn_desc* d, int b, int bq, int nq, int nk) {
  const int S = d->seq_len, bk = ha::kBlockK;
  const ha_segment* seg = d->segments + (int64_t)b * d->n_segments;
  std::vector<int> vmax;  // per key tile: the largest visibility end of its keys
  if (has_gen(d)) {
    vmax.assign(nk, 0);
    for (int s = 0; s < d->n_segments; ++s) {
      const int st = seg[s].start, en = st + seg[s].length;
      for (int kb = st / bk; kb < nk && kb * bk < en; ++kb)
        vmax[kb] = std::max(vmax[kb], seg[s].kind == HA_SEG_GEN ? en : S);
    }
  }
  std::vector<int> cost(nq);
  for (int qb = 0; qb < nq; ++qb) {
    const int r1 = S - (nq - 1 - qb) * bq, r0 = std::max(0, r1 - bq);
    int lmax = 0;
    for (int s = 0; s < d->n_segments; ++s) {
      const int st = seg[s].start, en = st + seg[s].length;
      if (en <= r0 || st >= r1) continue;
      lmax = std::max(lmax, seg[s].kind == HA_SEG_CAUSAL ? std::min(en, r1) : (seg[s].kind == HA_SEG_FULL ? S : en));
    }
    const int kend = (lmax + bk - 1) / bk;
    int n = kend;
    if (!vmax.empty())
      for (int kb = 0; kb < kend; ++kb) n -= vmax[kb] <= r0 ? 1 : 0;
    cost[qb] = n;
  }
  return cost;
}

// makespan of list scheduling in the given order on n machines
// (loads: the machines' loads, a min-heap reused between calls)
double list_schedule(const std::vector<double>& costs, int n, std::vector<double>& loads) {
  loads.assign(n, 0.0);  // all equal: already a heap
  double ms = 0.0;
  for (double c : costs) {
    std::pop_heap(loads.begin(), loads.end(), std::greater<double>());
    loads.back() += c;
    ms = std::max(ms, loads.back());
    std::push_heap(loads.begin(), loads.end(), std::greater<double>());
  }
  return ms;
}

// desc->split_parts: 1 never splits, P > 1 splits every query block into P parts.
SplitPlan plan_split(const ha_attn_desc* d) {
  SplitPlan plan;
  if (d->dtype != HA_DTYPE_BF16 || empty(d)) return plan;
  const int force = d->split_parts;
  if (force == 1) return plan;
  const int n_cus = plan_cus(d);
  if (n_cus <= 0) return plan;
  int bq, bk, nq, nk;
  tile_shape(d, &bq, &bk, &nq, &nk);
  const int nbg = d->batch * d->n_kv_heads;
  const bool affine = nbg % 8 == 0;  // the unsplit order keeps each pair on one XCD
  const int groups = affine ? 8 : 1;
  if ((int64_t)(nbg / groups) * nq > ha::kPlanMaxItems) return plan;  // the device sort's limit
  const int cus = std::max(1, affine ? n_cus / 8 : n_cus);
  constexpr double kItem = 4.0;  // fixed cost of a work item (start, last tile, stores), in tiles
  // This runs on the host at every call, so its buffers are reused: the block costs of each
  // batch item (made on first use), a group's costs, the two sorted runs of a candidate
  // list, the list and the machine loads of the simulation.
  std::vector<std::vector<int>> costs(d->batch);
  std::vector<int> it, prev_it;
  std::vector<double> whole_c, part_c, c, loads;
  int prev_best = 1;
  int slot = 0, n_splits = 0, longest = 0;
  for (int x = 0; x < groups; ++x) {
    it.clear();  // costs in the group's item order: pairs x, x + 8, ..., blocks from the last
    for (int bg = affine ? x : 0; bg < nbg; bg += affine ? 8 : 1) {
      const int b = bg / d->n_kv_heads;
      if (costs[b].empty()) costs[b] = block_costs(d, b, bq, nq, nk);
      for (int qb = nq - 1; qb >= 0; --qb) it.push_back(costs[b][qb]);
    }
    std::sort(it.begin(), it.end(), std::greater<int>());  // equal costs are interchangeable
    const int n = (int)it.size();
    int best = 1, k = 0, heavy = 0;
    if (n > 0) {
      const int cmax = it[0];
      while (heavy < n && 4 * it[heavy] >= 3 * cmax) ++heavy;
      k = heavy / cus * cus;  // the heavy items that fill whole rounds stay whole
      if (force > 1) {
        k = 0;
        heavy = n;
        best = force;
      } else if (x > 0 && it == prev_it) {
        best = prev_best;  // the same sorted costs as the previous group: the same decision
      } else if (k < heavy) {  // else no heavy item is left to split
        double best_ms = 0.0, whole_ms = 0.0;
        for (int parts : {1, 2, 3, 4, 6, 8, 12, 16, 24, 32}) {
          if (parts > 1 && parts > cmax) break;
          // the candidate list in descending cost: the whole items (it is sorted, so they
          // are) merged with the parts of the split ones (sorted too); the makespan of list
          // scheduling does not depend on the order among equal costs
          whole_c.clear();
          part_c.clear();
          for (int i = 0; i < n; ++i) {
            if (parts > 1 && i >= k && i < heavy) {
              const double pc = std::ceil((double)it[i] / parts) + kItem;
              for (int p = 0; p < parts; ++p) part_c.push_back(pc);
            } else {
              whole_c.push_back((double)it[i] + kItem);
            }
          }
          c.resize(whole_c.size() + part_c.size());
          std::merge(whole_c.begin(), whole_c.end(), part_c.begin(), part_c.end(), c.begin(),
                     std::greater<double>());
          const double ms = list_schedule(c, cus, loads) + (parts > 1 ? kItem : 0.0);  // + the merge
          if (parts == 1) whole_ms = ms;
          if (parts == 1 || ms < best_ms) {
            best = parts;
            best_ms = ms;
          }
        }
        if (best_ms > 0.97 * whole_ms) best = 1;  // not worth a merge
      }
      prev_it.swap(it);  // it is rebuilt for the next group
      prev_best = best;
    }
    plan.n[x] = n;
    plan.best[x] = best;
    plan.k[x] = k;
    plan.heavy[x] = heavy;
    plan.slot_base[x] = slot;
    plan.split_base[x] = n_splits;
    plan.len[x] = best > 1 ? n + (heavy - k) * (best - 1) : n;
    if (best > 1) {
      slot += (heavy - k) * best;
      n_splits += heavy - k;
    }
    longest = std::max(longest, plan.len[x]);
  }
  if (slot == 0) return plan;  // nothing to split: the unsplit order is as good
  plan.groups = groups;
  plan.affine = affine ? 1 : 0;
  plan.longest = longest;
  plan.n_items = longest * groups;
  plan.n_slots = slot;
  plan.n_splits = n_splits;
  plan.active = true;
  return plan;
}

struct Workspace {
  size_t row_limit, ranges, q_rot, k_rot, key_vis, tiles, tile_count, total;
  size_t items, part_o, part_l, part_m;  // split query blocks: items, then the split table
};

// Bytes of the Gen Image plan arrays, placed at *at (offsets into the workspace).
void take_hole(const ha_attn_desc* d, int nq, int nk, size_t* at, size_t* key_vis, size_t* tiles,
               size_t* tile_count) {
  *key_vis = *at;
  *at = round256(*at + (size_t)d->batch * ha::key_vis_stride(d->seq_len) * 4);
  *tiles = *at;
  *at = round256(*at + (size_t)d->batch * nq * nk * 4);
  *tile_count = *at;
  *at = round256(*at + (size_t)d->batch * nq * 2 * 4);
}

HolePlan hole_plan(const ha_attn_desc* d, char* ws, size_t key_vis, size_t tiles, size_t tile_count) {
  HolePlan h;
  if (!has_gen(d)) return h;
  h.key_vis = reinterpret_cast<int32_t*>(ws + key_vis);
  h.tiles = reinterpret_cast<int32_t*>(ws + tiles);
  h.tile_count = reinterpret_cast<int32_t*>(ws + tile_count);
  return h;
}

Workspace workspace_layout(const ha_attn_desc* d, bool prologue, const SplitPlan& split = SplitPlan{}) {
  int bq, bk, nq, nk;
  tile_shape(d, &bq, &bk, &nq, &nk);
  const size_t elem = d->dtype == HA_DTYPE_F32 ? 4 : 2;
  Workspace w{};
  size_t at = 0;
  w.row_limit = at;
  at = round256(at + (size_t)d->batch * d->seq_len * 4);
  w.ranges = at;
  at = round256(at + (size_t)d->batch * nq * 2 * 4);
  if (prologue) {
    w.q_rot = at;
    at = round256(at + (size_t)d->batch * d->seq_len * d->n_q_heads * d->head_dim * elem);
    w.k_rot = at;
    at = round256(at + (size_t)d->batch * d->seq_len * d->n_kv_heads * d->head_dim * elem);
  }
  if (has_gen(d)) take_hole(d, nq, nk, &at, &w.key_vis, &w.tiles, &w.tile_count);
  if (split.active) {
    const size_t G = d->n_q_heads / d->n_kv_heads;
    auto take = [&](size_t& field, size_t bytes) {
      field = at;
      at = round256(at + bytes);
    };
    take(w.items, (size_t)(split.n_items + split.n_splits) * 16);
    take(w.part_o, (size_t)split.n_slots * bq * G * d->head_dim * 4);
    take(w.part_l, (size_t)split.n_slots * bq * G * 4);
    take(w.part_m, (size_t)split.n_slots * bq * G * 4);
  }
  w.total = at;
  return w;
}

// ---------------------------------------------------------------- training
ha_status check_train(const ha_attn_desc* d) {
  if (d->dtype != HA_DTYPE_BF16) return fail(HA_ERR_UNSUPPORTED, "training entry points take bf16 tensors");
  const int group = d->n_q_heads / d->n_kv_heads;
  if (group > 4) return fail(HA_ERR_UNSUPPORTED, "training: n_q_heads / n_kv_heads = %d; supported: 1, 2, 4", group);
  return HA_OK;
}

bool has_norm(const ha_prologue_desc* p) { return p && p->q_norm_weight; }

struct BwdWorkspace {
  size_t row_limit, ranges, q_rot, k_rot, delta, dq_rot, dk_rot, dwq, dwk, dw_scratch, key_vis, tiles, tile_count,
      part_dk, part_dv, total;
  ha::KvPlan kv;  // the dK/dV launch plan (G = 4)
};

BwdWorkspace bwd_workspace_layout(const ha_attn_desc* d, bool norm) {
  int bq, bk, nq, nk;
  tile_shape(d, &bq, &bk, &nq, &nk);
  const size_t B = d->batch, S = d->seq_len, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
  BwdWorkspace w{};
  size_t at = 0;
  auto take = [&](size_t& field, size_t bytes) {
    field = at;
    at = round256(at + bytes);
  };
  take(w.row_limit, B * S * 4);
  take(w.ranges, B * nq * 2 * 4);
  take(w.q_rot, B * S * Hq * D * 2);
  take(w.k_rot, B * S * Hkv * D * 2);
  take(w.delta, B * Hq * S * 4);
  take(w.dq_rot, B * S * Hq * D * 4);
  take(w.dk_rot, B * S * Hkv * D * 4);
  if (norm) {
    take(w.dwq, B * S * D * 4);
    take(w.dwk, B * S * D * 4);
    take(w.dw_scratch, (size_t)ha::dw_scratch_floats((int)D) * 4);
  }
  if (has_gen(d)) take_hole(d, nq, nk, &at, &w.key_vis, &w.tiles, &w.tile_count);
  w.kv = ha::kv_plan(d->batch, d->seq_len, d->n_kv_heads, d->n_q_heads / d->n_kv_heads, plan_cus(d));
  if (w.kv.tail_parts > 1) {  // the tail's partial dK and dV, fp32
    const size_t part = (size_t)w.kv.tail_parts * B * (S - w.kv.k_main) * Hkv * D * 4;
    take(w.part_dk, part);
    take(w.part_dv, part);
  }
  w.total = at;
  return w;
}

ha_status check_workspace(const void* workspace, size_t have, size_t need) {
  if (!workspace) return fail(HA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(HA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (have < need) return fail(HA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  return HA_OK;
}

}  // namespace

extern "C" {

int ha_abi_version(void) { return HA_ABI_VERSION; }

const char* ha_last_error(void) { return g_last_error.c_str(); }

ha_status ha_rope_table_fill(double theta, int32_t head_dim, int32_t n_pos, float* host_out) {
  if (!host_out) return fail(HA_ERR_INVALID_ARG, "host_out is NULL");
  if (head_dim != 64 && head_dim != 128) return fail(HA_ERR_UNSUPPORTED, "head_dim %d; supported: 64, 128", head_dim);
  if (n_pos < 1) return fail(HA_ERR_INVALID_ARG, "n_pos must be >= 1");
  if (!(theta > 1.0) || !std::isfinite(theta)) return fail(HA_ERR_INVALID_ARG, "theta must be finite and > 1");
  const int half = head_dim / 2;
  for (int i = 0; i < half; ++i) {
    const double f = std::pow(theta, -2.0 * i / head_dim);
    for (int64_t p = 0; p < n_pos; ++p) {
      const double ang = (double)p * f;
      host_out[(p * half + i) * 2 + 0] = (float)std::cos(ang);
      host_out[(p * half + i) * 2 + 1] = (float)std::sin(ang);
    }
  }
  return ok();
}

float ha_q_prescale(const ha_attn_desc* desc) {
  if (check_desc(desc) != HA_OK) return 0.f;
  g_last_error.clear();
  return q_prescale(desc);
}

ha_status ha_tile_shape(const ha_attn_desc* desc, int32_t* block_q, int32_t* block_k, int32_t* n_q_blocks,
                        int32_t* n_k_blocks) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if (!block_q || !block_k || !n_q_blocks || !n_k_blocks) return fail(HA_ERR_INVALID_ARG, "output pointer is NULL");
  int bq, bk, nq, nk;
  tile_shape(desc, &bq, &bk, &nq, &nk);
  *block_q = bq;
  *block_k = bk;
  *n_q_blocks = nq;
  *n_k_blocks = nk;
  return ok();
}

ha_status ha_classify_tiles(const ha_attn_desc* desc, uint8_t* labels, int32_t* ranges, int32_t* row_limit,
                            void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if (!labels && !ranges && !row_limit) return fail(HA_ERR_INVALID_ARG, "no output requested");
  if ((ranges && !aligned(ranges, 4)) || (row_limit && !aligned(row_limit, 4)))
    return fail(HA_ERR_ALIGNMENT, "ranges and row_limit must be 4-byte aligned");
  if (empty(desc)) return ok();
  st = run_classify(desc, labels, ranges, row_limit, static_cast<hipStream_t>(stream));
  return st == HA_OK ? ok() : st;
}

ha_status ha_qk_prologue(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q_in, const void* k_in,
                         void* q_out, void* k_out, void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if ((st = check_prologue(desc, pro)) != HA_OK) return st;
  if (empty(desc)) return ok();
  if ((st = check_tensor(q_in, "q_in")) != HA_OK || (st = check_tensor(k_in, "k_in")) != HA_OK ||
      (st = check_tensor(q_out, "q_out")) != HA_OK || (st = check_tensor(k_out, "k_out")) != HA_OK)
    return st;
  if ((st = check_positions_debug(desc, pro, static_cast<hipStream_t>(stream))) != HA_OK) return st;
  st = run_prologue(desc, pro, q_in, k_in, q_out, k_out, pro->q_out_scale > 0.f ? pro->q_out_scale : 1.f,
                    static_cast<hipStream_t>(stream));
  return st == HA_OK ? ok() : st;
}

size_t ha_attn_workspace_bytes(const ha_attn_desc* desc, const ha_prologue_desc* pro) {
  if (check_desc(desc) != HA_OK) return 0;
  return workspace_layout(desc, pro != nullptr, plan_split(desc)).total;
}

ha_status ha_attn_fwd_planned(const ha_attn_desc* desc, const void* q, const void* k, const void* v,
                              const int32_t* row_limit, const int32_t* ranges, void* out, void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if (empty(desc)) return ok();
  if ((st = check_tensor(q, "q")) != HA_OK || (st = check_tensor(k, "k")) != HA_OK ||
      (st = check_tensor(v, "v")) != HA_OK || (st = check_tensor(out, "out")) != HA_OK)
    return st;
  if (!row_limit || !ranges) return fail(HA_ERR_INVALID_ARG, "row_limit and ranges are required");
  if (!aligned(row_limit, 4) || !aligned(ranges, 4))
    return fail(HA_ERR_ALIGNMENT, "row_limit and ranges must be 4-byte aligned");
  if (has_gen(desc))
    return fail(HA_ERR_UNSUPPORTED, "Gen Image segments need the full tile plan: use ha_attn_fwd");
  st = run_attn(desc, q, k, v, row_limit, ranges, out, desc->q_prescaled == 1, static_cast<hipStream_t>(stream));
  return st == HA_OK ? ok() : st;
}

}  // extern "C"

namespace {

// The forward after validation, with the workspace already checked against the layout w
// of plan (both as attn_fwd chose them).
ha_status attn_fwd_run(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q, const void* k,
                       const void* v, void* out, float* lse, void* workspace, const SplitPlan& plan,
                       const Workspace& w, void* stream);

ha_status attn_fwd(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q, const void* k,
                   const void* v, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if (pro && (st = check_prologue(desc, pro)) != HA_OK) return st;
  if (empty(desc)) return ok();
  if ((st = check_tensor(q, "q")) != HA_OK || (st = check_tensor(k, "k")) != HA_OK ||
      (st = check_tensor(v, "v")) != HA_OK || (st = check_tensor(out, "out")) != HA_OK)
    return st;
  // the split plan when the workspace holds it (the bytes that ha_attn_workspace_bytes
  // gives), else one work item per query block
  SplitPlan plan = plan_split(desc);
  Workspace w = workspace_layout(desc, pro != nullptr, plan);
  if (plan.active && workspace_bytes < w.total) {
    plan = SplitPlan{};
    w = workspace_layout(desc, pro != nullptr);
  }
  if ((st = check_workspace(workspace, workspace_bytes, w.total)) != HA_OK) return st;
  return attn_fwd_run(desc, pro, q, k, v, out, lse, workspace, plan, w, stream);
}

ha_status attn_fwd_run(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q, const void* k,
                       const void* v, void* out, float* lse, void* workspace, const SplitPlan& plan,
                       const Workspace& w, void* stream) {
  ha_status st = HA_OK;
  char* ws = static_cast<char*>(workspace);
  int32_t* row_limit = reinterpret_cast<int32_t*>(ws + w.row_limit);
  int32_t* ranges = reinterpret_cast<int32_t*>(ws + w.ranges);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const HolePlan hole = hole_plan(desc, ws, w.key_vis, w.tiles, w.tile_count);
  SplitRun split;
  if (plan.active) {
    split.items = reinterpret_cast<int32_t*>(ws + w.items);
    split.n_items = plan.n_items;
    split.part_o = reinterpret_cast<float*>(ws + w.part_o);
    split.part_l = reinterpret_cast<float*>(ws + w.part_l);
    split.part_m = reinterpret_cast<float*>(ws + w.part_m);
  }
  if ((st = check_positions_debug(desc, pro, s)) != HA_OK) return st;
  if ((st = run_classify(desc, nullptr, ranges, row_limit, s, hole)) != HA_OK) return st;
  if (plan.active) {
    // the work item table, from the tile counts the classifier just wrote
    ha::PlanArgs pa{};
    int bq, bk, nq, nk;
    tile_shape(desc, &bq, &bk, &nq, &nk);
    pa.cost = hole.tile_count ? hole.tile_count : ranges;
    pa.items = split.items;
    pa.splits = split.items + (size_t)plan.n_items * 4;
    pa.nq = nq;
    pa.Hkv = desc->n_kv_heads;
    pa.groups = plan.groups;
    pa.affine = plan.affine;
    pa.longest = plan.longest;
    for (int x = 0; x < plan.groups; ++x) {
      pa.n[x] = plan.n[x];
      pa.best[x] = plan.best[x];
      pa.k[x] = plan.k[x];
      pa.heavy[x] = plan.heavy[x];
      pa.slot_base[x] = plan.slot_base[x];
      pa.split_base[x] = plan.split_base[x];
      pa.len[x] = plan.len[x];
    }
    if ((st = check_launch(ha::launch_plan(pa, s), s, "split plan table")) != HA_OK) return st;
  }
  const void* qa = q;
  const void* ka = k;
  if (pro) {
    void* qr = ws + w.q_rot;
    void* kr = ws + w.k_rot;
    if ((st = run_prologue(desc, pro, q, k, qr, kr, q_prescale(desc), s)) != HA_OK) return st;
    qa = qr;
    ka = kr;
  }
  st = run_attn(desc, qa, ka, v, row_limit, ranges, out, pro != nullptr, s, lse, 0, hole, split);
  if (st == HA_OK && plan.active) {
    ha::CombineArgs c{};
    int bq, bk, nq, nk;
    tile_shape(desc, &bq, &bk, &nq, &nk);
    c.splits = split.items + (size_t)plan.n_items * 4;
    c.part_o = split.part_o;
    c.part_l = split.part_l;
    c.part_m = split.part_m;
    c.out = out;
    c.lse = lse;
    c.n_splits = plan.n_splits;
    c.S = desc->seq_len;
    c.Hq = desc->n_q_heads;
    c.Hkv = desc->n_kv_heads;
    c.nq = nq;
    c.BQ = bq;
    c.G = desc->n_q_heads / desc->n_kv_heads;
    c.D = desc->head_dim;
    st = check_launch(ha::launch_combine(c, s), s, "merge of split query blocks");
  }
  return st == HA_OK ? ok() : st;
}

}  // namespace

extern "C" {

ha_status ha_qk_prologue_from(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q_in,
                              const void* k_in, void* q_out, void* k_out, int32_t token_begin, void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if ((st = check_prologue(desc, pro)) != HA_OK) return st;
  if (token_begin < 0 || token_begin > desc->seq_len)
    return fail(HA_ERR_INVALID_ARG, "token_begin %d outside [0, seq_len %d]", token_begin, desc->seq_len);
  if (empty(desc) || token_begin == desc->seq_len) return ok();
  if ((st = check_tensor(q_in, "q_in")) != HA_OK || (st = check_tensor(k_in, "k_in")) != HA_OK ||
      (st = check_tensor(q_out, "q_out")) != HA_OK || (st = check_tensor(k_out, "k_out")) != HA_OK)
    return st;
  if ((st = check_positions_debug(desc, pro, static_cast<hipStream_t>(stream))) != HA_OK) return st;
  st = run_prologue(desc, pro, q_in, k_in, q_out, k_out, pro->q_out_scale > 0.f ? pro->q_out_scale : 1.f,
                    static_cast<hipStream_t>(stream), token_begin);
  return st == HA_OK ? ok() : st;
}

ha_status ha_attn_fwd_planned_from(const ha_attn_desc* desc, const void* q, const void* k, const void* v,
                                   const int32_t* row_limit, const int32_t* ranges, void* out, int32_t row_begin,
                                   void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if (row_begin < 0 || row_begin > desc->seq_len)
    return fail(HA_ERR_INVALID_ARG, "row_begin %d outside [0, seq_len %d]", row_begin, desc->seq_len);
  if (empty(desc) || row_begin == desc->seq_len) return ok();
  if ((st = check_tensor(q, "q")) != HA_OK || (st = check_tensor(k, "k")) != HA_OK ||
      (st = check_tensor(v, "v")) != HA_OK || (st = check_tensor(out, "out")) != HA_OK)
    return st;
  if (!row_limit || !ranges) return fail(HA_ERR_INVALID_ARG, "row_limit and ranges are required");
  if (!aligned(row_limit, 4) || !aligned(ranges, 4))
    return fail(HA_ERR_ALIGNMENT, "row_limit and ranges must be 4-byte aligned");
  if (has_gen(desc))
    return fail(HA_ERR_UNSUPPORTED, "Gen Image segments need the full tile plan: use ha_attn_fwd");
  // the rows kept from an earlier step must not see keys at or after row_begin: a causal
  // row sees keys up to itself, a full row every key, an image row keys up to its
  // segment's end
  for (int b = 0; b < desc->batch; ++b)
    for (int t = 0; t < desc->n_segments; ++t) {
      const ha_segment& g = desc->segments[(int64_t)b * desc->n_segments + t];
      const int end = g.start + g.length;
      if ((g.kind == HA_SEG_FULL && g.start < row_begin && row_begin < desc->seq_len) ||
          ((g.kind == HA_SEG_GCA || g.kind == HA_SEG_GEN) && g.start < row_begin && row_begin < end))
        return fail(HA_ERR_INVALID_ARG,
                    "row_begin %d: rows of batch %d segment %d (kind %d, [%d, %d)) below it attend to keys at or "
                    "after it",
                    row_begin, b, t, g.kind, g.start, end);
    }
  st = run_attn(desc, q, k, v, row_limit, ranges, out, desc->q_prescaled == 1, static_cast<hipStream_t>(stream),
                nullptr, row_begin);
  return st == HA_OK ? ok() : st;
}

ha_status ha_attn_fwd(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q, const void* k,
                      const void* v, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd(desc, pro, q, k, v, out, nullptr, workspace, workspace_bytes, stream);
}

ha_status ha_attn_fwd_lse(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q, const void* k,
                          const void* v, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if ((st = check_train(desc)) != HA_OK) return st;
  if (!empty(desc) && (!lse || !aligned(lse, 4))) return fail(HA_ERR_INVALID_ARG, "lse must be a 4-byte aligned pointer");
  return attn_fwd(desc, pro, q, k, v, out, lse, workspace, workspace_bytes, stream);
}

ha_status ha_attn_fwd_static(const ha_attn_desc* desc, const void* q, const void* k, const void* v, void* out,
                             void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if (empty(desc)) return ok();
  if ((st = check_tensor(q, "q")) != HA_OK || (st = check_tensor(k, "k")) != HA_OK ||
      (st = check_tensor(v, "v")) != HA_OK || (st = check_tensor(out, "out")) != HA_OK)
    return st;
  // as ha_attn_fwd without a prologue: the split plan when the scratch array holds it, else
  // one work item per query block, else the problem is too large for the array
  SplitPlan plan = plan_split(desc);
  Workspace w = workspace_layout(desc, false, plan);
  if (plan.active && w.total > ha::kStaticScratchBytes) {
    plan = SplitPlan{};
    w = workspace_layout(desc, false);
  }
  if (w.total > ha::kStaticScratchBytes)
    return fail(HA_ERR_WORKSPACE,
                "ha_attn_fwd_static: this problem needs %zu bytes of scratch, the static array holds %zu "
                "(use ha_attn_fwd with a workspace)",
                w.total, ha::kStaticScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = ha::static_scratch(&scratch);
  if (e != hipSuccess) return fail(HA_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
  st = attn_fwd_run(desc, nullptr, q, k, v, out, nullptr, scratch, plan, w, stream);
  return st == HA_OK ? ok() : st;
}

ha_status ha_qkv_prologue(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* x, int32_t hidden,
                          const void* w_qkv, void* q_out, void* k_out, void* v_out, void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if (pro && (st = check_prologue(desc, pro)) != HA_OK) return st;
  if (desc->dtype != HA_DTYPE_BF16) return fail(HA_ERR_UNSUPPORTED, "ha_qkv_prologue takes bf16 tensors");
  if (desc->head_dim != 128) return fail(HA_ERR_UNSUPPORTED, "ha_qkv_prologue: head_dim %d; supported: 128", desc->head_dim);
  if (hidden < 64 || hidden % 64 != 0)
    return fail(HA_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 64", hidden);
  if (empty(desc)) return ok();
  const void* tensors[] = {x, w_qkv, q_out, k_out, v_out};
  const char* names[] = {"x", "w_qkv", "q_out", "k_out", "v_out"};
  for (int t = 0; t < 5; ++t)
    if ((st = check_tensor(tensors[t], names[t])) != HA_OK) return st;
  ha::QkvArgs a{};
  a.x = x;
  a.w = w_qkv;
  a.q_out = q_out;
  a.k_out = k_out;
  a.v_out = v_out;
  a.T = desc->batch * desc->seq_len;
  a.K = hidden;
  a.Hq = desc->n_q_heads;
  a.Hkv = desc->n_kv_heads;
  a.q_scale = pro && pro->q_out_scale > 0.f ? pro->q_out_scale : 1.f;
  a.rotate = pro && pro->rope_kind != HA_ROPE_NONE;
  if (a.rotate) {
    a.positions = pro->positions;
    a.cos_sin = pro->cos_sin;
    a.n_pos = pro->n_pos;
    a.n_axes = n_axes_of(pro->rope_kind);
    axis_table(pro, desc->head_dim, a.axis);
  }
  if (has_norm(pro)) {
    a.wq = pro->q_norm_weight;
    a.wk = pro->k_norm_weight;
    a.eps = pro->eps;
  }
  if ((st = check_positions_debug(desc, pro, static_cast<hipStream_t>(stream))) != HA_OK) return st;
  int dev = 0, n_cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    n_cus = 0;  // unknown: every token goes to the half-height tiles
    (void)hipGetLastError();  // not reported by the launch check below
  }
  st = check_launch(ha::launch_qkv(a, n_cus, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream),
                    "qkv projection");
  return st == HA_OK ? ok() : st;
}

size_t ha_attn_bwd_workspace_bytes(const ha_attn_desc* desc, const ha_prologue_desc* pro) {
  if (check_desc(desc) != HA_OK) return 0;
  return bwd_workspace_layout(desc, has_norm(pro)).total;
}

ha_status ha_attn_bwd(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q, const void* k,
                      const void* v, const void* out, const float* lse, const void* dout, void* dq, void* dk,
                      void* dv, float* dw_q, float* dw_k, void* workspace, size_t workspace_bytes, void* stream) {
  ha_status st = check_desc(desc);
  if (st != HA_OK) return st;
  if ((st = check_train(desc)) != HA_OK) return st;
  if (pro && (st = check_prologue(desc, pro)) != HA_OK) return st;
  if (desc->q_prescaled != 0) return fail(HA_ERR_INVALID_ARG, "ha_attn_bwd: desc->q_prescaled must be 0");
  const bool norm = has_norm(pro);
  if (norm != (dw_q != nullptr) || norm != (dw_k != nullptr))
    return fail(HA_ERR_INVALID_ARG, "dw_q and dw_k are required exactly when the prologue has RMSNorm");
  if (norm && (!aligned(dw_q, 4) || !aligned(dw_k, 4))) return fail(HA_ERR_ALIGNMENT, "dw_q, dw_k must be 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = desc->head_dim;
  if (empty(desc)) {
    // no tokens: the weight gradients are empty sums
    if (norm) {
      if ((st = check_launch(ha::launch_dw_reduce(nullptr, nullptr, 0, D, nullptr, dw_q, dw_k, s), s, "dw")) != HA_OK)
        return st;
    }
    return ok();
  }
  const void* tensors[] = {q, k, v, out, dout, dq, dk, dv};
  const char* names[] = {"q", "k", "v", "out", "dout", "dq", "dk", "dv"};
  for (int t = 0; t < 8; ++t)
    if ((st = check_tensor(tensors[t], names[t])) != HA_OK) return st;
  if (!lse || !aligned(lse, 4)) return fail(HA_ERR_INVALID_ARG, "lse must be a 4-byte aligned pointer");
  const BwdWorkspace w = bwd_workspace_layout(desc, norm);
  if ((st = check_workspace(workspace, workspace_bytes, w.total)) != HA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  int32_t* row_limit = reinterpret_cast<int32_t*>(ws + w.row_limit);
  int32_t* ranges = reinterpret_cast<int32_t*>(ws + w.ranges);
  void* q_rot = ws + w.q_rot;
  void* k_rot = ws + w.k_rot;
  float* delta = reinterpret_cast<float*>(ws + w.delta);
  float* dq_rot = reinterpret_cast<float*>(ws + w.dq_rot);
  float* dk_rot = reinterpret_cast<float*>(ws + w.dk_rot);

  const HolePlan hole = hole_plan(desc, ws, w.key_vis, w.tiles, w.tile_count);
  if ((st = check_positions_debug(desc, pro, s)) != HA_OK) return st;
  if ((st = run_classify(desc, nullptr, ranges, row_limit, s, hole)) != HA_OK) return st;
  // q' = scale log2(e) (normalised, rotated q) and the rotated k, as the forward used them
  ha_prologue_desc plain{};
  plain.rope_kind = HA_ROPE_NONE;
  if ((st = run_prologue(desc, pro ? pro : &plain, q, k, q_rot, k_rot, q_prescale(desc), s)) != HA_OK) return st;
  const int B = desc->batch, S = desc->seq_len, Hq = desc->n_q_heads, Hkv = desc->n_kv_heads;
  if ((st = check_launch(ha::launch_bwd_delta(out, dout, delta, B, S, Hq, D, s), s, "backward delta")) != HA_OK)
    return st;
  ha::BwdArgs a{};
  int bq, bk, nq, nk;
  tile_shape(desc, &bq, &bk, &nq, &nk);
  a.q = q_rot;
  a.k = k_rot;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.row_limit = row_limit;
  a.ranges = ranges;
  a.dq = dq_rot;
  a.dk = dk_rot;
  a.dv = dv;
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.nq = nq;
  a.scale = (float)softmax_scale(desc);
  a.key_vis = hole.key_vis;
  a.tiles = hole.tiles;
  a.tile_count = hole.tile_count;
  a.kv_stride = ha::key_vis_stride(S);
  a.nk = nk;
  a.k_main = w.kv.k_main;
  a.tail_parts = w.kv.tail_parts;
  a.part_dk = w.kv.tail_parts > 1 ? reinterpret_cast<float*>(ws + w.part_dk) : nullptr;
  a.part_dv = w.kv.tail_parts > 1 ? reinterpret_cast<float*>(ws + w.part_dv) : nullptr;
  if ((st = check_launch(ha::launch_bwd_dkdv(a, s), s, "backward dK dV")) != HA_OK) return st;
  if ((st = check_launch(ha::launch_bwd_dq(a, s), s, "backward dQ")) != HA_OK) return st;
  // through the rotary embedding and RMSNorm to the inputs
  ha::PrologueBwdArgs p{};
  p.dq_rot = dq_rot;
  p.dk_rot = dk_rot;
  p.q_in = q;
  p.k_in = k;
  p.dq = dq;
  p.dk = dk;
  p.rotate = pro && pro->rope_kind != HA_ROPE_NONE;
  if (p.rotate) {
    p.positions = pro->positions;
    p.cos_sin = pro->cos_sin;
    p.n_axes = n_axes_of(pro->rope_kind);
    p.n_pos = pro->n_pos;
    axis_table(pro, D, p.axis);
  }
  if (norm) {
    p.wq = pro->q_norm_weight;
    p.wk = pro->k_norm_weight;
    p.eps = pro->eps;
    p.dwq_part = reinterpret_cast<float*>(ws + w.dwq);
    p.dwk_part = reinterpret_cast<float*>(ws + w.dwk);
  }
  p.B = B;
  p.S = S;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  if ((st = check_launch(ha::launch_prologue_bwd(p, s), s, "backward prologue")) != HA_OK) return st;
  if (norm) {
    float* scratch = reinterpret_cast<float*>(ws + w.dw_scratch);
    if ((st = check_launch(ha::launch_dw_reduce(p.dwq_part, p.dwk_part, (int64_t)B * S, D, scratch, dw_q, dw_k, s), s,
                           "dw")) != HA_OK)
      return st;
  }
  return ok();
}

}  // extern "C"
