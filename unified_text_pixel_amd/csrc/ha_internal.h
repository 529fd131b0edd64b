// Internal interface between the host dispatch (ha_host.cpp) and the gfx950 kernels.
// Nothing here is part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ha_attn.h"

namespace ha {

// Segment tables of several batch items, passed by value as kernel arguments.
constexpr int kArgSegs = 128;
struct SegArgs {
  int32_t n_items;  // batch items covered by this launch
  int32_t b0;       // first batch item
  int32_t n_seg;    // segments per item
  int32_t start[kArgSegs];
  int32_t end[kArgSegs];
  int32_t kind[kArgSegs];
};

// Gen Images (multi-image training): key j is seen only by rows i < key_vis[j] (the end
// of its Gen Image; S for every other key; 0 for the padding after S). Rows of key_vis
// are key_vis_stride(S) long, a multiple of every key block the kernels read.
constexpr int kKeyVisAlign = 256;
inline int key_vis_stride(int S) { return (S + kKeyVisAlign - 1) / kKeyVisAlign * kKeyVisAlign; }

struct ClassifyArgs {
  int32_t S, nq, nk, bq, bk;
  uint8_t* labels;     // [B][nq][nk] or null
  int32_t* ranges;     // [B][nq][2] or null: key tiles by the row limits alone
  int32_t* row_limit;  // [B][S] or null: the key prefix of each row before any hole
  int32_t has_gen;     // some segment is a Gen Image (labels then account for the holes)
  int32_t* key_vis;    // [B][key_vis_stride(S)] or null
  int32_t* tiles;      // [B][nq][nk] or null: each query block's key tiles to execute,
                       // FULL tiles inside the sequence first, then the rest
  int32_t* tile_count; // [B][nq][2]: (inside FULL tiles, all listed tiles)
  int32_t kv_stride;
  SegArgs seg;
};
hipError_t launch_classify(const ClassifyArgs& a, hipStream_t stream);

// Work item table of a split plan, built on the device from the classifier's per-block tile
// counts. The host decides per XCD group x (8 groups when the (batch, KV head) pairs split
// evenly over the XCDs, else 1) which items of the group's list, sorted longest first, are
// split and into how many parts; the kernel sorts (stably, by tile count) and writes the
// table: entry e of the table is (b * Hkv + g, query block, part | parts << 16, slot or -1),
// item f of group x's final list at entry f * groups + x, -1 rows as padding; then the
// split table [n_splits][4] of (b * Hkv + g, query block, first slot, parts).
constexpr int kPlanGroups = 8;
constexpr int kPlanMaxItems = 1024;  // items per group before splitting
struct PlanArgs {
  const int32_t* cost;  // [B][nq][2]: field 1 is the number of key tiles the block executes
  int32_t* items;       // [longest * groups][4]
  int32_t* splits;      // [n_splits][4]
  int32_t nq, Hkv, groups, affine, longest;
  // per group: items n (pairs of the group x nq), split parts best (1: none), sorted
  // positions [k, heavy) split, first slot and first split-table row, final list length
  int32_t n[kPlanGroups], best[kPlanGroups], k[kPlanGroups], heavy[kPlanGroups];
  int32_t slot_base[kPlanGroups], split_base[kPlanGroups], len[kPlanGroups];
};
hipError_t launch_plan(const PlanArgs& a, hipStream_t stream);

struct PrologueArgs {
  const void* q_in;
  const void* k_in;
  void* q_out;
  void* k_out;
  const int32_t* positions;  // [B][S][n_axes] or null (no rotation)
  const float* cos_sin;      // [n_pos][D/2][2]
  const float* wq;           // [D] or null (no RMSNorm)
  const float* wk;
  int32_t B, S, Hq, Hkv, D, n_axes, n_pos;
  int32_t rotate;  // 0: no rotary embedding
  float eps;
  float q_scale;   // q outputs are multiplied by this before rounding
  int32_t f32;     // 1: fp32 tensors, 0: bf16
  int32_t token_begin;  // tokens [token_begin, S) of every batch item are processed
  uint8_t axis[64];  // rotary axis of pair i
};
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream);

// Debug check of rotary positions (HA_DEBUG): the first index of positions[0, count) outside
// [0, n_pos), or -1, and the value found there. Synchronises the stream.
hipError_t check_positions(const int32_t* positions, int64_t count, int32_t n_pos, hipStream_t stream,
                           int64_t* first_bad, int32_t* value);

// Attention tile shape: block_q query tokens per work item, kBlockK keys per tile.
constexpr int kBlockK = 64;
int attn_block_q(int head_dim, int group, bool f32);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* row_limit;  // [B][S]
  const int32_t* ranges;     // [B][nq][2]
  int32_t B, S, Hq, Hkv, D, nq;
  float scale_log2e;         // softmax scale * log2(e)
  int32_t q_prescaled;       // 1: q already carries scale_log2e
  int32_t f32;
  float* lse;                // [B][Hq][S] row log-sum-exp (natural log), or null
  int32_t nq_run;            // compute the last nq_run query blocks of each (batch, KV head)
  int32_t row_begin;         // rows below it are computed with their block but not written
  // Gen Image layouts (else null): the classifier's key visibility and tile lists
  const int32_t* key_vis;
  const int32_t* tiles;
  const int32_t* tile_count;
  int32_t kv_stride, nk;
  // split query blocks (bf16, else null): the work item table [n_items][4] of (b * Hkv + g,
  // query block, part | parts << 16, partial slot or -1) and the partial outputs per slot:
  // part_o [slot][BQ][G][D], part_l and part_m [slot][BQ][G]
  const int32_t* items;
  int32_t n_items;
  float* part_o;
  float* part_l;
  float* part_m;
  // workgroups per query block: 1, or (bf16, group 4, plain tile ranges) one per 32-row
  // slice, which spreads a problem with fewer work items than CUs over more of them
  int32_t slices;
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);
// Workgroups per query block when the work items are too few to fill the CUs (1: no slices).
int attn_slices(int head_dim, int group, bool f32);

// Merge of split query blocks: splits [n_splits][4] of (b * Hkv + g, query block, first
// slot, parts); writes out (bf16) and, when lse is set, the row lse.
struct CombineArgs {
  const int32_t* splits;
  const float* part_o;
  const float* part_l;
  const float* part_m;
  void* out;
  float* lse;
  int32_t n_splits, S, Hq, Hkv, nq, BQ, G, D;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// ---- allocation-free forward (ha_scratch.hip)
// Bytes of the device-side scratch array; its address on the current device (looked up
// once per device and kept).
constexpr size_t kStaticScratchBytes = HA_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(void** addr);

// ---- QKV projection with the prologue in its epilogue (ha_qkv.hip)
struct QkvArgs {
  const void* x;             // bf16 [T][K]
  const void* w;             // bf16 [(Hq + 2 Hkv) 128][K], rows q heads, k heads, v heads
  void* q_out;               // bf16 [T][Hq][128]
  void* k_out;               // bf16 [T][Hkv][128]
  void* v_out;               // bf16 [T][Hkv][128]
  const int32_t* positions;  // [T][n_axes] (rotate)
  const float* cos_sin;      // [n_pos][64][2]
  const float* wq;           // [128] or null (no RMSNorm)
  const float* wk;
  int32_t T, K, Hq, Hkv, n_axes, n_pos, rotate;
  int32_t m_begin;           // first token of this launch (tokens [m_begin, T))
  float eps, q_scale;
  uint8_t axis[64];
};
int qkv_block_tokens();
hipError_t launch_qkv(const QkvArgs& a, int n_cus, hipStream_t stream);

// ---- backward (ha_attn_bwd.hip, ha_prologue.hip)

// Key block of the dK/dV kernel: 32 keys per wave, 8 / G waves per query head.
int bwd_block_k(int group);

struct BwdArgs {
  const void* q;             // q' = scale * log2(e) * (rotated q), bf16 [B][S][Hq][D]
  const void* k;             // rotated k, bf16 [B][S][Hkv][D]
  const void* v;             // bf16 [B][S][Hkv][D]
  const void* dout;          // bf16 [B][S][Hq][D]
  const float* lse;          // [B][Hq][S], natural log
  const float* delta;        // [B][Hq][S]: dout . out per row
  const int32_t* row_limit;  // [B][S]
  const int32_t* ranges;     // [B][nq][2], query blocks of attn_block_q rows
  float* dq;                 // gradient of the rotated q, fp32 [B][S][Hq][D]
  float* dk;                 // gradient of the rotated k, fp32 [B][S][Hkv][D]
  void* dv;                  // bf16 [B][S][Hkv][D]
  int32_t B, S, Hq, Hkv, D, nq;
  float scale;               // softmax scale
  // Gen Image layouts (else null), as in AttnArgs
  const int32_t* key_vis;
  const int32_t* tiles;
  const int32_t* tile_count;
  int32_t kv_stride, nk;
  // dK/dV launch plan (the host's kv_plan): keys [0, k_main) two heads per step over
  // 128-key blocks (G = 4 only); keys [k_main, S) G heads per step over 256/G-key blocks,
  // their 32-row steps cut into tail_parts ranges whose fp32 partial dK and dV go to
  // part_dk / part_dv [tail_parts][B][S - k_main][Hkv][D] and are summed in part order
  int32_t k_main, tail_parts;
  float* part_dk;
  float* part_dv;
  // one launch's key range [k_begin, k_end) and step ranges (set by launch_bwd_dkdv)
  int32_t k_begin, k_end, n_parts;
};
// dK/dV launch plan: see BwdArgs
struct KvPlan {
  int k_main = 0, tail_parts = 1;
};
KvPlan kv_plan(int B, int S, int Hkv, int G, int n_cus);
hipError_t launch_bwd_delta(const void* out, const void* dout, float* delta, int B, int S, int Hq, int D,
                            hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);

// Rotary and RMSNorm backward: d(rotated) fp32 -> d(input) in the tensors' dtype, plus per
// token sums over heads of dy * x * r for the norm weights' gradient.
struct PrologueBwdArgs {
  const float* dq_rot;  // [B][S][Hq][D]
  const float* dk_rot;  // [B][S][Hkv][D]
  const void* q_in;     // the forward prologue's inputs (needed with RMSNorm)
  const void* k_in;
  void* dq;             // [B][S][Hq][D]
  void* dk;             // [B][S][Hkv][D]
  float* dwq_part;      // [B*S][D] or null (no RMSNorm)
  float* dwk_part;
  const int32_t* positions;
  const float* cos_sin;
  const float* wq;
  const float* wk;
  int32_t B, S, Hq, Hkv, D, n_axes, n_pos;
  int32_t rotate;
  float eps;
  int32_t f32;
  uint8_t axis[64];
};
hipError_t launch_prologue_bwd(const PrologueBwdArgs& a, hipStream_t stream);
// dw_q[d] = sum over rows of part_q[row][d] (fp32), for rows in [0, n), in a fixed order,
// and dw_k from part_k alike; scratch holds dw_scratch_floats(D) floats of per-workgroup
// sums (unused when n == 0)
int dw_scratch_floats(int D);
hipError_t launch_dw_reduce(const float* part_q, const float* part_k, int64_t n, int D, float* scratch, float* dw_q,
                            float* dw_k, hipStream_t stream);

}  // namespace ha
