// Segment-table tile classifier.
//
// Every query row of the unified sequence attends to a key prefix [0, lim(i)):
//   causal rows (text, markers, condition, reference)  lim = i + 1
//   HiDream-O1 generation rows (full attention)         lim = S
//   HunyuanImage 3.0 image rows (generalized causal)    lim = end of their own segment
// because {j <= i} together with the row's own segment [s0, e0) (which contains i) is
// [0, e0). (HiDream-O1 atlas page, "How it works"; hidream-o1-p100a model card, "What
// this model is"; HunyuanImage 3.0 digest, "Generalized Causal Attention".)
// Query blocks are aligned to the end of the sequence (the first block is the ragged one),
// where the pages' layouts put the generation tokens that carry almost all of the work, so
// those rows fill whole blocks. With prefixes, the tiles of one query block are FULL on
// [0, kfull), PARTIAL on
// [kfull, kend) and SKIP beyond, where kfull comes from the block's smallest limit and
// kend from its largest; the classifier writes those two integers, the per-row limits
// and, on request, the explicit per-tile labels.
//
// Gen Images of a multi-image training sequence (HunyuanImage 3.0 digest, "Generalized
// Causal Attention", the multi-generation training paragraph and Figure 4(b)) are hidden
// from every token after them, which cuts holes into those prefixes. Pair (i, j) is then
// allowed iff j < lim(i) and i < kvis(j), kvis(j) being the end of j's Gen Image (S for
// other keys). A tile is FULL iff every row's limit covers it and every key's kvis lies
// past the block's last row; it is SKIP when no row's limit reaches it or every key's kvis
// is at or before the block's first row (exact for these segment kinds). For such layouts
// the classifier also writes kvis and, per query block, the list of tiles to execute.
#include "ha_internal.h"

namespace ha {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void classify_kernel(ClassifyArgs a) {
  const int qb = blockIdx.x;
  const int item = blockIdx.y;
  const int b = a.seg.b0 + item;
  const int S = a.S;
  const int seg0 = item * a.seg.n_seg;

  __shared__ int s_min, s_max;
  if (threadIdx.x == 0) {
    s_min = S;
    s_max = 0;
  }
  __syncthreads();

  // query blocks are cut back from the end of the sequence: the first one is ragged
  const int r1 = S - (a.nq - 1 - qb) * a.bq;
  const int r0 = max(0, r1 - a.bq);
  int lo = S, hi = 0;
  for (int i = r0 + threadIdx.x; i < r1; i += kThreads) {
    int lim = i + 1;
    for (int s = 0; s < a.seg.n_seg; ++s) {  // uniform loop over the (small) table
      const int st = a.seg.start[seg0 + s], en = a.seg.end[seg0 + s];
      if (i >= st && i < en) {
        const int kind = a.seg.kind[seg0 + s];
        lim = kind == 0 ? i + 1 : (kind == 1 ? S : en);
      }
    }
    if (a.row_limit) a.row_limit[(int64_t)b * S + i] = lim;
    lo = min(lo, lim);
    hi = max(hi, lim);
  }
  atomicMin(&s_min, lo);
  atomicMax(&s_max, hi);
  __syncthreads();

  const int kfull = s_min >= S ? a.nk : s_min / a.bk;
  const int kend = (s_max + a.bk - 1) / a.bk;
  if (threadIdx.x == 0 && a.ranges) {
    a.ranges[((int64_t)b * a.nq + qb) * 2 + 0] = kfull;
    a.ranges[((int64_t)b * a.nq + qb) * 2 + 1] = kend;
  }

  // key visibility of keys [r0, r1) (the blocks cover [0, S) once), and of the padding
  if (a.key_vis) {
    int32_t* kv = a.key_vis + (int64_t)b * a.kv_stride;
    for (int j = r0 + threadIdx.x; j < r1; j += kThreads) {
      int vis = S;
      for (int s = 0; s < a.seg.n_seg; ++s)
        if (a.seg.kind[seg0 + s] == 3 && j >= a.seg.start[seg0 + s] && j < a.seg.end[seg0 + s])
          vis = a.seg.end[seg0 + s];
      kv[j] = vis;
    }
    if (qb == a.nq - 1)
      for (int j = S + threadIdx.x; j < a.kv_stride; j += kThreads) kv[j] = 0;
  }

  // label of key tile kb: the range of kvis over its keys comes from the segment table
  auto label = [&](int kb) {
    const int c0 = kb * a.bk, c1 = min(c0 + a.bk, S);
    if (!a.has_gen) return kb < kfull ? 1 : (kb < kend ? 2 : 0);
    int vmin = S, vmax = 0;
    for (int s = 0; s < a.seg.n_seg; ++s) {
      const int st = a.seg.start[seg0 + s], en = a.seg.end[seg0 + s];
      if (st >= c1 || en <= c0) continue;
      const int vis = a.seg.kind[seg0 + s] == 3 ? en : S;
      vmin = min(vmin, vis);
      vmax = max(vmax, vis);
    }
    if (s_max <= c0 || vmax <= r0) return 0;
    if (s_min >= c1 && vmin > r1 - 1) return 1;
    return 2;
  };
  if (a.labels) {
    uint8_t* row = a.labels + ((int64_t)b * a.nq + qb) * a.nk;
    for (int kb = threadIdx.x; kb < a.nk; kb += kThreads) row[kb] = (uint8_t)label(kb);
  }

  // the tiles to execute, in order: FULL tiles inside the sequence, then the others that
  // are not SKIP (compacted by the first wave, 64 tiles per round)
  if (a.tiles && threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int32_t* list = a.tiles + ((int64_t)b * a.nq + qb) * a.nk;
    int n = 0, nfull = 0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int kb0 = 0; kb0 < a.nk; kb0 += 64) {
        const int kb = kb0 + lane;
        bool take = false;
        if (kb < a.nk) {
          const int lab = label(kb);
          const bool inside_full = lab == 1 && (kb + 1) * a.bk <= S;
          take = pass == 0 ? inside_full : (lab != 0 && !inside_full);
        }
        const unsigned long long m = __ballot(take);
        if (take) list[n + __popcll(m & ((1ull << lane) - 1ull))] = kb;
        n += __popcll(m);
      }
      if (pass == 0) nfull = n;
    }
    if (lane == 0) {
      a.tile_count[((int64_t)b * a.nq + qb) * 2 + 0] = nfull;
      a.tile_count[((int64_t)b * a.nq + qb) * 2 + 1] = n;
    }
  }
}

// ---------------------------------------------------------------- split plan table
// One workgroup per XCD group x. Item j of the group is pair j / nq of the group (pairs x,
// x + 8, ... when affine, else every pair) and query block nq - 1 - j % nq, with cost the
// number of key tiles the classifier counted for that block. The list sorted by cost,
// longest first and stable in j, has its positions [k, heavy) split into best parts of
// ceil(cost / best) tiles; that list, sorted again the same way, is the group's final
// order. A position's rank in a stable sort is the number of entries that sort before
// it, counted directly (the lists hold at most kPlanMaxItems items; the parts of one item
// stay adjacent because nothing lies between them before the sort).
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  const int x = blockIdx.x, tid = threadIdx.x;
  const int n = a.n[x], best = a.best[x], k = a.k[x], heavy = a.heavy[x];
  __shared__ int cost[kPlanMaxItems], order[kPlanMaxItems];
  // per sorted position: the cost of one entry of the final list and how many entries (parts)
  // the item makes, side by side so that one read serves the count below
  __shared__ int2 cm[kPlanMaxItems];
  auto pair_of = [&](int j) { return a.affine ? x + 8 * (j / a.nq) : j / a.nq; };
  for (int j = tid; j < n; j += kPlanThreads) {
    const int b = pair_of(j) / a.Hkv, qb = a.nq - 1 - j % a.nq;
    cost[j] = a.cost[((int64_t)b * a.nq + qb) * 2 + 1];
  }
  __syncthreads();
  for (int j = tid; j < n; j += kPlanThreads) {
    const int cj = cost[j];
    int r = 0;
    for (int u = 0; u < n; ++u) r += (cost[u] > cj || (cost[u] == cj && u < j)) ? 1 : 0;
    order[r] = j;
  }
  __syncthreads();
  for (int r = tid; r < n; r += kPlanThreads) {
    const bool split = best > 1 && r >= k && r < heavy;
    const int c = cost[order[r]];
    cm[r] = make_int2(split ? (c + best - 1) / best : c, split ? best : 1);
  }
  __syncthreads();
  for (int r = tid; r < n; r += kPlanThreads) {
    const int2 mine = cm[r];
    const int cr = mine.x, mult = mine.y;
    int f = 0;  // entries of the final list before this item's first part
    int u = 0;
    for (; u + 8 <= n; u += 8) {  // eight reads in flight, then the eight counts
      int2 e[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) e[t] = cm[u + t];
#pragma unroll
      for (int t = 0; t < 8; ++t) f += (e[t].x > cr || (e[t].x == cr && u + t < r)) ? e[t].y : 0;
    }
    for (; u < n; ++u) {
      const int2 e = cm[u];
      f += (e.x > cr || (e.x == cr && u < r)) ? e.y : 0;
    }
    const int j = order[r];
    const int bg = pair_of(j), qb = a.nq - 1 - j % a.nq;
    const bool split = mult > 1;
    const int slot0 = split ? a.slot_base[x] + (r - k) * best : -1;
    for (int p = 0; p < mult; ++p) {
      if (f + p >= a.len[x]) break;  // cannot happen: the list holds exactly len entries
      int32_t* e = a.items + ((int64_t)(f + p) * a.groups + x) * 4;
      e[0] = bg;
      e[1] = qb;
      e[2] = split ? (p | (best << 16)) : (1 << 16);
      e[3] = split ? slot0 + p : -1;
    }
    if (split) {
      int32_t* sp = a.splits + (int64_t)(a.split_base[x] + r - k) * 4;
      sp[0] = bg;
      sp[1] = qb;
      sp[2] = slot0;
      sp[3] = best;
    }
  }
  for (int f = a.len[x] + tid; f < a.longest; f += kPlanThreads) {  // padding of shorter lists
    int32_t* e = a.items + ((int64_t)f * a.groups + x) * 4;
    e[0] = -1;
    e[1] = e[2] = e[3] = 0;
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(a.groups), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_classify(const ClassifyArgs& a, hipStream_t stream) {
  dim3 grid(a.nq, a.seg.n_items);
  hipLaunchKernelGGL(classify_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ha
