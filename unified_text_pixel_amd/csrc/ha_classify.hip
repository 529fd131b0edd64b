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
  if (a.labels) {
    uint8_t* row = a.labels + ((int64_t)b * a.nq + qb) * a.nk;
    for (int kb = threadIdx.x; kb < a.nk; kb += kThreads)
      row[kb] = kb < kfull ? 1 : (kb < kend ? 2 : 0);
  }
}

}  // namespace

hipError_t launch_classify(const ClassifyArgs& a, hipStream_t stream) {
  dim3 grid(a.nq, a.seg.n_items);
  hipLaunchKernelGGL(classify_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ha
