// Internal interface between the host dispatch (ha_host.cpp) and the gfx950 kernels.
// Nothing here is part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

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

struct ClassifyArgs {
  int32_t S, nq, nk, bq, bk;
  uint8_t* labels;     // [B][nq][nk] or null
  int32_t* ranges;     // [B][nq][2] or null
  int32_t* row_limit;  // [B][S] or null
  SegArgs seg;
};
hipError_t launch_classify(const ClassifyArgs& a, hipStream_t stream);

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
  uint8_t axis[64];  // rotary axis of pair i
};
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream);

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
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);

}  // namespace ha
